// Layout shared by the chain kernel and its launcher: the per-linear
// descriptor the kernel reads from the workspace, and the workspace header
// (barrier state and status word).
#pragma once

#include <stdint.h>

namespace w4a16 {

// Per-linear descriptor in the workspace (device memory).
struct ChainDesc {
  const uint32_t* codes;
  const uint16_t* scales;
  const int32_t* zeros;
  const uint16_t* gamma;
  uint16_t* y;
  int64_t ldy;
  int32_t N, K, input, v_offset, head_dim, group;
  int32_t batches_per_block, batches_rem;   // 4-row batches of a block: base + (b < rem)
  int32_t slices;                           // 2048-input slices: ceil(K / 2048)
  // pair > 0: the next linear takes SwiGLU of this output and N = 2 pair;
  // each block then owns the same gate rows k and up rows pair + k
  // (batches_* count the gate half) and writes the glued next input
  int32_t pair;
  int32_t glued;                            // input read as formed from the glue region
  int32_t pad;
};
static_assert(sizeof(ChainDesc) % 8 == 0, "descriptor alignment");

// Workspace header, in 32-bit words, each on its own 64-byte line: arrival
// counters of 16 block groups, the top counter, the status word, and 8
// copies of the barrier generation; then the glue region (a SwiGLU input
// formed once by its producer, BF16 [M][K], at most 2 x 32768), then the
// descriptors.
constexpr int kChainGroups = 16, kChainGenCopies = 8;
constexpr int kChainTopWord = 16 * kChainGroups;
constexpr int kChainStatusWord = kChainTopWord + 16;
constexpr int kChainGenWord0 = kChainStatusWord + 16;
constexpr int64_t kChainHeaderBytes = 2048;
static_assert((kChainGenWord0 + 16 * kChainGenCopies) * 4 <= kChainHeaderBytes, "header size");
constexpr int64_t kChainGlueBytes = (int64_t)2 * 32768 * 2;
constexpr int64_t kChainDescOffset = kChainHeaderBytes + kChainGlueBytes;

}  // namespace w4a16
