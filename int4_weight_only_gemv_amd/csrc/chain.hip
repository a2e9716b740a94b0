// Decode of a chain of dependent W4A16 linears in one persistent launch
// (gfx950).
//
// A decoder's weight stream is a chain: each linear's input is formed from
// the previous linear's output (in a decoder layer: qkv, o, gate_up,
// down).  Launched one linear at a time, every launch pays the
// dispatch, the ramp until its first loads return and the tail of its last
// blocks, about 1.5-3 us each, and nothing streams in between ("Weight-Only
// Quantization and Mixed Precision", "7. The Marlin Kernel": round trips
// between separate kernels eat the benefit).  Here one block per CU runs the
// whole chain:
//
//   for each linear l:
//     stage X_l in LDS: formed from the previous output by the linear's glue
//       (as is, SwiGLU of [gate | up], or single-key attention: each head's
//       value vector), times the optional producer weight, rounded to BF16,
//       and stored pair-permuted with the activation sums of every 32 inputs;
//     the block's rows of W_l, four rows x 2048 inputs per wave item, with
//       the exact operands 128 + q and the per-group fold of the decode
//       kernel (s (P - (128 + z) Xsum), v_dot2_f32_bf16);
//     the K slices of a row summed in LDS in a fixed order, Y_l stored BF16;
//     all blocks meet at a grid barrier; right after arriving, each wave
//     issues the loads of its first item of W_{l+1} (they do not depend on
//     X), so the weight stream flows through the barrier and the staging of
//     X_{l+1}.
//
// The outputs pass between blocks (and the XCDs' separate L2 caches) as
// 32-bit agent-scope atomic stores and loads, which are coherent across the
// device without the L2 write-back and invalidation an agent-scope fence
// costs (measured on MI355X: 5.3 against 1.7 us per barrier).  The barrier
// is two-level: blocks arrive on 16 counters on separate cache lines, the
// last of each group on a top counter, and the last of all publishes the
// next generation into 8 copies that the blocks poll (one flat counter: 3.7
// us).  The grid is one block per CU, all resident at once (the block's
// registers fill a CU), launched normally (a cooperative launch costs ~20 us
// more).  Every barrier wait is bounded: a block that waits longer than the
// plan's spin limit records a timeout in the workspace status word and goes
// on, so every launch ends.  Results are deterministic.

#include "chain.h"
#include "common.h"

#include <atomic>

#include "w4a16.h"

namespace w4a16 {

namespace {

constexpr int kChainWaves = 16;
constexpr int kChainThreads = kChainWaves * 64;
constexpr int kChainSlice = 2048;     // inputs per wave item: 64 lanes x 32

constexpr int kGroups = kChainGroups, kGenCopies = kChainGenCopies;
constexpr int kTopWord = kChainTopWord, kStatusWord = kChainStatusWord, kGenWord0 = kChainGenWord0;

__device__ __forceinline__ unsigned ld_coherent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The 32 inputs of chunk c of activation row m, formed by the linear's glue,
// times gamma, rounded to BF16, as four natural-order dwords of pairs.  The
// previous output is read with coherent 32-bit loads (two BF16 values each;
// rows are 16-byte aligned, a chunk never straddles a head of ATTN1 when
// head_dim % 32 == 0, otherwise element by element).
__device__ __forceinline__ float lo16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void form_chunk(const ChainDesc& d, const ChainDesc* prev, const uint16_t* X0,
                                           int64_t ldx, int m, int c, u32x4 raw[4]) {
  const int k0 = 32 * c;
  float v[32];
  if (d.input == W4A16_CHAIN_X0) {
    const u32x4* p = reinterpret_cast<const u32x4*>(X0 + (int64_t)m * ldx + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = lo16(w[j]);
        v[8 * i + 2 * j + 1] = hi16(w[j]);
      }
    }
  } else {
    const unsigned* row = reinterpret_cast<const unsigned*>(prev->y + (int64_t)m * prev->ldy);
    if (d.input == W4A16_CHAIN_PREV) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const unsigned w = ld_coherent(row + k0 / 2 + t);
        v[2 * t] = lo16(w);
        v[2 * t + 1] = hi16(w);
      }
    } else if (d.input == W4A16_CHAIN_SWIGLU) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const unsigned wg = ld_coherent(row + k0 / 2 + t), wu = ld_coherent(row + (d.K + k0) / 2 + t);
        const float g0 = lo16(wg), g1 = hi16(wg);
        v[2 * t] = g0 * __builtin_amdgcn_rcpf(1.f + __expf(-g0)) * lo16(wu);
        v[2 * t + 1] = g1 * __builtin_amdgcn_rcpf(1.f + __expf(-g1)) * hi16(wu);
      }
    } else {   // W4A16_CHAIN_ATTN1
      if (d.head_dim % 32 == 0 && (d.v_offset & 1) == 0) {
        const int h = k0 / d.head_dim;
        const int src = d.v_offset + (h / d.group) * d.head_dim + (k0 - h * d.head_dim);   // even
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const unsigned w = ld_coherent(row + src / 2 + t);
          v[2 * t] = lo16(w);
          v[2 * t + 1] = hi16(w);
        }
      } else {
#pragma unroll 4
        for (int t = 0; t < 32; ++t) {
          const int k = k0 + t;
          const int h = k / d.head_dim;
          const int e = d.v_offset + (h / d.group) * d.head_dim + (k - h * d.head_dim);
          const unsigned w = ld_coherent(row + e / 2);
          v[t] = (e & 1) ? hi16(w) : lo16(w);
        }
      }
    }
  }
  if (d.gamma) {
    const u32x4* gp = reinterpret_cast<const u32x4*>(d.gamma + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = gp[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] *= lo16(w[j]);
        v[8 * i + 2 * j + 1] *= hi16(w[j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      raw[i][j] = (uint32_t)f32_to_bf16_rne(v[8 * i + 2 * j]) | ((uint32_t)f32_to_bf16_rne(v[8 * i + 2 * j + 1]) << 16);
}

// Block barrier without a wait on vector memory (the compiler may not move
// memory accesses across it; loads in flight stay in flight).
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Grid barrier, arrival half: the block's stores are complete (every wave
// waited for its stores, then the block synchronised), thread 0 arrives on its group's counter, the last
// of a group on the top counter, and the last of all resets the counters and
// publishes the next generation.  Returns true in the thread that published.
__device__ __forceinline__ bool grid_arrive(unsigned* bar, unsigned nblocks, unsigned gen) {
  if (threadIdx.x != 0) return false;
  const unsigned g = blockIdx.x % kGroups;
  const unsigned gsize = (nblocks - g + kGroups - 1) / kGroups;
  const unsigned groups = nblocks < (unsigned)kGroups ? nblocks : (unsigned)kGroups;
  const unsigned a = __hip_atomic_fetch_add(bar + 16 * g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a != gsize - 1) return false;
  st_coherent(bar + 16 * g, 0u);
  const unsigned t = __hip_atomic_fetch_add(bar + kTopWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t != groups - 1) return false;
  st_coherent(bar + kTopWord, 0u);
#pragma unroll
  for (int j = 0; j < kGenCopies; ++j) st_coherent(bar + kGenWord0 + 16 * j, gen + 1u);
  return true;
}

// Grid barrier, waiting half (thread 0; bounded), then the block follows.
__device__ __forceinline__ void grid_wait(unsigned* bar, unsigned gen, bool published, int spin_limit) {
  if (threadIdx.x == 0 && !published) {
    const unsigned* w = bar + kGenWord0 + 16 * (blockIdx.x % kGenCopies);
    int spins = 0;
    while (ld_coherent(w) == gen) {
      if (++spins > spin_limit) {
        st_coherent(bar + kStatusWord, (unsigned)W4A16_CHAIN_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  block_sync_lds();
}

template <int M>
__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainDesc* __restrict__ descs, int n_linears,
                                                              const uint16_t* __restrict__ X0, int64_t ldx,
                                                              unsigned* __restrict__ bar, int spin_limit,
                                                              int max_k, int max_rows) {
  constexpr int R = 4;                          // rows per item
  constexpr int MP = M == 1 ? 1 : 2;            // values per lane after the group step
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // X of the current linear, pair-permuted, [m][chunk c = 64 slice + lane][i]
  // stored as [m][slice][i][lane] (16 bytes per lane and i: conflict-free reads)
  const int xsl = max_k / kChainSlice + 1;                                      // slice slots per row of X
  u32x4* xs = reinterpret_cast<u32x4*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)M * xsl * 4 * 64 * 16);   // [m][chunk]
  float* red = xsum + (size_t)M * (max_k / 32);                                  // [slice][row][m]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const unsigned nblocks = gridDim.x;
  const int b = blockIdx.x;
  unsigned gen = 0;
  if (threadIdx.x == 0) gen = ld_coherent(bar + kGenWord0 + 16 * (blockIdx.x % kGenCopies));

  // double-buffered item loads: four code rows and one scale / zero point
  u32x4 cb[2][R];
  uint32_t sb[2];
  int zb[2];
  auto item_load = [&](int buf, const ChainDesc& d, int row0, int it) {
    const int batch = it / d.slices, sl = it - batch * d.slices;
    const int chunks = d.K / 32;
    const int c = min(sl * 64 + lane, chunks - 1);    // inactive lanes read valid memory
    const int64_t vrow = d.K / 32;                     // 16-byte vectors per code row
    const u32x4* cbase = reinterpret_cast<const u32x4*>(d.codes) + c;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int row = min(row0 + batch * R + j, d.N - 1);
      cb[buf][j] = __builtin_nontemporal_load(cbase + (int64_t)row * vrow);
    }
    const int G = d.K / kGroup;
    const int mrow = min(row0 + batch * R + (lane & 3), d.N - 1);
    sb[buf] = d.scales[(int64_t)mrow * G + c / 4];
    zb[buf] = d.zeros[(int64_t)mrow * G + c / 4];
  };
  auto block_rows = [&](const ChainDesc& d, int& row0, int& nb) {
    nb = d.batches_per_block + (b < d.batches_rem ? 1 : 0);
    row0 = R * (b * d.batches_per_block + min(b, d.batches_rem));
  };

  // the first linear's first item
  {
    const ChainDesc d = descs[0];
    int row0, nb;
    block_rows(d, row0, nb);
    if (wave < nb * d.slices) item_load(0, d, row0, wave);
  }

  for (int l = 0; l < n_linears; ++l) {
    const ChainDesc d = descs[l];
    const ChainDesc* prev = l > 0 ? descs + (l - 1) : nullptr;
    int row0, nb;
    block_rows(d, row0, nb);
    const int chunks = d.K / 32;
    const int items = nb * d.slices;

    // ---- stage X_l: one 32-input chunk per thread and step (the loads of
    // the previous output wait behind the prefetched weights, which were
    // issued first and land during the barrier)
    for (int e = threadIdx.x; e < M * chunks; e += kChainThreads) {
      const int m = e / chunks, c = e - m * chunks;
      u32x4 raw[4];
      form_chunk(d, prev, X0, ldx, m, c, raw);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sum = dot2(raw[i][j], kOnePair, sum);
      const int sl = c >> 6, ln = c & 63;
#pragma unroll
      for (int i = 0; i < 4; ++i) xs[((size_t)(m * xsl + sl) * 4 + i) * 64 + ln] = x_pairs_from_natural(raw[i]);
      xsum[m * (max_k / 32) + c] = sum;
    }
    block_sync_lds();

    // ---- the block's rows: items (4-row batch, 2048-input slice)
    auto compute = [&](int buf, int it) {
      const int batch = it / d.slices, sl = it - batch * d.slices;
      const int c = sl * 64 + lane;
      const bool active = c < chunks;
      u32x4 xp[M][4];
      float xsg[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 v = xs[((size_t)(m * xsl + sl) * 4 + i) * 64 + lane];
          if (!active) v = u32x4{0u, 0u, 0u, 0u};
          xp[m][i] = v;
        }
        if (active) s = xsum[m * (max_k / 32) + c];
        s += dpp<kDppXor1>(s);
        xsg[m] = s + dpp<kDppXor2>(s);
      }
      float P[R][M];
#pragma unroll
      for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int m = 0; m < M; ++m) P[j][m] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 q = codes_to_bias128_pairs(cb[buf][j][i]);
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) P[j][m] = dot2(q[jj], xp[m][i][jj], P[j][m]);
        }
      }
      // sum over the four lanes of a group, lane l keeping row l % 4 ...
      float h[2][M];
      {
        const uint32_t up = (lane & 2) ? ~0u : 0u;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int m = 0; m < M; ++m)
            h[r][m] = pick(up, P[r + 2][m] + dpp<kDppXor2>(P[r + 2][m]), P[r][m] + dpp<kDppXor2>(P[r][m]));
      }
      float part[MP];
      {
        const uint32_t up = (lane & 1) ? ~0u : 0u;
        const float s = bf16_to_f32(sb[buf]);
        const float zb128 = (float)zb[buf] + 128.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float q = pick(up, h[1][m] + dpp<kDppXor1>(h[1][m]), h[0][m] + dpp<kDppXor1>(h[0][m]));
          // ... and removes the bias and zero point of that (row, group)
          part[m] = s * fmaf(-zb128, xsg[m], q);
        }
#pragma unroll
        for (int m = M; m < MP; ++m) part[m] = 0.f;
      }
      // then over the 16 groups of the slice (lane bits 2..5)
      lane_tree_sum<MP, MP == 1 ? 0 : 1>(part, lane);
      int m;
      if (tree_result<MP, MP == 1 ? 0 : 1>(lane, m) && m < M)
        red[((size_t)sl * max_rows + batch * R + (lane & 3)) * M + m] = part[0];
    };
    int it = wave;
    while (true) {
      if (it >= items) break;
      if (it + kChainWaves < items) item_load(1, d, row0, it + kChainWaves);
      compute(0, it);
      it += kChainWaves;
      if (it >= items) break;
      if (it + kChainWaves < items) item_load(0, d, row0, it + kChainWaves);
      compute(1, it);
      it += kChainWaves;
    }
    block_sync_lds();

    // ---- the K slices of each row in a fixed order, BF16 store of row pairs
    // as coherent 32-bit stores (rows start at a multiple of 4; an odd last
    // row of the linear updates its half of the word atomically)
    const int rows = min(R * nb, d.N - row0);
    auto row_value = [&](int r, int m) {
      float v = red[(size_t)r * M + m];
      for (int sl = 1; sl < d.slices; ++sl) v += red[((size_t)sl * max_rows + r) * M + m];
      return (uint32_t)f32_to_bf16_rne(v);
    };
    for (int e = threadIdx.x; e < ((rows + 1) / 2) * M; e += kChainThreads) {
      const int r = 2 * (e / M), m = e - (e / M) * M;
      unsigned* yw = reinterpret_cast<unsigned*>(d.y + (int64_t)m * d.ldy + row0 + r);
      if (r + 1 < rows) {
        st_coherent(yw, row_value(r, m) | (row_value(r + 1, m) << 16));
      } else {
        __hip_atomic_fetch_and(yw, 0xFFFF0000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(yw, row_value(r, m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    if (l + 1 < n_linears) {
      // the block's stores are complete before it arrives (a block barrier
      // alone does not wait for global stores)
      wait_vmcnt<0>();
      __syncthreads();
      const bool published = grid_arrive(bar, nblocks, gen);
      // the next linear's first item streams through the barrier
      const ChainDesc dn = descs[l + 1];
      int r0n, nbn;
      block_rows(dn, r0n, nbn);
      if (wave < nbn * dn.slices) item_load(0, dn, r0n, wave);
      grid_wait(bar, gen, published, spin_limit);
      gen += 1u;
    }
  }
}

}  // namespace

// Launch one chain (the caller has validated the plan): M = 1 or 2, one
// block per CU.
int launch_chain(const void* descs, int n_linears, int M, const uint16_t* X0, int64_t ldx, unsigned* bar,
                 int spin_limit, int max_k, int max_rows, int grid, size_t lds_bytes, hipStream_t stream) {
  const ChainDesc* dd = reinterpret_cast<const ChainDesc*>(descs);
  if (M == 1) {
    static bool attr1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<1>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    if (!attr1) return 4;
    hipLaunchKernelGGL(chain_kernel<1>, dim3(grid), dim3(kChainThreads), lds_bytes, stream, dd, n_linears, X0, ldx,
                       bar, spin_limit, max_k, max_rows);
  } else {
    static bool attr2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<2>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    if (!attr2) return 4;
    hipLaunchKernelGGL(chain_kernel<2>, dim3(grid), dim3(kChainThreads), lds_bytes, stream, dd, n_linears, X0, ldx,
                       bar, spin_limit, max_k, max_rows);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// ---------------------------------------------------------------------------
// The same launch for callers that cannot allocate: barrier state and
// descriptors in a file-scope device array of fixed size (one copy per GPU,
// kept until the process ends; calls that overlap on one GPU race).
// ---------------------------------------------------------------------------

namespace {

constexpr int64_t kScratchBytes = kChainHeaderBytes + (int64_t)W4A16_CHAIN_NOALLOC_MAX_LINEARS * sizeof(ChainDesc);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current (the array's name is a host-side stand-in).
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// the barrier state must start at zero: a fill kernel (no memset node)
__global__ void clear_words_kernel(unsigned* p, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0u;
}

}  // namespace

int launch_chain_noalloc(const ChainDesc* d, int n_linears, int M, const uint16_t* X0, int64_t ldx, int max_k,
                         int max_rows, int grid, size_t lds_bytes, int* status, hipStream_t stream) {
  char* ws = static_cast<char*>(scratch_address());
  if (!ws) return 4;
  // descriptors: the host copy (the caller's stack) must be consumed before
  // this call returns, so the copy is waited for
  if (hipMemcpyAsync(ws + kChainHeaderBytes, d, (size_t)n_linears * sizeof(ChainDesc), hipMemcpyHostToDevice,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return 4;
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, reinterpret_cast<unsigned*>(ws),
                     (int)(kChainHeaderBytes / 4));
  if (hipGetLastError() != hipSuccess) return 4;
  if (int st = launch_chain(ws + kChainHeaderBytes, n_linears, M, X0, ldx, reinterpret_cast<unsigned*>(ws),
                            W4A16_CHAIN_SPIN_LIMIT, max_k, max_rows, grid, lds_bytes, stream))
    return st;
  if (status) {
    unsigned v = 0;
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpy(&v, ws + kChainStatusWord * 4, 4, hipMemcpyDeviceToHost) != hipSuccess)
      return 4;
    *status = (int)v;
  }
  return 0;
}

}  // namespace w4a16
