// Group-wise asymmetric (and, as a variant, symmetric) INT4 quantise + pack
// (offline step of the W4A16 path).
//
// Scheme: Axe Corsa model card, "The Two-Stage Pipeline" (asymmetric, one
// BF16 scale and one INT32 zero point per group of 128 consecutive weights)
// and "What the Tensor Types Tell You" (packed codes); the min/max affine
// rule with rounding and clipping follows "Quantization I: int8, int4, the
// basics", "Concept".  The exact float32 steps are documented on w4a16_pack
// in w4a16.h; this file must be compiled without FMA contraction and with
// correctly rounded division so that every step is a single IEEE operation.
//
// Mapping: one lane per output word (8 consecutive k of one row); the 16
// lanes of an aligned 16-lane segment cover one group of 128 (8 or 4 lanes a
// group of 64 or 32), so the group min/max is a butterfly inside the
// segment.

#include "common.h"

namespace w4a16 {
namespace {

constexpr float kFltMin = 1.17549435e-38f;  // 2^-126

// min / max over an aligned segment of `seg` lanes (4, 8 or 16)
__device__ __forceinline__ float seg_min(float v, int seg) {
  for (int off = seg >> 1; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off, 16));
  return v;
}
__device__ __forceinline__ float seg_max(float v, int seg) {
  for (int off = seg >> 1; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 16));
  return v;
}

__device__ __forceinline__ float bf16_rtz(float f) {
  return __uint_as_float(__float_as_uint(f) & 0xFFFF0000u);
}

// kW8: the W8A16 variant, 8-bit codes 0..255 (step D / 255), two code words
// per lane (byte j of word i holds k = 4i + j)
template <bool kVecLoad, bool kAwq, bool kSym, bool kW8>
__global__ __launch_bounds__(256) void pack_kernel(
    const uint16_t* __restrict__ W, int64_t ldw, const float* __restrict__ awq_s,
    int64_t words_per_row, int64_t total_words, int seg, uint32_t* __restrict__ codes,
    uint16_t* __restrict__ scales, int32_t* __restrict__ zeros) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // Every lane of a live segment takes part in the shuffles; segments are
  // whole because words_per_row is a multiple of 16.
  const bool live = t < total_words;
  const int64_t tw = live ? t : total_words - 1;
  const int64_t n = tw / words_per_row;
  const int64_t wi = tw - n * words_per_row;
  const uint16_t* src = W + n * ldw + wi * 8;

  uint32_t raw[4];
  if (kVecLoad) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    raw[0] = v.x; raw[1] = v.y; raw[2] = v.z; raw[3] = v.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = (uint32_t)src[2 * i] | ((uint32_t)src[2 * i + 1] << 16);
  }
  float w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = bf16_to_f32(raw[i] & 0xFFFFu);
    w[2 * i + 1] = bf16_to_f32(raw[i] >> 16);
  }
  if (kAwq) {
    const float* sp = awq_s + wi * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = __fmul_rn(w[j], sp[j]);
  }

  float mn = w[0], mx = w[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) { mn = fminf(mn, w[j]); mx = fmaxf(mx, w[j]); }
  mn = seg_min(mn, seg);
  mx = seg_max(mx, seg);

  float s;
  int z;
  if (kSym) {
    // symmetric: the grid centred on zero reaches the largest magnitude,
    // codes -7..7 stored with zero point 8
    const float a = fmaxf(fabsf(mn), fabsf(mx));
    s = bf16_rtz(__fdiv_rn(a, 7.0f));
    if (!(s >= kFltMin)) {
      s = bf16_rtz(a);
      if (!(s >= kFltMin)) s = 1.0f;
    }
    z = 8;
  } else {
    const float d = __fsub_rn(mx, mn);
    s = bf16_rtz(__fdiv_rn(d, kW8 ? 255.0f : 15.0f));
    if (!(s >= kFltMin)) {  // degenerate group: zero or subnormal step
      s = bf16_rtz(fmaxf(fabsf(mn), fabsf(mx)));
      if (!(s >= kFltMin)) s = 1.0f;
    }
    z = (int)roundf(__fdiv_rn(-mn, s));
  }

  constexpr int kQmax = kW8 ? 255 : 15;
  uint32_t word = 0, word2 = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int q = (int)roundf(__fdiv_rn(w[j], s)) + z;
    q = q < 0 ? 0 : (q > kQmax ? kQmax : q);
    if (kW8) {
      if (j < 4) word |= (uint32_t)q << (8 * j);
      else word2 |= (uint32_t)q << (8 * (j - 4));
    } else {
      word |= (uint32_t)q << (4 * j);
    }
  }
  if (live) {
    if (kW8) {
      codes[2 * t] = word;
      codes[2 * t + 1] = word2;
    } else {
      codes[t] = word;
    }
    if ((wi & (seg - 1)) == 0) {
      const int64_t gi = n * (words_per_row / seg) + wi / seg;
      scales[gi] = (uint16_t)(__float_as_uint(s) >> 16);
      zeros[gi] = z;
    }
  }
}

}  // namespace

namespace {
template <bool kSym, bool kW8>
void launch_pack_t(const uint16_t* W, int64_t ldw, const float* awq_s, int64_t words_per_row,
                   int64_t total, int seg, uint32_t* codes, uint16_t* scales, int32_t* zeros,
                   bool vec, hipStream_t stream) {
  const int threads = 256;
  const dim3 grid((unsigned)((total + threads - 1) / threads));
  if (vec) {
    if (awq_s)
      hipLaunchKernelGGL((pack_kernel<true, true, kSym, kW8>), grid, dim3(threads), 0, stream, W, ldw,
                         awq_s, words_per_row, total, seg, codes, scales, zeros);
    else
      hipLaunchKernelGGL((pack_kernel<true, false, kSym, kW8>), grid, dim3(threads), 0, stream, W, ldw,
                         awq_s, words_per_row, total, seg, codes, scales, zeros);
  } else {
    if (awq_s)
      hipLaunchKernelGGL((pack_kernel<false, true, kSym, kW8>), grid, dim3(threads), 0, stream, W, ldw,
                         awq_s, words_per_row, total, seg, codes, scales, zeros);
    else
      hipLaunchKernelGGL((pack_kernel<false, false, kSym, kW8>), grid, dim3(threads), 0, stream, W, ldw,
                         awq_s, words_per_row, total, seg, codes, scales, zeros);
  }
}
}  // namespace

// group: 32, 64 or 128 inputs per quantisation group (checked by the caller)
int launch_pack(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, const float* awq_s,
                int group, uint32_t* codes, uint16_t* scales, int32_t* zeros, bool symmetric,
                bool int8, hipStream_t stream) {
  const int64_t words_per_row = K / 8;
  const int64_t total = N * words_per_row;
  const int seg = group / 8;
  const bool vec = ((reinterpret_cast<uintptr_t>(W) & 15u) == 0) && (ldw % 8 == 0);
  if (int8)
    launch_pack_t<false, true>(W, ldw, awq_s, words_per_row, total, seg, codes, scales, zeros, vec, stream);
  else if (symmetric)
    launch_pack_t<true, false>(W, ldw, awq_s, words_per_row, total, seg, codes, scales, zeros, vec, stream);
  else
    launch_pack_t<false, false>(W, ldw, awq_s, words_per_row, total, seg, codes, scales, zeros, vec, stream);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
