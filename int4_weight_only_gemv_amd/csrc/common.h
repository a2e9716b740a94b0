// Device helpers shared by the HIP kernels of the W4A16 library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;
constexpr int kWave = 64;

// BF16 0x4300 is 128.0 and its 7 mantissa bits count in units of 1, so a
// 4-bit code placed in the low mantissa bits gives 128 + code exactly.
constexpr uint32_t kOnePair = 0x3F803F80u;  // BF16 (1.0, 1.0)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> BF16 bits, round to nearest even; NaN becomes the quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Eight 4-bit codes of one word -> eight BF16 operands 128 + q, ordered so
// that dword j holds (code j, code j+4).  The matching activation operand
// must use the same pairing (see x_pairs_from_natural).
//
// Seven ops per word: one mask for the even codes (one per byte), a shift and
// a mask for the odd codes, then one byte permute per dword that places two
// code bytes under the exponent byte 0x43 of BF16 128.0.
constexpr uint32_t kExpBytes = 0x43434343u;
constexpr uint32_t kSelLoHalf = 0x04020400u;  // (S1.b0, 0x43, S1.b2, 0x43)
constexpr uint32_t kSelHiHalf = 0x04030401u;  // (S1.b1, 0x43, S1.b3, 0x43)

__device__ __forceinline__ u32x4 codes_to_bias128_pairs(uint32_t w) {
  const uint32_t even = w & 0x0F0F0F0Fu;          // bytes: q0 q2 q4 q6
  const uint32_t odd = (w >> 4) & 0x0F0F0F0Fu;    // bytes: q1 q3 q5 q7
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(kExpBytes, even, kSelLoHalf);  // (q0, q4)
  r[1] = __builtin_amdgcn_perm(kExpBytes, odd, kSelLoHalf);   // (q1, q5)
  r[2] = __builtin_amdgcn_perm(kExpBytes, even, kSelHiHalf);  // (q2, q6)
  r[3] = __builtin_amdgcn_perm(kExpBytes, odd, kSelHiHalf);   // (q3, q7)
  return r;
}

// Eight consecutive BF16 activations x0..x7 loaded as dwords
// (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> the pairing (x0,x4) (x1,x5) (x2,x6)
// (x3,x7) used by codes_to_bias128_pairs.
__device__ __forceinline__ u32x4 x_pairs_from_natural(u32x4 d) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
  return r;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi on two BF16 pairs, float32 result.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// up ? a : b as one bit-select on a lane mask (all ones or zero).  Written
// as bit operations so that the compiler keeps the two values in registers
// instead of turning a select between array elements into an indexed
// access (which it lowers to a chain of compares and selects).
__device__ __forceinline__ float pick(uint32_t up_mask, float a, float b) {
  return __uint_as_float((__float_as_uint(a) & up_mask) | (__float_as_uint(b) & ~up_mask));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// D = A * B + C on a 16x16 output tile with K = 32 (BF16 in, FP32 out).
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Compute units of the current device (queried once per device; host code).
inline int device_cu_count() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

}  // namespace w4a16
