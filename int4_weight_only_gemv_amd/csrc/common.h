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

// Eight codes of one word -> BF16 operands 4^E (128 + q) in natural k
// order: dword j holds (code 2j, code 2j+1).  eb holds the exponent byte
// 0x43 + E in every byte (0x43: BF16 128.0, whose low mantissa bits count
// in units of one).
__device__ __forceinline__ u32x4 codes_to_bias128_natural(uint32_t w, uint32_t eb) {
  const uint32_t even = w & 0x0F0F0F0Fu;          // bytes q0 q2 q4 q6
  const uint32_t odd = (w >> 4) & 0x0F0F0F0Fu;    // bytes q1 q3 q5 q7
  const uint32_t lo = __builtin_amdgcn_perm(odd, even, 0x05010400u);  // q0 q1 q2 q3
  const uint32_t hi = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // q4 q5 q6 q7
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(eb, lo, 0x04010400u);  // (q0, q1)
  r[1] = __builtin_amdgcn_perm(eb, lo, 0x04030402u);  // (q2, q3)
  r[2] = __builtin_amdgcn_perm(eb, hi, 0x04010400u);  // (q4, q5)
  r[3] = __builtin_amdgcn_perm(eb, hi, 0x04030402u);  // (q6, q7)
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

typedef __attribute__((address_space(3))) void lds_void;

// One direct-to-LDS copy (global_load_lds_dwordx4): lane l's 16 bytes at src
// land at lds_dst + 16 l.  lds_dst must be the same for the whole wave.
// (Kept in a device function: inside a kernel body the target builtin stops
// the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}

// Block barrier that the compiler may not move memory accesses across
// (the bare builtin does not order them at the IR level).
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Block barrier after this wave's LDS writes are done, leaving its global
// and direct-to-LDS loads in flight (a __syncthreads() also waits for every
// direct-to-LDS copy, since those count as LDS writes, which would drain a
// prefetch ring at every barrier).  For LDS data written with ordinary
// stores only.
__device__ __forceinline__ void block_barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int V>
struct Ic {
  static constexpr int value = V;
};

// f(Ic<I>{}) for I = B .. E-1, in order (a loop whose index is a constant)
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(Ic<B>{});
    static_for<B + 1, E>(f);
  }
}

// Wait until at most n vector-memory operations of this wave are in flight
// and all of its LDS operations are done (so LDS writes made before the
// following barrier are visible to the whole block after it).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }
constexpr int log2_exact(int v) { return v <= 1 ? 0 : 1 + log2_exact(v / 2); }

// Cross-lane sums without LDS: DPP for lanes within a 16-lane row, the
// permlane swaps across rows.  DPP quad_perm [1,0,3,2] / [2,3,0,1] reads lane
// l ^ 1 / l ^ 2; row_ror:n gives lane l the value of lane l - n (mod 16) of
// its row; v_permlane32_swap exchanges the upper 32 lanes of its first operand
// with the lower 32 of its second, v_permlane16_swap the odd 16-lane rows of
// its first operand with the even rows of its second.
constexpr int kDppXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRor8 = 0x128;    // row_ror:8: lane l ^ 8
constexpr int kDppRor12 = 0x12C;   // row_ror:12: lane l + 4 (mod 16)

template <int C>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), C, 0xF, 0xF, false));
}

// x(l) + x(l ^ 2^bit) for lane bit 5, 4 or 3, in every lane; for bit 2
// exact only in lanes whose bit 2 is clear.
template <int BIT>
__device__ __forceinline__ float pair_sum(float x) {
  if constexpr (BIT >= 4) {
    const auto r = BIT == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (BIT == 3) {
    return x + dpp<kDppRor8>(x);
  } else {
    static_assert(BIT == 2, "lane bits 2..5");
    return x + dpp<kDppRor12>(x);
  }
}

// One halving step on lane bit 5, 4 or 3: lanes whose bit is clear end with
// a(l) + a(l ^ 2^bit), lanes whose bit is set with b(l) + b(l ^ 2^bit).
template <int BIT>
__device__ __forceinline__ float halve(float a, float b, int lane) {
  if constexpr (BIT >= 4) {
    const auto r = BIT == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                            : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    static_assert(BIT == 3, "halving on lane bits 3..5");
    return pick((lane & 8) ? ~0u : 0u, pair_sum<3>(b), pair_sum<3>(a));
  }
}

// Sum of MP = 2^LM values per lane over lane bits 2..5 (the 16 lane groups of
// four): halving on bits 5, 4, .. (value i + MP/2 moves to the lanes whose
// bit 5 is set, and so on), then plain sums on the remaining bits.  After it,
// a lane whose bits 2 .. 5-LM are clear holds in part[0] the sum of value m
// over its four-lane position, m read from its bits 5 .. 6-LM (bit 5 the
// highest).
template <int MP, int LM>
__device__ __forceinline__ void lane_tree_sum(float* part, int lane) {
  static_assert(MP == (1 << LM) && LM <= 3, "at most 8 values per lane");
  static_for<0, LM>([&](auto bi) {
    constexpr int b = decltype(bi)::value, n = MP >> b;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) part[i] = halve<5 - b>(part[i], part[i + n / 2], lane);
  });
  static_for<LM, 4>([&](auto bi) {
    constexpr int b = decltype(bi)::value;
    part[0] = pair_sum<5 - b>(part[0]);
  });
}

// The value index a lane holds after lane_tree_sum<MP, LM>, and whether it
// holds a finished sum.
template <int MP, int LM>
__device__ __forceinline__ bool tree_result(int lane, int& m) {
  m = 0;
  int half = MP / 2;
#pragma unroll
  for (int b = 0; b < LM; ++b, half >>= 1)
    if (lane & (32 >> b)) m += half;
  return ((lane >> 2) & ((16 >> LM) - 1)) == 0;
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
