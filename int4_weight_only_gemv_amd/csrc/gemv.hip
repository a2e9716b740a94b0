// Decode-shaped fused W4A16 matmul, 1 <= M <= 32 (gfx950).
//
// Y[m, n] = sum_g s[n,g] * sum_{k in g} X[m,k] * (q[n,k] - z[n,g])
// (Axe Corsa model card, "The Two-Stage Pipeline": dequantisation fused
// into the multiply, weights rebuilt in registers; "Quantization I",
// "Concept": only the packed form crosses the memory bus).
//
// All kernels turn a code word into exact BF16 operands 128 + q by OR-ing
// each nibble into the mantissa of BF16 128.0 (two ops per pair of codes, no
// conversions) and remove the bias and the zero point once per group in
// float32 with one fused multiply-add whose product is exact:
//     acc += s * (P - (128 + z) * Xsum),   P = sum_k x (128 + q).
// No weight is ever rounded.
//
// gemv_dot (M <= 2, and M <= 4 for K > 16384): a wave owns a 2048-input
// slice of K for a run of rows; its 64 lanes read 16 contiguous bytes each,
// so every load instruction moves 1 KiB of one row -- the fully coalesced
// pattern that streams HBM fastest.  The lane's 32 activations per batch row
// stay in registers for all rows, the products run on v_dot2_f32_bf16, and
// per-row partial sums are folded across lanes with a halving butterfly
// (ds_bpermute), then across the K slices of the block through LDS in a
// fixed order.
//
// gemv_quad (3 <= M <= 8, K <= 16384): the same streaming pattern (four rows
// x 256 contiguous bytes per load instruction), but the products run on the
// matrix cores as sixteen 4x4 blocks per instruction, so more activation
// rows cost almost no vector ALU time.
//
// gemv_tile (the rest, up to M = 32): 16-row tiles of W meet X (M padded to
// 16 or 32) on v_mfma_f32_16x16x32_bf16, one group of a tile per 16-byte
// load per lane; the same A operand against a B of ones gives the per-group
// activation sums.  The waves of a block split K and add their partial tiles
// through LDS in a fixed order.
//
// No kernel uses atomics or workspace: results are deterministic.

#include "common.h"

#include <cmath>

namespace w4a16 {
namespace {

// ---------------------------------------------------------------------------
// gemv_dot
// ---------------------------------------------------------------------------

constexpr int kSlice = 2048;      // inputs per wave: 64 lanes x 32
constexpr int kMaxSlices = 16;    // K <= 32768 on this kernel

constexpr int pow2_at_least(int v) { return v <= 1 ? 1 : 2 * pow2_at_least((v + 1) / 2); }
constexpr int log2_exact(int v) { return v <= 1 ? 0 : 1 + log2_exact(v / 2); }

// PL: groups smaller than 128 inputs (lg = log2 of the group size, 5 or 6):
// each lane folds scale and zero point into its own 32 products for all R
// rows (the fold is linear, so a group split over lanes sums correctly)
// before the cross-lane sums.  Otherwise lg = 7 and the four lanes of a
// group are summed first and fold once.
// W8: the W8A16 variant, 8-bit codes (byte j of word i is k = 4i + j); each
// byte's nibbles l, h become exact BF16 operands 128 + l (like INT4 codes)
// and 256 + 16 h (8 h in mantissa bits 3..6 with the exponent's low bit
// set), so P = P_l + P_h = sum x q + 384 Xsum.
template <int M, int R, int NB, bool PL, bool W8>
__global__ __launch_bounds__(1024) void gemv_dot_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K, int lg,
    uint16_t* __restrict__ Y, int64_t ldy) {
  static_assert(R == 4, "a group spans 4 lanes; lane l corrects row l % 4 of its group");
  constexpr int RB = R * NB;                  // rows per block
  constexpr int MP = pow2_at_least(M);        // values per lane after the group step
  constexpr int LM = log2_exact(MP);
  __shared__ float red[kMaxSlices][RB * M];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int k0 = wave * kSlice + lane * 32;
  const bool active = k0 < K;
  const int kc = active ? k0 : K - 32;        // inactive lanes read valid memory, weigh zero
  const int G = K >> lg;
  const int g = kc >> lg;                     // this lane's group (lanes 4i .. 4i+3 share one at 128)
  const int64_t wpr = K / 8;

  const int row0 = blockIdx.x * RB;
  constexpr int CW = W8 ? 2 : 1;              // 16-byte code vectors per lane and row
  const int64_t vrow = W8 ? K / 16 : wpr / 4; // 16-byte vectors per code row
  const u32x4* cbase = reinterpret_cast<const u32x4*>(codes) + kc / (32 / CW);
  u32x4 cb[2][R][CW];
  // scale and zero point of row (lane % 4), group g; with PL those of all
  // R rows
  uint32_t sb[2][PL ? R : 1];
  int zb[2][PL ? R : 1];
  auto load = [&](int buf, int batch) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int row = min(row0 + batch * R + j, N - 1);
#pragma unroll
      for (int v = 0; v < CW; ++v) cb[buf][j][v] = __builtin_nontemporal_load(cbase + (int64_t)row * vrow + v);
    }
    if constexpr (PL) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int row = min(row0 + batch * R + j, N - 1);
        sb[buf][j] = scales[(int64_t)row * G + g];
        zb[buf][j] = zeros[(int64_t)row * G + g];
      }
    } else {
      const int mrow = min(row0 + batch * R + (lane & 3), N - 1);
      sb[buf][0] = scales[(int64_t)mrow * G + g];
      zb[buf][0] = zeros[(int64_t)mrow * G + g];
    }
  };

  load(0, 0);  // the weight stream first: it is the long-latency path

  // this lane's 32 activations of every batch row, paired like the codes,
  // and the activation sums of its group
  u32x4 xp[M][4];
  float xsg[M];   // activation sums of the lane's group (with PL: of its own 32 inputs)
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(X + m * ldx + kc);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 raw = xr[i];
      if (!active) raw = u32x4{0u, 0u, 0u, 0u};
      xp[m][i] = W8 ? raw : x_pairs_from_natural(raw);
#pragma unroll
      for (int j = 0; j < 4; ++j) sum = dot2(raw[j], kOnePair, sum);
    }
    if constexpr (PL) {
      xsg[m] = sum;
    } else {
      sum += __shfl_xor(sum, 1);
      xsg[m] = sum + __shfl_xor(sum, 2);
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int cur = nb & 1;
    if (nb + 1 < NB) load(cur ^ 1, nb + 1);
    // P[j][m]: this lane's 32 products of row j with activation row m
    float P[R][M];
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
      for (int m = 0; m < M; ++m) P[j][m] = 0.f;
      if constexpr (W8) {
        float Ph[M];
#pragma unroll
        for (int m = 0; m < M; ++m) Ph[m] = 0.f;
#pragma unroll
        for (int v = 0; v < CW; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // word i of vector v: inputs 16 v + 4 i .. +3, activation dwords d, d + 1
            const uint32_t w = cb[cur][j][v][i];
            const uint32_t lb = w & 0x0F0F0F0Fu, hb = ((w >> 1) & 0x78787878u) | 0x80808080u;
            const uint32_t l01 = __builtin_amdgcn_perm(kExpBytes, lb, 0x04010400u);
            const uint32_t l23 = __builtin_amdgcn_perm(kExpBytes, lb, 0x04030402u);
            const uint32_t h01 = __builtin_amdgcn_perm(kExpBytes, hb, 0x04010400u);
            const uint32_t h23 = __builtin_amdgcn_perm(kExpBytes, hb, 0x04030402u);
            const int d = 8 * v + 2 * i;
#pragma unroll
            for (int m = 0; m < M; ++m) {
              P[j][m] = dot2(l01, xp[m][d >> 2][d & 3], P[j][m]);
              P[j][m] = dot2(l23, xp[m][d >> 2][(d & 3) + 1], P[j][m]);
              Ph[m] = dot2(h01, xp[m][d >> 2][d & 3], Ph[m]);
              Ph[m] = dot2(h23, xp[m][d >> 2][(d & 3) + 1], Ph[m]);
            }
          }
#pragma unroll
        for (int m = 0; m < M; ++m) P[j][m] += Ph[m];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 b = codes_to_bias128_pairs(cb[cur][j][0][i]);
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) P[j][m] = dot2(b[jj], xp[m][i][jj], P[j][m]);
        }
      }
      if constexpr (PL) {
        const float s = bf16_to_f32(sb[cur][j]);
        const float zb128 = (float)zb[cur][j] + 128.f;
#pragma unroll
        for (int m = 0; m < M; ++m) P[j][m] = s * fmaf(-zb128, xsg[m], P[j][m]);
      }
    }
    // Sum over the 4 lanes of the group with a halving butterfly (lane bit 1
    // picks rows {0,1} or {2,3}, bit 0 one of those), so that lane l ends
    // with the group sums of row l % 4 ...
    float h[2][M];
    {
      const uint32_t up = (lane & 2) ? ~0u : 0u;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float send = pick(up, P[r][m], P[r + 2][m]);
          const float keep = pick(up, P[r + 2][m], P[r][m]);
          h[r][m] = keep + __shfl_xor(send, 2);
        }
    }
    float part[MP];
    {
      const uint32_t up = (lane & 1) ? ~0u : 0u;
      const float s = bf16_to_f32(sb[cur][0]);
      const float zb128 = (float)zb[cur][0] + (W8 ? 384.f : 128.f);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float send = pick(up, h[0][m], h[1][m]);
        const float keep = pick(up, h[1][m], h[0][m]);
        const float q = keep + __shfl_xor(send, 1);
        // ... and removes the bias and zero point of that (row, group) once
        // (already done per lane with PL)
        part[m] = PL ? q : s * fmaf(-zb128, xsg[m], q);
      }
#pragma unroll
      for (int m = M; m < MP; ++m) part[m] = 0.f;
    }
    // then over the 16 groups of the slice (lane bits 2..5): halving on the
    // activation rows first, plain sums after
    int mask = 4;
#pragma unroll
    for (int cur_n = MP; cur_n > 1; cur_n >>= 1) {
      const uint32_t up = (lane & mask) ? ~0u : 0u;
#pragma unroll
      for (int i = 0; i < cur_n / 2; ++i) {
        const float send = pick(up, part[i], part[i + cur_n / 2]);
        const float keep = pick(up, part[i + cur_n / 2], part[i]);
        part[i] = keep + __shfl_xor(send, mask);
      }
      mask <<= 1;
    }
#pragma unroll
    for (; mask <= 32; mask <<= 1) part[0] += __shfl_xor(part[0], mask);
    // lane l < 4 MP holds row l % 4 and activation row m from its bits 2..
    if (lane < 4 * MP) {
      int m = 0, half = MP / 2;
#pragma unroll
      for (int b = 0; b < LM; ++b, half >>= 1)
        if (lane & (4 << b)) m += half;
      if (m < M) red[wave][nb * R * M + (lane & 3) * M + m] = part[0];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < RB * M; idx += blockDim.x) {
    const int j = idx / M, m = idx - j * M;
    const int row = row0 + j;
    if (row >= N) continue;
    float v = red[0][idx];
    for (int w = 1; w < S; ++w) v += red[w][idx];
    Y[m * ldy + row] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------------------------------
// gemv_quad (M <= 8): sixteen 4x4 products per matrix instruction
// ---------------------------------------------------------------------------
//
// v_mfma_f32_4x4x4_16b_bf16 runs 16 independent products of a 4x4 A block
// and a 4x4 B block (K = 4): lane 4b + i supplies row i of block b's A, lane
// 4b + j column j of block b's B, and lane 4b + j receives column j of block
// b's result with row r in register r.  Here the four B columns are four
// weight rows and the A rows up to four activation rows (two instructions
// for M <= 8), and block b takes its own 32 inputs of the wave's 512-input
// slice.  So one 16-byte load per lane brings four weight rows x 256
// contiguous bytes (eight whole 128-byte lines, as coalesced as one 1 KiB
// row) and feeds eight instructions, and the products cost no vector ALU
// time: what remains on the VALU is the unpack (7 ops per word), the
// per-(row, group) correction and the cross-lane sums, so each further
// activation row adds little vector ALU work.  The same A against a B of
// ones gives the activation sums of each lane's 32 inputs once, up front.
// A wave keeps its activations in registers for all of its rows; the waves
// of a block split K and add their partial rows through LDS in a fixed
// order.

constexpr int kQuadSlice = 512;   // inputs per wave and slice: 16 blocks x 32
constexpr int kQuadMaxWaves = 16;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4x4x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                           f32x4 c) {
  const u32x2 a = {a0, a1}, b = {b0, b1};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a),
                                                __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

template <int M, int T, int NB>
__global__ __launch_bounds__(1024) void gemv_quad_kernel(
    const uint16_t* __restrict__ X, int Mrt, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K, int lg,
    uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int MS = (M + 3) / 4;             // activation row sets of four
  constexpr int MP = pow2_at_least(M);        // values per lane in the halving butterfly
  constexpr int LM = log2_exact(MP);
  static_assert(LM <= 4, "at most 16 values per lane");
  __shared__ float red[kQuadMaxWaves][NB * 4 * M];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int bq = lane >> 2;                   // block of the 4x4 products: 32 inputs
  const int j = lane & 3;                     // weight row (B column) / activation row (A row)
  const int G = K >> lg;                      // groups of 2^lg inputs (32, 64 or 128)
  const int64_t vpr = K / 32;                 // 16-byte vectors per code row

  int kc[T], g[T];
  bool act[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int k = (wave * T + t) * kQuadSlice + 32 * bq;
    act[t] = k < K;
    kc[t] = act[t] ? k : K - 32;              // inactive lanes read valid memory, weigh zero
    g[t] = kc[t] >> lg;                       // a block of 32 inputs lies in one group
  }
  const int row0 = blockIdx.x * NB * 4;
  const u32x4* cbase = reinterpret_cast<const u32x4*>(codes);

  u32x4 cb[2];
  uint32_t sb[2];
  int zb[2];
  auto load = [&](int buf, int nb, int t) {
    const int row = min(row0 + nb * 4 + j, N - 1);
    cb[buf] = __builtin_nontemporal_load(cbase + (int64_t)row * vpr + kc[t] / 32);
    sb[buf] = scales[(int64_t)row * G + g[t]];
    zb[buf] = zeros[(int64_t)row * G + g[t]];
  };
  load(0, 0, 0);  // the weight stream first

  // lane (bq, i) holds activation rows i, i + 4 of its 32 inputs, paired
  // like the codes, and every lane the sums of the 32 inputs of its block
  u32x4 xa[T][MS][4];
  f32x4 xs[T][MS];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int m = j + 4 * ms;
      const bool live = act[t] && m < Mrt;
      const u32x4* xr = reinterpret_cast<const u32x4*>(X + (int64_t)min(m, Mrt - 1) * ldx + kc[t]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 raw = xr[i];
        if (!live) raw = u32x4{0u, 0u, 0u, 0u};
        xa[t][ms][i] = x_pairs_from_natural(raw);
      }
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          sum = mfma4x4x4(xa[t][ms][i][2 * h], xa[t][ms][i][2 * h + 1], kOnePair, kOnePair, sum);
      xs[t][ms] = sum;
    }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float acc[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) acc[m] = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int f = nb * T + t;
      const int cur = f & 1;
      if (f + 1 < NB * T) load(cur ^ 1, (f + 1) / T, (f + 1) % T);
      f32x4 d[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) d[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 q = codes_to_bias128_pairs(cb[cur][i]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
            d[ms] = mfma4x4x4(xa[t][ms][i][2 * h], xa[t][ms][i][2 * h + 1], q[2 * h], q[2 * h + 1],
                              d[ms]);
      }
      // this lane's block: s * (P - (128 + z) * Xsum) for weight row j, group g[t]
      const float s = bf16_to_f32(sb[cur]);
      const float zb128 = (float)zb[cur] + 128.f;
#pragma unroll
      for (int m = 0; m < M; ++m)
        acc[m] = fmaf(s, fmaf(-zb128, xs[t][m / 4][m % 4], d[m / 4][m % 4]), acc[m]);
    }
    // sum over the 16 blocks (lane bits 2..5): halving on the activation
    // rows first (bit 5 first), plain sums after
    int mask = 32;
#pragma unroll
    for (int cur_n = MP; cur_n > 1; cur_n >>= 1) {
      const uint32_t up = (lane & mask) ? ~0u : 0u;
#pragma unroll
      for (int i = 0; i < cur_n / 2; ++i) {
        const float send = pick(up, acc[i], acc[i + cur_n / 2]);
        const float keep = pick(up, acc[i + cur_n / 2], acc[i]);
        acc[i] = keep + __shfl_xor(send, mask);
      }
      mask >>= 1;
    }
#pragma unroll
    for (; mask >= 4; mask >>= 1) acc[0] += __shfl_xor(acc[0], mask);
    // lane (bq, j) now holds weight row j and activation row m from the top
    // LM bits of bq; the lanes with zero low bits store it
    if ((bq & ((16 >> LM) - 1)) == 0) {
      int m = 0, half = MP / 2;
#pragma unroll
      for (int b = 0; b < LM; ++b, half >>= 1)
        if (lane & (32 >> b)) m += half;
      if (m < M) red[wave][nb * 4 * M + j * M + m] = acc[0];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NB * 4 * M; idx += blockDim.x) {
    const int r = idx / M, m = idx - r * M;
    const int row = row0 + r;
    if (row >= N || m >= Mrt) continue;
    float v = red[0][idx];
    for (int w = 1; w < S; ++w) v += red[w][idx];
    Y[m * ldy + row] = f32_to_bf16_rne(v);
  }
}

// Long rows (more slices than one wave can hold the activations of): each
// wave runs every S-th slice in turn, loads that slice's activations, and
// adds into per-row accumulators of all NB batches, so the activations are
// fetched once per slice and the sums across lanes run once per row at the
// end.  NB is even so that the double buffer's parity is static.
template <int M, int NB>
__global__ __launch_bounds__(1024) void gemv_quad_long_kernel(
    const uint16_t* __restrict__ X, int Mrt, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K, int lg,
    uint16_t* __restrict__ Y, int64_t ldy) {
  static_assert(NB % 2 == 0, "even batch count");
  constexpr int MS = (M + 3) / 4;
  constexpr int MP = pow2_at_least(M);
  constexpr int LM = log2_exact(MP);
  static_assert(LM <= 4, "at most 16 values per lane");
  __shared__ float red[kQuadMaxWaves][NB * 4 * M];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int bq = lane >> 2;
  const int j = lane & 3;
  const int G = K >> lg;
  const int64_t vpr = K / 32;
  const int slices = (K + kQuadSlice - 1) / kQuadSlice;
  const int row0 = blockIdx.x * NB * 4;
  const u32x4* cbase = reinterpret_cast<const u32x4*>(codes);

  float acc[NB][MP];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int m = 0; m < MP; ++m) acc[nb][m] = 0.f;

  if (wave < slices) {
    auto lane_k = [&](int t, bool& act) {
      const int k = t * kQuadSlice + 32 * bq;
      act = k < K;
      return act ? k : K - 32;
    };
    u32x4 cb[2];
    uint32_t sb[2];
    int zb[2];
    auto load = [&](int buf, int nb, int t) {
      bool act;
      const int kc = lane_k(t, act);
      const int row = min(row0 + nb * 4 + j, N - 1);
      cb[buf] = __builtin_nontemporal_load(cbase + (int64_t)row * vpr + kc / 32);
      sb[buf] = scales[(int64_t)row * G + (kc >> lg)];
      zb[buf] = zeros[(int64_t)row * G + (kc >> lg)];
    };
    load(0, 0, wave);
    for (int t = wave; t < slices; t += S) {
      bool act;
      const int kc = lane_k(t, act);
      u32x4 xa[MS][4];
      f32x4 xs[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int m = j + 4 * ms;
        const bool live = act && m < Mrt;
        const u32x4* xr = reinterpret_cast<const u32x4*>(X + (int64_t)min(m, Mrt - 1) * ldx + kc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 raw = xr[i];
          if (!live) raw = u32x4{0u, 0u, 0u, 0u};
          xa[ms][i] = x_pairs_from_natural(raw);
        }
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            sum = mfma4x4x4(xa[ms][i][2 * h], xa[ms][i][2 * h + 1], kOnePair, kOnePair, sum);
        xs[ms] = sum;
      }
      const int tn = t + S < slices ? t + S : t;   // the last slice re-reads itself
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int cur = nb & 1;
        if (nb + 1 < NB) load(cur ^ 1, nb + 1, t);
        else load(cur ^ 1, 0, tn);
        f32x4 d[MS];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) d[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 q = codes_to_bias128_pairs(cb[cur][i]);
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
              d[ms] = mfma4x4x4(xa[ms][i][2 * h], xa[ms][i][2 * h + 1], q[2 * h], q[2 * h + 1],
                                d[ms]);
        }
        const float s = bf16_to_f32(sb[cur]);
        const float zb128 = (float)zb[cur] + 128.f;
#pragma unroll
        for (int m = 0; m < M; ++m)
          acc[nb][m] = fmaf(s, fmaf(-zb128, xs[m / 4][m % 4], d[m / 4][m % 4]), acc[nb][m]);
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int mask = 32;
#pragma unroll
    for (int cur_n = MP; cur_n > 1; cur_n >>= 1) {
      const uint32_t up = (lane & mask) ? ~0u : 0u;
#pragma unroll
      for (int i = 0; i < cur_n / 2; ++i) {
        const float send = pick(up, acc[nb][i], acc[nb][i + cur_n / 2]);
        const float keep = pick(up, acc[nb][i + cur_n / 2], acc[nb][i]);
        acc[nb][i] = keep + __shfl_xor(send, mask);
      }
      mask >>= 1;
    }
#pragma unroll
    for (; mask >= 4; mask >>= 1) acc[nb][0] += __shfl_xor(acc[nb][0], mask);
    if ((bq & ((16 >> LM) - 1)) == 0) {
      int m = 0, half = MP / 2;
#pragma unroll
      for (int b = 0; b < LM; ++b, half >>= 1)
        if (lane & (32 >> b)) m += half;
      if (m < M) red[wave][nb * 4 * M + j * M + m] = acc[nb][0];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NB * 4 * M; idx += blockDim.x) {
    const int r = idx / M, m = idx - r * M;
    const int row = row0 + r;
    if (row >= N || m >= Mrt) continue;
    float v = red[0][idx];
    for (int w = 1; w < S; ++w) v += red[w][idx];
    Y[m * ldy + row] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------------------------------
// gemv_tile (9 <= M <= 32, and the shapes the other kernels leave): weights
// on the matrix cores, codes streamed
// ---------------------------------------------------------------------------
//
// D = A B on v_mfma_f32_16x16x32_bf16 with A = 16 activation rows (M padded)
// and B = 16 weight rows, so lane (r16, q) of a result tile holds weight row
// r16 for activation rows 4q .. 4q+3 and needs one scale / zero point.  One
// 16-byte load per lane brings four code words of one row: a row tile's
// group (16 rows x 64 B) per instruction; word 4q + t feeds k-step t, so
// k-step t covers inputs 32q + 8t .. +7 of the group in lane group q, and
// the activation fragment of lane (m, q) for k-step t is the 16 bytes of X
// at that position, paired like the codes.  The same A against a B of ones
// gives the activation sums of the group in the result layout.  A wave runs
// RT row tiles over its share of the groups, the next group's codes and
// activations in flight; the waves of a block split K and add their partial
// tiles through LDS in a fixed order.

constexpr int kTileMaxWaves = 8;

template <int MT, int RT>
__global__ __launch_bounds__(512) void gemv_tile_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy) {
  __shared__ float red[kTileMaxWaves][RT * MT * 4][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int S = blockDim.x / kWave;
  const int G = K / kGroup;
  const int r16 = lane & 15, q = lane >> 4;
  const int gb = (G * wave) / S, ge = (G * (wave + 1)) / S;

  // weight rows of this lane (one per row tile), clamped for loads
  const u32x4* crow[RT];
  const uint16_t* srow[RT];
  const int32_t* zrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = min((int)blockIdx.x * 16 * RT + 16 * rt + r16, N - 1);
    crow[rt] = reinterpret_cast<const u32x4*>(codes + (int64_t)n * (K / 8)) + q;
    srow[rt] = scales + (int64_t)n * G;
    zrow[rt] = zeros + (int64_t)n * G;
  }
  // activation rows of this lane (A operand rows r16 + 16 mt); rows past M
  // read row 0 and are zeroed after the load
  const u32x4* xrow[MT];
  bool xvalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = r16 + 16 * mt;
    xvalid[mt] = m < M;
    xrow[mt] = reinterpret_cast<const u32x4*>(X + (int64_t)(xvalid[mt] ? m : 0) * ldx) + 4 * q;
  }

  const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};
  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (gb < ge) {
    u32x4 cw[2][RT];          // code words of a group: word 4q + t in element t
    u32x4 xr[2][4][MT];       // activation fragments of a group, per k-step
    uint32_t sr[2][RT];
    int zr[2][RT];
    auto load = [&](int buf, int g) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        cw[buf][rt] = __builtin_nontemporal_load(crow[rt] + g * 4);
        sr[buf][rt] = srow[rt][g];
        zr[buf][rt] = zrow[rt][g];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xr[buf][t][mt] = xrow[mt][g * 16 + t];
    };
    auto compute = [&](int buf) {
      f32x4 P[RT][MT], xs[MT];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          u32x4 raw = xr[buf][t][mt];
          if (!xvalid[mt]) raw = u32x4{0u, 0u, 0u, 0u};
          a[mt] = x_pairs_from_natural(raw);
          xs[mt] = mfma16x16x32(a[mt], ones, t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : xs[mt]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const u32x4 b = codes_to_bias128_pairs(cw[buf][rt][t]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            P[rt][mt] = mfma16x16x32(a[mt], b, t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[rt][mt]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float sc = bf16_to_f32(sr[buf][rt]);
        const float zb = (float)zr[buf][rt] + 128.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[rt][mt][i] = fmaf(sc, fmaf(-zb, xs[mt][i], P[rt][mt][i]), acc[rt][mt][i]);
      }
    };
    load(0, gb);
    int g = gb;
    for (; g + 1 < ge; g += 2) {
      load(1, g + 1);
      compute(0);
      if (g + 2 < ge) load(0, g + 2);
      compute(1);
    }
    if (g < ge) compute(0);
  }

  if (S > 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][(rt * MT + mt) * 4 + i][lane] = acc[rt][mt][i];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = red[0][(rt * MT + mt) * 4 + i][lane];
          for (int w = 1; w < S; ++w) v += red[w][(rt * MT + mt) * 4 + i][lane];
          acc[rt][mt][i] = v;
        }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = (int)blockIdx.x * 16 * RT + 16 * rt + r16;
    if (n >= N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mt + 4 * q + i;
        if (m < M) Y[(int64_t)m * ldy + n] = f32_to_bf16_rne(acc[rt][mt][i]);
      }
  }
}

// ---------------------------------------------------------------------------
// launch selection
// ---------------------------------------------------------------------------

constexpr int kDotMaxM = 4;

int cu_count() { return device_cu_count(); }

template <int M, int NB, bool PL, bool W8>
void launch_dot_nb(const uint16_t* X, int64_t ldx, const uint32_t* codes, const uint16_t* scales,
                   const int32_t* zeros, int N, int K, int lg, uint16_t* Y, int64_t ldy,
                   hipStream_t stream) {
  constexpr int R = 4;
  const int S = (K + kSlice - 1) / kSlice;
  hipLaunchKernelGGL((gemv_dot_kernel<M, R, NB, PL, W8>), dim3((unsigned)((N + R * NB - 1) / (R * NB))),
                     dim3(S * kWave), 0, stream, X, ldx, codes, scales, zeros, N, K, lg, Y, ldy);
}

template <int M, bool PL, bool W8 = false>
void launch_dot(const uint16_t* X, int64_t ldx, const uint32_t* codes, const uint16_t* scales,
                const int32_t* zeros, int N, int K, int lg, uint16_t* Y, int64_t ldy,
                hipStream_t stream) {
  // Rows per block: R = 4 rows per batch, NB batches, the next batch's loads
  // in flight while the current one is reduced.  Per-wave timelines on the
  // box show that a CU's share of the bandwidth does not grow with the
  // number of blocks it holds, so a block count that is not a multiple of
  // the CU count leaves a tail; and that about eight waves per CU with a
  // few batches each keep the stream full with the least queueing.  So:
  // aim at 8 waves per CU (NB ~ waves needed / (8 CUs)), then step down to
  // the nearest NB whose block count fills the CUs evenly.  Fitted to
  // timings of every decode layer of the 8B- and 70B-shaped sets and the
  // 40-layer stack.
  constexpr int R = 4;
  // more batches would spill at M = 4 (with 8-bit codes, from M = 3)
  constexpr int kMaxNB = (W8 && M >= 3) ? 1 : (M >= 4 ? 2 : 8);
  const int S = (K + kSlice - 1) / kSlice;
  const int cus = cu_count();
  auto balance = [&](int nb) {
    const double per_cu = (double)((N + R * nb - 1) / (R * nb)) / cus;
    return per_cu / std::ceil(per_cu);
  };
  const int64_t waves1 = (int64_t)((N + R - 1) / R) * S;   // waves at one batch each
  int nb0 = (int)std::min<int64_t>(kMaxNB, std::max<int64_t>(1, (waves1 + 8 * cus - 1) / (8 * cus)));
  int nb = 0;
  for (int c = nb0; c >= 1 && nb == 0; --c)
    if (balance(c) >= 0.97) nb = c;
  if (nb == 0) {   // nothing fills evenly: the best fill, nearest to nb0
    nb = nb0;
    for (int c = 1; c <= kMaxNB; ++c)
      if (balance(c) > balance(nb) + 1e-9 ||
          (balance(c) > balance(nb) - 1e-9 && std::abs(c - nb0) < std::abs(nb - nb0)))
        nb = c;
  }
  switch (nb) {
#define W4A16_DOT(V)                                                                   \
  case V:                                                                              \
    launch_dot_nb<M, (V <= kMaxNB ? V : kMaxNB), PL, W8>(X, ldx, codes, scales, zeros, N, K, lg, Y, ldy, stream); \
    break;
    W4A16_DOT(8) W4A16_DOT(7) W4A16_DOT(6) W4A16_DOT(5) W4A16_DOT(4) W4A16_DOT(3) W4A16_DOT(2)
#undef W4A16_DOT
    default:
      launch_dot_nb<M, 1, PL, W8>(X, ldx, codes, scales, zeros, N, K, lg, Y, ldy, stream);
  }
}


template <int M, int T, int NB>
void launch_quad_nb(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes,
                    const uint16_t* scales, const int32_t* zeros, int N, int K, int lg, uint16_t* Y,
                    int64_t ldy, hipStream_t stream) {
  const int slices = (K + kQuadSlice - 1) / kQuadSlice;
  const int S = (slices + T - 1) / T;
  hipLaunchKernelGGL((gemv_quad_kernel<M, T, NB>), dim3((unsigned)((N + 4 * NB - 1) / (4 * NB))),
                     dim3(S * kWave), 0, stream, X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy);
}

template <int M, int T>
void launch_quad_t(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes,
                   const uint16_t* scales, const int32_t* zeros, int N, int K, int lg, uint16_t* Y,
                   int64_t ldy, hipStream_t stream) {
  // Rows per block: 4 x NB.  The largest NB (at most 8) whose block count
  // fills the CUs evenly; fitted to timings of the decode layers of the 8B-
  // and 70B-shaped sets and the 40-layer stack at M = 4 and 8.
  const int cus = cu_count();
  auto balance = [&](int nb) {
    const double per_cu = (double)((N + 4 * nb - 1) / (4 * nb)) / cus;
    return per_cu / std::ceil(per_cu);
  };
  int nb = 0;
  for (int c = 8; c >= 1 && nb == 0; --c)
    if (balance(c) >= 0.95) nb = c;
  if (nb == 0) {
    nb = 1;
    for (int c = 2; c <= 8; ++c)
      if (balance(c) > balance(nb) + 1e-9) nb = c;
  }
  switch (nb) {
#define W4A16_QUAD(V)                                                                     \
  case V:                                                                                 \
    launch_quad_nb<M, T, V>(X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy, stream); \
    break;
    W4A16_QUAD(8) W4A16_QUAD(7) W4A16_QUAD(6) W4A16_QUAD(5) W4A16_QUAD(4) W4A16_QUAD(3)
    W4A16_QUAD(2)
#undef W4A16_QUAD
    default:
      launch_quad_nb<M, T, 1>(X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy, stream);
  }
}

template <int M, int NB>
void launch_quad_long_nb(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes,
                         const uint16_t* scales, const int32_t* zeros, int N, int K, int lg,
                         uint16_t* Y, int64_t ldy, int S, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_quad_long_kernel<M, NB>), dim3((unsigned)((N + 4 * NB - 1) / (4 * NB))),
                     dim3(S * kWave), 0, stream, X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy);
}

// Long rows: S = 16 waves (one block per CU) or 8 (two), NB = the fewest
// even batches whose blocks fit on the CUs in one pass; fitted to timings
// of the down projections of the 70B-shaped set and the 40-layer stack.
// Returns false when that leaves fewer blocks than half the CUs (a short
// layer: the caller takes another kernel).
template <int M>
bool launch_quad_long(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes,
                      const uint16_t* scales, const int32_t* zeros, int N, int K, int lg, uint16_t* Y,
                      int64_t ldy, hipStream_t stream, bool need) {
  constexpr int kMaxNB = M <= 4 ? 8 : 4;   // more rows of accumulators would spill
  const int cus = cu_count();
  const int slices = (K + kQuadSlice - 1) / kQuadSlice;
  int S = 0, nb = 0;
  for (int s : {16, 8}) {
    const int st = std::min(s, slices);
    const int64_t cap = (int64_t)cus * (16 / s);
    for (int c = 2; c <= kMaxNB && nb == 0; c += 2)
      if ((N + 4 * c - 1) / (4 * c) <= cap) nb = c;
    if (nb) { S = st; break; }
  }
  if (nb == 0) { S = std::min(8, slices); nb = kMaxNB; }
  if (!need && (N + 4 * nb - 1) / (4 * nb) < cus / 2) return false;
  switch (nb) {
#define W4A16_QL(V)                                                                           \
  case V:                                                                                     \
    launch_quad_long_nb<M, (V <= kMaxNB ? V : kMaxNB)>(X, Mrt, ldx, codes, scales, zeros, N, K, \
                                                       lg, Y, ldy, S, stream);                \
    break;
    W4A16_QL(2) W4A16_QL(4) W4A16_QL(6) W4A16_QL(8)
  }
#undef W4A16_QL
  return true;
}

// 3 <= M <= 8, K <= 16384: one wave slice of 512 inputs (T = 1) up to 16
// waves, two slices per wave beyond that
template <int M>
void launch_quad(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes,
                 const uint16_t* scales, const int32_t* zeros, int N, int K, int lg, uint16_t* Y,
                 int64_t ldy, hipStream_t stream) {
  const int slices = (K + kQuadSlice - 1) / kQuadSlice;
  if (slices <= kQuadMaxWaves)
    launch_quad_t<M, 1>(X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy, stream);
  else
    launch_quad_t<M, 2>(X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy, stream);
}

}  // namespace

int launch_gemm(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*, const int32_t*,
                int64_t, int64_t, int, uint16_t*, int64_t, hipStream_t);

namespace {
// Groups of 32 or 64 inputs (lg = 5, 6): the per-lane fold of gemv_dot for
// M <= 2, the 32-input blocks of the quad kernels (one group per block at
// any size) up to M = 8, and the prefill kernel above.
int launch_gemv_small_groups(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                             const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                             int lg, uint16_t* Y, int64_t ldy, hipStream_t stream) {
  const int n = (int)N, k = (int)K, m = (int)M;
  if (M <= 2 && K <= (int64_t)kSlice * kMaxSlices) {
    if (M == 1) launch_dot<1, true>(X, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream);
    else launch_dot<2, true>(X, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream);
  } else if (M <= 8 && K <= (int64_t)2 * kQuadSlice * kQuadMaxWaves) {
    if (M <= 4) launch_quad<4>(X, m, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream);
    else launch_quad<8>(X, m, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream);
  } else if (M <= 8) {
    if (M <= 4) launch_quad_long<4>(X, m, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream, true);
    else launch_quad_long<8>(X, m, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream, true);
  } else {
    return launch_gemm(X, M, ldx, codes, scales, zeros, N, K, 1 << lg, Y, ldy, stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
}  // namespace

// W8A16 variant, 1 <= M <= 4, K <= 32768 (checked by the caller)
int launch_gemv_int8(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                     const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                     uint16_t* Y, int64_t ldy, hipStream_t stream) {
  const int n = (int)N, k = (int)K;
  switch (M) {
    case 1: launch_dot<1, false, true>(X, ldx, codes, scales, zeros, n, k, 7, Y, ldy, stream); break;
    case 2: launch_dot<2, false, true>(X, ldx, codes, scales, zeros, n, k, 7, Y, ldy, stream); break;
    case 3: launch_dot<3, false, true>(X, ldx, codes, scales, zeros, n, k, 7, Y, ldy, stream); break;
    default: launch_dot<4, false, true>(X, ldx, codes, scales, zeros, n, k, 7, Y, ldy, stream); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// group: 32, 64 or 128 inputs per quantisation group (checked by the caller)
int launch_gemv(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t ldy, hipStream_t stream) {
  if (group != kGroup)
    return launch_gemv_small_groups(X, M, ldx, codes, scales, zeros, N, K, group == 32 ? 5 : 6, Y,
                                    ldy, stream);
  constexpr int lg = 7;
  if (M >= 3 && M <= 8 && K <= (int64_t)2 * kQuadSlice * kQuadMaxWaves) {
    if (M <= 4)
      launch_quad<4>(X, (int)M, ldx, codes, scales, zeros, (int)N, (int)K, lg, Y, ldy, stream);
    else
      launch_quad<8>(X, (int)M, ldx, codes, scales, zeros, (int)N, (int)K, lg, Y, ldy, stream);
    return hipGetLastError() == hipSuccess ? 0 : 4;
  }
  if (M >= 3 && M <= 8) {
    const bool done =
        M <= 4 ? launch_quad_long<4>(X, (int)M, ldx, codes, scales, zeros, (int)N, (int)K, lg, Y,
                                     ldy, stream, false)
               : launch_quad_long<8>(X, (int)M, ldx, codes, scales, zeros, (int)N, (int)K, lg, Y,
                                     ldy, stream, true);
    if (done) return hipGetLastError() == hipSuccess ? 0 : 4;
  }
  if (M <= kDotMaxM && K <= (int64_t)kSlice * kMaxSlices) {
    const int n = (int)N, k = (int)K;
    switch (M) {
      case 1: launch_dot<1, false>(X, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream); break;
      case 2: launch_dot<2, false>(X, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream); break;
      case 3: launch_dot<3, false>(X, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream); break;
      default: launch_dot<4, false>(X, ldx, codes, scales, zeros, n, k, lg, Y, ldy, stream); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
  }
  // Row tiles per wave: more for tall layers (each activation fragment is
  // reused by every tile); four waves per block split K.  Fitted to timings
  // of the 8B- and 70B-shaped layers at M = 8, 16, 32.
  const int n_ = (int)N, k_ = (int)K, m_ = (int)M;
  const int G = k_ / kGroup;
  const int S = max(1, min(4, G / 2));
  const dim3 block(S * kWave);
  int rt = n_ >= 16384 ? 4 : (n_ >= 6144 ? 2 : 1);
  if (M > 16 && rt > 2) rt = 2;   // four tiles of 32 activation rows would spill
  const dim3 grid((unsigned)((n_ + 16 * rt - 1) / (16 * rt)));
#define W4A16_TILE(MT, RT)                                                                       \
  hipLaunchKernelGGL((gemv_tile_kernel<MT, RT>), grid, block, 0, stream, X, m_, ldx, codes, scales, \
                     zeros, n_, k_, Y, ldy)
  if (M <= 16) {
    if (rt == 4) W4A16_TILE(1, 4); else if (rt == 2) W4A16_TILE(1, 2); else W4A16_TILE(1, 1);
  } else {
    if (rt == 2) W4A16_TILE(2, 2); else W4A16_TILE(2, 1);
  }
#undef W4A16_TILE
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
