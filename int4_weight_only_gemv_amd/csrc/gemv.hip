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
// per-row partial sums are folded across lanes (DPP and permlane swaps, no
// LDS), then across the K slices of the block through LDS in a fixed order.
//
// gemv_quad (3 <= M <= 8, K <= 16384, or longer rows split over blocks
// through a caller's workspace): the same streaming pattern (four rows x 256
// contiguous bytes per load instruction), but the products run on the
// matrix cores as sixteen 4x4 blocks per instruction, so more activation
// rows cost almost no vector ALU time.
//
// gemv_walk (9 <= M <= 32): 16-row tiles of W meet X (M padded to 16 or
// 32) on v_mfma_f32_16x16x32_bf16.  A block of 16 waves holds the
// activations of its run of K in registers and walks a run of row tiles,
// codes streaming through LDS by direct-to-LDS copies; rows longer than 32
// groups split K over blocks through a caller's workspace.
//
// gemv_ring (the shapes the others leave: long rows without a workspace,
// M <= 8 rows too long for gemv_dot and gemv_quad): one 16-row tile per
// block, its waves splitting K, codes through a two-stage LDS ring.
//
// Sums across waves and blocks run in a fixed order: results are
// deterministic.

#include "common.h"

#include <cmath>

namespace w4a16 {
namespace {

// ---------------------------------------------------------------------------
// gemv_dot
// ---------------------------------------------------------------------------

constexpr int kSlice = 2048;      // inputs per wave: 64 lanes x 32
constexpr int kMaxSlices = 16;    // K <= 32768 on this kernel

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
      sum += dpp<kDppXor1>(sum);
      xsg[m] = sum + dpp<kDppXor2>(sum);
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
    // Sum over the 4 lanes of the group, halving on the rows (lane bit 1
    // picks rows {0,1} or {2,3}, bit 0 one of those), so that lane l ends
    // with the group sums of row l % 4 ...
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
      const float s = bf16_to_f32(sb[cur][0]);
      const float zb128 = (float)zb[cur][0] + (W8 ? 384.f : 128.f);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float q = pick(up, h[1][m] + dpp<kDppXor1>(h[1][m]), h[0][m] + dpp<kDppXor1>(h[0][m]));
        // ... and removes the bias and zero point of that (row, group) once
        // (already done per lane with PL)
        part[m] = PL ? q : s * fmaf(-zb128, xsg[m], q);
      }
#pragma unroll
      for (int m = M; m < MP; ++m) part[m] = 0.f;
    }
    // then over the 16 groups of the slice (lane bits 2..5)
    lane_tree_sum<MP, LM>(part, lane);
    int m;
    if (tree_result<MP, LM>(lane, m) && m < M) red[wave][nb * R * M + (lane & 3) * M + m] = part[0];
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

constexpr int kQuadRing = 3;      // code vectors in flight per lane

// Split-K workspace (shared by the quad and walk kernels): a fixed region of
// kSplitMaxRanges counters, one per 64-byte line, then the partial outputs.
// Each launch leaves every counter at zero.
constexpr int kSplitMaxRanges = 1024;
constexpr int kSplitCounterBytes = 64;
constexpr int64_t kSplitCounterWords = (int64_t)kSplitMaxRanges * kSplitCounterBytes / 4;

template <int M, int T, int NB, bool SPLIT>
__global__ __launch_bounds__(1024) void gemv_quad_kernel(
    const uint16_t* __restrict__ X, int Mrt, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K, int lg,
    uint16_t* __restrict__ Y, int64_t ldy, int KS, unsigned* __restrict__ ws) {
  constexpr int MS = (M + 3) / 4;             // activation row sets of four
  constexpr int MP = pow2_at_least(M);        // values per lane in the lane tree
  constexpr int LM = log2_exact(MP);
  constexpr int F = NB * T;                   // items: (batch of four rows, slice)
  constexpr int D = F < kQuadRing ? F : kQuadRing;
  // two slices of eight activation rows fill the registers: the activation
  // sums then wait in LDS (each lane its own)
  constexpr bool kXsLds = M > 4 && T > 1;
  __shared__ float red[kQuadMaxWaves][NB * 4 * M];
  __shared__ f32x4 xs_lds[kXsLds ? kQuadMaxWaves : 1][kXsLds ? T * MS : 1][kWave];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int bq = lane >> 2;                   // block of the 4x4 products: 32 inputs
  const int j = lane & 3;                     // weight row (B column) / activation row (A row)
  const int G = K >> lg;                      // groups of 2^lg inputs (32, 64 or 128)
  const int64_t vpr = K / 32;                 // 16-byte vectors per code row

  // block = (range of NB batches of four rows, run ks of the KS runs of K)
  if constexpr (!SPLIT) KS = 1;
  const int range = (int)blockIdx.x / KS, ks = (int)blockIdx.x - range * KS;
  const int Kr = K / KS, kb = ks * Kr;        // the run: inputs kb .. kb + Kr - 1
  int kc[T], g[T];
  bool act[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int k = (wave * T + t) * kQuadSlice + 32 * bq;
    act[t] = k < Kr;
    kc[t] = kb + (act[t] ? k : Kr - 32);      // inactive lanes read valid memory, weigh zero
    g[t] = kc[t] >> lg;                       // a block of 32 inputs lies in one group
  }
  const int row0 = range * NB * 4;
  const u32x4* cbase = reinterpret_cast<const u32x4*>(codes);

  // item f = (batch f / T, slice f % T) in ring slot f % D
  u32x4 cb[D];
  uint32_t sb[D];
  int zb[D];
  auto load = [&](int slot, int f) {
    const int nb = f / T, t = f % T;
    const int row = min(row0 + nb * 4 + j, N - 1);
    cb[slot] = __builtin_nontemporal_load(cbase + (int64_t)row * vpr + kc[t] / 32);
    sb[slot] = scales[(int64_t)row * G + g[t]];
    zb[slot] = zeros[(int64_t)row * G + g[t]];
  };
#pragma unroll
  for (int f = 0; f < D; ++f) load(f, f);     // the weight stream first

  // lane (bq, i) holds activation rows i, i + 4 of its 32 inputs, paired
  // like the codes, and every lane the sums of the 32 inputs of its block
  u32x4 xa[T][MS][4];
  f32x4 xs[kXsLds ? 1 : T][kXsLds ? 1 : MS];
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
      if constexpr (kXsLds) xs_lds[wave][t * MS + ms][lane] = sum;
      else xs[t][ms] = sum;
    }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float acc[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) acc[m] = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int f = nb * T + t;
      const int slot = f % D;
      const u32x4 c = cb[slot];
      const float s = bf16_to_f32(sb[slot]);
      const float zb128 = (float)zb[slot] + 128.f;
      if (f + D < F) load(slot, f + D);
      f32x4 d[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) d[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 q = codes_to_bias128_pairs(c[i]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
            d[ms] = mfma4x4x4(xa[t][ms][i][2 * h], xa[t][ms][i][2 * h + 1], q[2 * h], q[2 * h + 1],
                              d[ms]);
      }
      // this lane's block: s * (P - (128 + z) * Xsum) for weight row j, group g[t]
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float xsm = kXsLds ? xs_lds[wave][t * MS + m / 4][lane][m % 4] : xs[kXsLds ? 0 : t][kXsLds ? 0 : m / 4][m % 4];
        acc[m] = fmaf(s, fmaf(-zb128, xsm, d[m / 4][m % 4]), acc[m]);
      }
    }
    // sum over the 16 blocks (lane bits 2..5); lane (bq, j) then holds
    // weight row j and activation row m
    lane_tree_sum<MP, LM>(acc, lane);
    int m;
    if (tree_result<MP, LM>(lane, m) && m < M) red[wave][nb * 4 * M + j * M + m] = acc[0];
  }
  __syncthreads();
  if (!SPLIT) {
    for (int idx = threadIdx.x; idx < NB * 4 * M; idx += blockDim.x) {
      const int r = idx / M, m = idx - r * M;
      const int row = row0 + r;
      if (row >= N || m >= Mrt) continue;
      float v = red[0][idx];
      for (int w = 1; w < S; ++w) v += red[w][idx];
      Y[m * ldy + row] = f32_to_bf16_rne(v);
    }
    return;
  }
  // K split over KS blocks: this block's sums go to the workspace with
  // coherent stores (contiguous per wave instruction); it waits for them,
  // counts itself in on its range's counter, and the last of the KS adds
  // the partials in run order, stores Y and resets the counter
  unsigned* part = ws + kSplitCounterWords + ((int64_t)range * KS + ks) * (NB * 4 * M);
  for (int idx = threadIdx.x; idx < NB * 4 * M; idx += blockDim.x) {
    float v = red[0][idx];
    for (int w = 1; w < S; ++w) v += red[w][idx];
    __hip_atomic_store(part + idx, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_vmcnt<0>();
  __syncthreads();
  unsigned* counter = ws + (int64_t)range * (kSplitCounterBytes / 4);
  __shared__ unsigned last;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(KS - 1);
  __syncthreads();
  if (!last) return;
  const unsigned* part0 = ws + kSplitCounterWords + (int64_t)range * KS * (NB * 4 * M);
  for (int idx = threadIdx.x; idx < NB * 4 * M; idx += blockDim.x) {
    const int r = idx / M, m = idx - r * M;
    const int row = row0 + r;
    if (row >= N || m >= Mrt) continue;
    float v = 0.f;
    for (int k = 0; k < KS; ++k)
      v += __uint_as_float(__hip_atomic_load(part0 + (int64_t)k * (NB * 4 * M) + idx, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
    Y[m * ldy + row] = f32_to_bf16_rne(v);
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    lane_tree_sum<MP, LM>(acc[nb], lane);
    int m;
    if (tree_result<MP, LM>(lane, m) && m < M) red[wave][nb * 4 * M + j * M + m] = acc[nb][0];
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
// Shared pieces of the matrix-core decode kernels (9 <= M <= 32)
// ---------------------------------------------------------------------------
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): lane (r16, q) holds A row
// r16 (an activation row) and B column r16 (a weight row) for inputs
// 8q .. 8q+7 of a K step, and result column r16 for activation rows
// 4q .. 4q+3.  K step t of a group covers its inputs 32t .. 32t+31: lane
// (r16, q) takes the group's code word 4t + q and the activations
// 32t + 8q .. +7 of its row.  The same A against a B of ones gives the
// group's activation sums.  Per group and weight row
//     acc += s * (P - (128 + z) * Xsum),   P = sum_k x (128 + q),
// with one exact product, as in the other kernels.
//
// Codes travel by direct-to-LDS copies (global_load_lds_dwordx4) of 8 code
// rows x 128 bytes (two groups): whole 128-byte lines, the pattern that reads
// HBM fastest, and code bytes in flight hold no registers.  A copy puts row
// r's 16-byte chunk c into slot c ^ r (^ 1 for the second copy of a 16-row
// tile) of the row's 128 LDS bytes, which spreads the 4-byte B reads of one
// instruction over all 64 banks.

constexpr int kRingCopy = 1024;   // one copy: 8 code rows x 128 bytes

// ---------------------------------------------------------------------------
// gemv_walk (9 <= M <= 32): activations held, row tiles walked
// ---------------------------------------------------------------------------
//
// A block of 16 waves owns a run of 16-row tiles of W and a run of at most 32
// groups of K (all of K, or one of KS equal runs; KS > 1 needs a workspace).
// Wave w owns two groups of the run: it reads their activations once, as
// whole 128-byte lines, moves them into the A layout with lane permutes, and
// keeps them (and their activation sums) in registers for every row tile of
// the block, so X crosses the L2 once per block.  The two groups' slot in
// the run is (w + block) % 16, so that at any moment the blocks read
// different parts of X.  The block's scales and zero points come into LDS
// with coalesced loads (rows padded to an odd number of words, so that the
// 16 rows of one read instruction fall on distinct banks).  Then each wave
// streams its two groups of every row tile through a two-tile ring in LDS,
// one tile ahead, and per tile the 16 waves' partial tiles are added through
// LDS in a fixed order.  The issue order is: the first tile's code copies,
// the activations, the scales and zero points; inside the walk the only
// global operations are the code copies, so a fixed count of the in-order
// memory counter tells when a tile has landed.  The barriers inside the walk
// wait for LDS only (a __syncthreads() would also wait for the ring's
// copies in flight).
//
// KS = 1: the outputs collect in LDS and leave with coalesced stores.
// KS > 1: each block stores its partial outputs into the workspace with
// 32-bit agent-scope atomic stores (coherent across the XCDs' L2 caches),
// waits for them, then counts itself in on its row range's counter; the
// block that arrives last adds the KS partials in the order of their runs,
// stores Y and resets the counter to zero for the next launch.  Results do
// not depend on arrival order.

constexpr int kWalkWaves = 16;
constexpr int kWalkGroups = 2 * kWalkWaves;   // groups per block
constexpr int kWalkTile = 2 * kRingCopy;      // one wave's codes of a row tile
constexpr int kWalkRing = 2;                  // ring depth (tiles)
constexpr int kWalkMetaMax = 4096;            // scales (and zero points) per block
// LDS row strides of the block's tables, an odd number of 4-byte words
constexpr int kWalkSStride = 2 * kWalkGroups + 2;   // scales: 34 BF16 per row
constexpr int kWalkZStride = kWalkGroups + 1;       // zero points: 33 per row
constexpr int kWalkOStride = 34;                    // outputs: 34 BF16 per row (32 columns of M)
// Workspace of the split-K walk: the shared counter region (one counter per
// row range on its own 64-byte line, the same place for every shape and
// kernel), then the partial outputs, [range][run][tmax tiles][MT x 256]
// floats in the lanes' order.
constexpr int kWalkMaxRanges = kSplitMaxRanges;
constexpr int64_t kWalkCounterBytes = kSplitCounterBytes;

// dynamic LDS of a block walking at most tmax tiles
constexpr int walk_lds_bytes(int MT, int tmax) {
  return kWalkWaves * kWalkRing * kWalkTile             // code rings
         + 16 * tmax * kWalkSStride * 2                 // scales
         + 16 * tmax * kWalkZStride * 4                 // zero points
         + kWalkWaves * MT * 1024                       // partial tiles
         + 16 * tmax * kWalkOStride * 2;                // outputs
}

template <int MT>
__global__ __launch_bounds__(1024) void gemv_walk_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int tiles, int tmax, int KS, unsigned* __restrict__ ws) {
  constexpr int D = kWalkRing;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int G = K / kGroup;
  // block = (row range, run ks of the KS runs of K groups)
  const int nranges = (int)gridDim.x / KS;
  const int range = (int)blockIdx.x / KS, ks = (int)blockIdx.x - range * KS;
  const int t0 = (int)(((int64_t)tiles * range) / nranges);
  const int T = (int)(((int64_t)tiles * (range + 1)) / nranges) - t0;
  const int r0 = 16 * t0;
  const int rows = min(16 * T, N - r0);
  const int kb0 = (G * ks) / KS, GB = (G * (ks + 1)) / KS - kb0;   // the block's groups
  const int gl = 2 * (((int)blockIdx.x + wave) % kWalkWaves);      // the wave's, block-local
  const int g0 = kb0 + gl, ng = max(0, min(2, GB - gl));

  uint8_t* my = smem + wave * (D * kWalkTile);
  uint16_t* meta_s = reinterpret_cast<uint16_t*>(smem + kWalkWaves * D * kWalkTile);
  int32_t* meta_z = reinterpret_cast<int32_t*>(meta_s + 16 * tmax * kWalkSStride);
  float* red = reinterpret_cast<float*>(meta_z + 16 * tmax * kWalkZStride);
  uint16_t* out = reinterpret_cast<uint16_t*>(red + kWalkWaves * MT * 256);

  // 1. code copies of tile 0: lane -> row lane / 8 of a copy's 8, LDS slot
  //    lane % 8, which takes the row's chunk slot ^ row ^ h (copy h of the
  //    tile's two); rows past N re-read row N - 1
  const int crow = lane >> 3;
  auto copy_tile = [&](int t) {
    uint8_t* dst = my + (t % D) * kWalkTile;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = min(r0 + 16 * t + 8 * h + crow, N - 1);
      const int chunk = min(4 * g0 + ((lane & 7) ^ crow ^ h), 4 * max(g0 + ng, 1) - 1);
      copy16_to_lds(reinterpret_cast<const char*>(codes) + (int64_t)n * (K / 2) + 16 * chunk,
                    dst + h * kRingCopy);
    }
  };
  if (ng > 0 && T > 0) copy_tile(0);
  asm volatile("" ::: "memory");
  // 2. activations of the wave's two groups (rows past M re-read row M - 1;
  //    their results are not stored), read as whole 128-byte lines: window
  //    w (inputs 64 w .. 64 w + 63 of the pair of groups) of rows 8h .. 8h+7
  //    of activation tile mt, lane l holding row l / 8, inputs 8 (l % 8) ..
  u32x4 xr[MT][4][2];
  if (ng > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint16_t* xrow = X + (int64_t)min(16 * mt + 8 * h + (lane >> 3), M - 1) * ldx + 8 * (lane & 7);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          xr[mt][w][h] = *reinterpret_cast<const u32x4*>(xrow + (g0 + min(w >> 1, ng - 1)) * kGroup + 64 * (w & 1));
      }
  }
  asm volatile("" ::: "memory");
  // 3. the block's scales and zero points: rows r0 .. r0 + rows - 1, groups
  //    kb0 .. kb0 + GB - 1
  const int nmeta = rows * GB;
  uint32_t sv[kWalkMetaMax / 1024];
  int zv[kWalkMetaMax / 1024];
#pragma unroll
  for (int k = 0; k < kWalkMetaMax / 1024; ++k) {
    const int e = (int)threadIdx.x + 1024 * k;
    if (e < nmeta) {
      const int r = e / GB, g = e - r * GB;
      sv[k] = scales[(int64_t)(r0 + r) * G + kb0 + g];
      zv[k] = zeros[(int64_t)(r0 + r) * G + kb0 + g];
    }
  }
  asm volatile("" ::: "memory");

  // the A fragments: lane (r16, q) of K step t of group g takes row r16,
  // inputs 32 t + 8 q .. of the group, i.e. window 2 g + t / 2, chunk
  // 4 (t % 2) + q, held by lane 8 (r16 % 8) + 4 (t % 2) + q of half r16 / 8;
  // then paired like the codes (code j with code j + 4 of a word)
  u32x4 xb[2][4][MT];
  if (ng > 0) {
    const bool lo = r16 < 8;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int src = 4 * (8 * (r16 & 7) + 4 * s2 + q);
          u32x4 f;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t a = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)xr[mt][w][0][d]);
            const uint32_t b = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)xr[mt][w][1][d]);
            f[d] = lo ? a : b;
          }
          xb[w >> 1][2 * (w & 1) + s2][mt] = x_pairs_from_natural(f);
        }
  }
  // activation sums of the two groups, in the result layout
  const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};
  f32x4 xs[2][MT];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      if (ng > 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) a = mfma16x16x32(xb[g][t][mt], ones, a);
      }
      xs[g][mt] = a;
    }
#pragma unroll
  for (int k = 0; k < kWalkMetaMax / 1024; ++k) {
    const int e = (int)threadIdx.x + 1024 * k;
    if (e < nmeta) {
      const int r = e / GB, g = e - r * GB;
      meta_s[r * kWalkSStride + g] = (uint16_t)sv[k];
      meta_z[r * kWalkZStride + g] = zv[k];
    }
  }
  __syncthreads();

  // KS > 1: this block's partial outputs in the workspace
  unsigned* part = ws + (int64_t)kWalkMaxRanges * (kWalkCounterBytes / 4) +
                   ((int64_t)range * KS + ks) * (16 * tmax * 32);
  // B word of K step k of group g: this lane's row sits in copy r16 / 8 at
  // row r16 % 8, word 4k + q of the group in chunk 4g + k, which the copy put
  // in slot (4g + k) ^ swizzle; bits 4..6 of the offset hold the slot
  const int bsw = (r16 & 7) ^ (r16 >> 3);
  const int boffx = ((r16 >> 3) * kRingCopy + 128 * (r16 & 7) + 4 * q) | (16 * bsw);
  auto tile = [&](int t, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ng > 0) {
      // tile t landed (nothing is issued after it but the next tile's
      // copies, issued just below); then the copies of tile t + 1 into the
      // slot tile t - 1 freed
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      if (t + 1 < T) copy_tile(t + 1);
      asm volatile("" ::: "memory");
      const uint8_t* st = my + slot * kWalkTile;
      const int row = 16 * t + r16;   // block-local row of this lane
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if (g < ng) {
          const float s = bf16_to_f32(meta_s[row * kWalkSStride + gl + g]);
          const float z128 = (float)meta_z[row * kWalkZStride + gl + g] + 128.f;
          f32x4 P[MT];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(st + (boffx ^ (16 * (4 * g + k))));
            const u32x4 bv = codes_to_bias128_pairs(w);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              P[mt] = mfma16x16x32(xb[g][k][mt], bv, k == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[mt]);
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][i] = fmaf(s, fmaf(-z128, xs[g][mt][i], P[mt][i]), acc[mt][i]);
        }
      }
    }
    // the waves' partial tiles, added in a fixed order (tile element
    // e = 64 v + l: activation tile v / 4, i = v % 4)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * MT * 4 + mt * 4 + i) * 64 + lane] = acc[mt][i];
    block_barrier_lds();
    for (int e = threadIdx.x; e < MT * 256; e += 1024) {
      float sum = red[e];
#pragma unroll
      for (int w = 1; w < kWalkWaves; ++w) sum += red[w * MT * 256 + e];
      const int v = e >> 6, l = e & 63;
      const int m = 16 * (v >> 2) + 4 * (l >> 4) + (v & 3);
      const int r = 16 * t + (l & 15);
      if (KS == 1)
        out[r * kWalkOStride + m] = f32_to_bf16_rne(sum);
      else   // in the reduction's own order: a wave's stores are contiguous
        __hip_atomic_store(part + t * (MT * 256) + e, __float_as_uint(sum), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    block_barrier_lds();
  };
  // tiles in pairs, so that each tile's ring slot is a constant
  for (int t = 0; t < T; t += 2) {
    tile(t, Ic<0>{});
    if (t + 1 < T) tile(t + 1, Ic<1>{});
  }

  if (KS == 1) {
    // the block's outputs: Y[m][r0 + r], consecutive threads on consecutive r
    for (int e = threadIdx.x; e < rows * M; e += 1024) {
      const int m = e / rows, r = e - m * rows;
      Y[(int64_t)m * ldy + r0 + r] = out[r * kWalkOStride + m];
    }
    return;
  }
  // the block's partial stores are complete before it counts itself in (a
  // block barrier alone does not wait for global stores); the last of the
  // range's KS blocks adds the partials in the order of their runs
  wait_vmcnt<0>();
  __syncthreads();
  unsigned* counter = ws + (int64_t)range * (kWalkCounterBytes / 4);
  unsigned* last = reinterpret_cast<unsigned*>(out);
  if (threadIdx.x == 0) {
    const unsigned a = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last = a == (unsigned)(KS - 1);
  }
  __syncthreads();
  if (!*last) return;
  const unsigned* part0 = ws + (int64_t)kWalkMaxRanges * (kWalkCounterBytes / 4) +
                          (int64_t)range * KS * (16 * tmax * 32);
  for (int ea = threadIdx.x; ea < T * MT * 256; ea += 1024) {
    const int t = ea / (MT * 256), e = ea - t * (MT * 256);
    const int v = e >> 6, l = e & 63;
    const int m = 16 * (v >> 2) + 4 * (l >> 4) + (v & 3);
    const int r = 16 * t + (l & 15);
    if (r >= rows || m >= M) continue;
    float sum = 0.f;
    for (int k = 0; k < KS; ++k)
      sum += __uint_as_float(__hip_atomic_load(part0 + (int64_t)k * (16 * tmax * 32) + ea, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT));
    Y[(int64_t)m * ldy + r0 + r] = f32_to_bf16_rne(sum);
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// gemv_ring (M <= 32, the shapes gemv_walk leaves: rows longer than 32
// groups without a workspace, and M <= 8 rows too long for gemv_dot and
// gemv_quad)
// ---------------------------------------------------------------------------
//
// A block owns 16 weight rows and all of K; its 8 waves split K into
// contiguous runs of groups.  A wave streams its run of codes through a ring
// of two stages in LDS (a stage is two groups, one copy of 8 rows x 128
// bytes per 8 rows), and loads each group's activations, scales and zero
// points one group ahead into registers.  Memory operations of a wave, in
// issue order: at each stage start the copies of the next stage, at each
// group the activations, scales and zero points of the next group; nothing
// past the run is issued, so a fixed count of the in-order memory counter
// tells when a stage has landed.  The waves' partial tiles are added through
// LDS in a fixed order.

constexpr int kRingWaves = 8;
constexpr int kRingStage = 2 * kRingCopy;   // one wave's stage: 16 rows x two groups

template <int MT>
__global__ __launch_bounds__(kRingWaves * 64) void gemv_ring_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int W = kRingWaves, S = 2;
  constexpr int kBatch = 4 * MT + 2;        // memory operations per group batch
  __shared__ __attribute__((aligned(1024))) uint8_t ring[W * S * kRingStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int G = K / kGroup;
  const int gb = (G * wave) / W, ge = (G * (wave + 1)) / W;   // this wave's groups
  const int NG = ge - gb, NS = (NG + 1) / 2;
  const int n0 = blockIdx.x * 16;
  uint8_t* my = ring + wave * (S * kRingStage);

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (NG > 0) {
    // copies: lane -> row lane / 8 of the copy's 8, LDS slot lane % 8, which
    // takes the row's chunk slot ^ row ^ h (rows past N re-read row N - 1)
    const int crow = lane >> 3;
    const char* cptr[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      cptr[h] = reinterpret_cast<const char*>(codes) + (int64_t)min(n0 + 8 * h + crow, N - 1) * (K / 2);
    const int clast = 4 * ge - 1;   // the run's last 16-byte chunk
    auto copy_stage = [&](int slot, int j) {
      uint8_t* dst = my + slot * kRingStage;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        copy16_to_lds(cptr[h] + 16 * min(4 * gb + 8 * j + ((lane & 7) ^ crow ^ h), clast), dst + h * kRingCopy);
    };

    // activations of rows 16 mt + r16 (rows past M re-read row M - 1; their
    // results are not stored), scales and zero points of this lane's row
    const u32x4* xp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      xp[mt] = reinterpret_cast<const u32x4*>(X + (int64_t)min(16 * mt + r16, M - 1) * ldx) + q;
    const int nrow = min(n0 + r16, N - 1);
    const uint16_t* sp = scales + (int64_t)nrow * G + gb;
    const int32_t* zp = zeros + (int64_t)nrow * G + gb;
    u32x4 xb[2][4][MT];
    uint32_t sb[2];
    int zb[2];
    auto load_batch = [&](int b, int i) {   // group gb + i into batch b
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xb[b][t][mt] = xp[mt][(gb + i) * 16 + 4 * t];
      sb[b] = sp[i];
      zb[b] = zp[i];
    };

    const int bsw = (r16 & 7) ^ (r16 >> 3);
    const int boffx = ((r16 >> 3) * kRingCopy + 128 * (r16 & 7) + 4 * q) | (16 * bsw);
    const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};
    auto compute = [&](int b, const uint8_t* st, auto gsc) {
      constexpr int gs = decltype(gsc)::value;
      f32x4 xs[MT], P[MT];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(st + (boffx ^ (16 * (4 * gs + t))));
        const u32x4 bv = codes_to_bias128_natural(w, kExpBytes);   // natural order, like X
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          xs[mt] = mfma16x16x32(xb[b][t][mt], ones, t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : xs[mt]);
          P[mt] = mfma16x16x32(xb[b][t][mt], bv, t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : P[mt]);
        }
      }
      const float s = bf16_to_f32(sb[b]);
      const float z128 = (float)zb[b] + 128.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = fmaf(s, fmaf(-z128, xs[mt][i], P[mt][i]), acc[mt][i]);
    };

    // prologue: stage 0 and batch 0
    copy_stage(0, 0);
    asm volatile("" ::: "memory");
    load_batch(0, 0);
    asm volatile("" ::: "memory");
    for (int i0 = 0; i0 < NG; i0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u;
        if (i >= NG) break;
        const int j = i >> 1;
        if (u == 0) {
          // stage j landed: its copies are followed by at least one batch
          // (batch 0 in the prologue, batch i - 1 after), so waiting until
          // at most one batch is in flight covers them.  Then the copies of
          // stage j + 1 into the slot stage j - 1 freed.
          wait_vmcnt<kBatch>();
          asm volatile("" ::: "memory");
          if (j + 1 < NS) copy_stage((j + 1) & 1, j + 1);
          asm volatile("" ::: "memory");
        }
        if (i + 1 < NG) load_batch(u ^ 1, i + 1);
        asm volatile("" ::: "memory");
        if (u == 1)
          compute(1, my + (j & 1) * kRingStage, Ic<1>{});
        else
          compute(0, my + (j & 1) * kRingStage, Ic<0>{});
      }
    }
  }

  // sum the waves' tiles in a fixed order (the ring is free once every copy
  // of this block has landed)
  wait_vmcnt<0>();
  __syncthreads();
  constexpr int V = MT * 4;   // values per lane
  float* red = reinterpret_cast<float*>(ring);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * V + mt * 4 + i) * 64 + lane] = acc[mt][i];
  __syncthreads();
  for (int e = threadIdx.x; e < V * 64; e += W * 64) {
    float sum = red[e];
    for (int w = 1; w < W; ++w) sum += red[w * V * 64 + e];
    const int v = e >> 6, l = e & 63;
    const int n = n0 + (l & 15);
    const int m = 16 * (v >> 2) + 4 * (l >> 4) + (v & 3);
    if (n < N && m < M) Y[(int64_t)m * ldy + n] = f32_to_bf16_rne(sum);
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
  // more batches would spill: from M = 3, and at M = 2 with 8-bit codes
  constexpr int kMaxNB = M >= 3 ? 1 : ((W8 && M == 2) ? 3 : 8);
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
  hipLaunchKernelGGL((gemv_quad_kernel<M, T, NB, false>), dim3((unsigned)((N + 4 * NB - 1) / (4 * NB))),
                     dim3(S * kWave), 0, stream, X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy, 1,
                     nullptr);
}

template <int M, int T>
void launch_quad_t(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes,
                   const uint16_t* scales, const int32_t* zeros, int N, int K, int lg, uint16_t* Y,
                   int64_t ldy, hipStream_t stream) {
  // Rows per block: 4 x NB.  The largest NB whose block count fills the CUs
  // evenly, from 16 batches (8 with two slices per wave; 4 with two slices
  // of eight activation rows, whose registers are full).  Few long blocks
  // stream best: the gate_up shape (28672 rows) runs 512 blocks of 14
  // batches at 0.83-0.89 of the time of 1024 blocks of 7.  Fitted to timings
  // of the decode layers of the 8B- and 70B-shaped sets and the 40-layer
  // stack at M = 4, 5 and 8.
  constexpr int kMaxNB = T > 1 ? (M > 4 ? 4 : 8) : 16;
  constexpr int kNBs[] = {16, 14, 12, 10, 8, 7, 6, 5, 4, 3, 2, 1};
  const int cus = cu_count();
  auto balance = [&](int nb) {
    const double per_cu = (double)((N + 4 * nb - 1) / (4 * nb)) / cus;
    return per_cu / std::ceil(per_cu);
  };
  int nb = 0;
  for (int c : kNBs)
    if (nb == 0 && c <= kMaxNB && balance(c) >= 0.95) nb = c;
  if (nb == 0) {
    nb = 1;
    for (int c : kNBs)
      if (c <= kMaxNB && balance(c) > balance(nb) + 1e-9) nb = c;
  }
  switch (nb) {
#define W4A16_QUAD(V)                                                                     \
  case V:                                                                                 \
    launch_quad_nb<M, T, (V <= kMaxNB ? V : kMaxNB)>(X, Mrt, ldx, codes, scales, zeros, N, K, lg, Y, ldy, stream); \
    break;
    W4A16_QUAD(16) W4A16_QUAD(14) W4A16_QUAD(12) W4A16_QUAD(10) W4A16_QUAD(8) W4A16_QUAD(7)
    W4A16_QUAD(6) W4A16_QUAD(5) W4A16_QUAD(4) W4A16_QUAD(3) W4A16_QUAD(2)
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

// K split over KS blocks through a caller's workspace, 3 <= M <= 8: rows
// longer than 8192 inputs.  KS = 2 or 4 runs with one
// 512-input slice per wave (at most 16 waves; a run's last slice may be
// partial, its idle lanes weigh zero), else two runs of two slices; then
// the largest NB (up to 16 with one slice per wave: few long blocks stream
// best) whose block count fills the CUs evenly.  Measured on the down
// projections at M = 8: 8B (K = 14336) 16.1 -> 14.0 us, 70B (K = 28672)
// 56.9 -> 46.9 -> 39.3 us (16 batches), the stack's (K = 27648, four runs of
// 13.5 slices, 10 batches) 54.6 -> 39.9 -> 29.3 us; at M = 4 the stack's
// 25.6 -> 23.1 us against the long-row kernel (the 70B shape's even).
constexpr int kQuadSplitMinNB2 = 4, kQuadSplitMaxNB2 = 5;

struct QuadSplitPlan {
  int KS, T, NB, ranges;
  int64_t ws_bytes;
};

template <int MT>
bool quad_split_plan(int64_t N, int64_t K, QuadSplitPlan& p) {
  if (K <= 8192) return false;
  p.KS = 0;
  for (int t = 1; t <= 2 && p.KS == 0; ++t)
    for (int ks : {2, 4})
      if (p.KS == 0 && K % ((int64_t)32 * ks) == 0 &&
          (K / ks + kQuadSlice - 1) / kQuadSlice <= (int64_t)kQuadMaxWaves * t) {
        p.KS = ks;
        p.T = t;
      }
  if (p.KS == 0) return false;
  const int cus = cu_count();
  auto ranges = [&](int nb) { return (int)((N + 4 * nb - 1) / (4 * nb)); };
  auto balance = [&](int nb) {
    const double per_cu = (double)ranges(nb) * p.KS / cus;
    return per_cu / std::ceil(per_cu);
  };
  constexpr int kNBs[] = {16, 14, 12, 10, 8, 6, 5, 4, 3, 2};
  // two slices per wave: at most 8 batches; of eight activation rows: 4 or
  // 5 (other counts spill)
  const bool full = MT > 4 && p.T > 1;
  auto allowed = [&](int c) {
    return (!full || (c >= kQuadSplitMinNB2 && c <= kQuadSplitMaxNB2)) && (p.T == 1 || c <= 8) &&
           ranges(c) <= kSplitMaxRanges;
  };
  p.NB = 0;
  for (int c : kNBs)
    if (p.NB == 0 && allowed(c) && balance(c) >= 0.95) p.NB = c;
  if (p.NB == 0)
    for (int c : kNBs)
      if (allowed(c) && (p.NB == 0 || balance(c) > balance(p.NB) + 1e-9)) p.NB = c;
  if (p.NB == 0) return false;
  p.ranges = ranges(p.NB);
  p.ws_bytes = (int64_t)kSplitMaxRanges * kSplitCounterBytes + (int64_t)p.ranges * p.KS * p.NB * 4 * MT * 4;
  return true;
}

template <int MT, int T, int NB>
void launch_quad_split_nb(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes, const uint16_t* scales,
                          const int32_t* zeros, int N, int K, uint16_t* Y, int64_t ldy, const QuadSplitPlan& p,
                          void* workspace, hipStream_t stream) {
  const int S = ((K / p.KS + kQuadSlice - 1) / kQuadSlice + T - 1) / T;
  hipLaunchKernelGGL((gemv_quad_kernel<MT, T, NB, true>), dim3((unsigned)(p.ranges * p.KS)), dim3(S * kWave), 0,
                     stream, X, Mrt, ldx, codes, scales, zeros, N, K, 7, Y, ldy, p.KS,
                     reinterpret_cast<unsigned*>(workspace));
}

template <int MT>
void launch_quad_split(const uint16_t* X, int Mrt, int64_t ldx, const uint32_t* codes, const uint16_t* scales,
                       const int32_t* zeros, int N, int K, uint16_t* Y, int64_t ldy, const QuadSplitPlan& p,
                       void* workspace, hipStream_t stream) {
#define W4A16_QS(TV, V)                                                                                  \
  if constexpr (!(MT > 4 && TV > 1 && (V > kQuadSplitMaxNB2 || V < kQuadSplitMinNB2)))                  \
    if (p.T == TV && p.NB == V) {                                                                        \
      launch_quad_split_nb<MT, TV, V>(X, Mrt, ldx, codes, scales, zeros, N, K, Y, ldy, p, workspace, stream); \
      return;                                                                                            \
    }
  W4A16_QS(1, 16) W4A16_QS(1, 14) W4A16_QS(1, 12) W4A16_QS(1, 10)
  W4A16_QS(1, 8) W4A16_QS(1, 6) W4A16_QS(1, 5) W4A16_QS(1, 4) W4A16_QS(1, 3) W4A16_QS(1, 2)
  W4A16_QS(2, 8) W4A16_QS(2, 6) W4A16_QS(2, 5) W4A16_QS(2, 4) W4A16_QS(2, 3) W4A16_QS(2, 2)
#undef W4A16_QS
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
                int64_t, int64_t, int, uint16_t*, int64_t, hipStream_t, void* = nullptr, int64_t = 0);

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

// ---------------------------------------------------------------------------
// gemv_walk / gemv_ring launches
// ---------------------------------------------------------------------------

namespace {

// The walk's plan for a shape: KS runs of K (the fewest with at most 32
// groups each), row ranges (one block per CU, more when a range's scales
// would not fit the block's table), tiles per range.  Returns false when
// the walk does not apply (KS > 1 without room for the split).
struct WalkPlan {
  int KS, nranges, tiles, tmax;
  int64_t ws_bytes;   // workspace the split needs (0 for KS = 1)
};

bool walk_plan(int64_t N, int64_t K, WalkPlan& p) {
  const int G = (int)(K / kGroup);
  p.KS = (G + kWalkGroups - 1) / kWalkGroups;
  const int GB = (G + p.KS - 1) / p.KS;
  p.tiles = (int)((N + 15) / 16);
  const int tcap = kWalkMetaMax / (16 * GB);   // tiles whose scales fit the table (>= 8)
  p.nranges = max(1, min(p.tiles, device_cu_count() / p.KS));
  p.nranges = max(p.nranges, (p.tiles + tcap - 1) / tcap);
  p.tmax = (p.tiles + p.nranges - 1) / p.nranges;
  if (p.KS > 1 && p.nranges > kWalkMaxRanges) return false;
  if ((int64_t)p.nranges * p.KS >= ((int64_t)1 << 31)) return false;
  p.ws_bytes = p.KS == 1 ? 0
                         : (int64_t)kWalkMaxRanges * kWalkCounterBytes +
                               (int64_t)p.nranges * p.KS * (16 * p.tmax * 32) * 4;
  return true;
}

template <int MT>
int launch_walk(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes, const uint16_t* scales,
                const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y, int64_t ldy, const WalkPlan& p,
                void* workspace, hipStream_t stream) {
  static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_walk_kernel<MT>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               160 * 1024) == hipSuccess;
  if (!attr) return 4;
  hipLaunchKernelGGL(gemv_walk_kernel<MT>, dim3((unsigned)(p.nranges * p.KS)), dim3(1024),
                     walk_lds_bytes(MT, p.tmax), stream, X, (int)M, ldx, codes, scales, zeros, (int)N,
                     (int)K, Y, ldy, p.tiles, p.tmax, p.KS, reinterpret_cast<unsigned*>(workspace));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

template <int MT>
int launch_ring(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes, const uint16_t* scales,
                const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y, int64_t ldy, hipStream_t stream) {
  hipLaunchKernelGGL(gemv_ring_kernel<MT>, dim3((unsigned)((N + 15) / 16)), dim3(kRingWaves * 64), 0,
                     stream, X, (int)M, ldx, codes, scales, zeros, (int)N, (int)K, Y, ldy);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// M <= 32 on the matrix cores (groups of 128): the walk when it applies
// (with a workspace of at least its ws_bytes when it splits K), the ring
// otherwise.  Rows past 16 (32) of M take the second activation tile.
int launch_gemv_mt(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                   const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                   int64_t ldy, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  WalkPlan p;
  if (walk_plan(N, K, p) && (p.KS == 1 || (workspace != nullptr && workspace_bytes >= p.ws_bytes))) {
    return M <= 16 ? launch_walk<1>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, p, workspace, stream)
                   : launch_walk<2>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, p, workspace, stream);
  }
  return M <= 16 ? launch_ring<1>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream)
                 : launch_ring<2>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream);
}

}  // namespace

// Workspace that lets launch_gemv split K for this shape (0: none needed).
int64_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int group) {
  if (group != kGroup || M <= 2) return 0;
  if (M <= 8) {
    QuadSplitPlan q;
    return (M <= 4 ? quad_split_plan<4>(N, K, q) : quad_split_plan<8>(N, K, q)) ? q.ws_bytes : 0;
  }
  WalkPlan p;
  return walk_plan(N, K, p) ? p.ws_bytes : 0;
}

// group: 32, 64 or 128 inputs per quantisation group (checked by the caller).
// workspace (may be null): zero-filled device memory of workspace_bytes,
// left zero-filled; with at least gemv_workspace_bytes() the decode kernels
// for 3 <= M <= 32 may split K over blocks.
int launch_gemv(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t ldy, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (group != kGroup)
    return launch_gemv_small_groups(X, M, ldx, codes, scales, zeros, N, K, group == 32 ? 5 : 6, Y,
                                    ldy, stream);
  constexpr int lg = 7;
  if (M >= 3 && M <= 8 && workspace != nullptr) {
    QuadSplitPlan q;
    const bool plan = M <= 4 ? quad_split_plan<4>(N, K, q) : quad_split_plan<8>(N, K, q);
    if (plan && workspace_bytes >= q.ws_bytes) {
      if (M <= 4)
        launch_quad_split<4>(X, (int)M, ldx, codes, scales, zeros, (int)N, (int)K, Y, ldy, q, workspace, stream);
      else
        launch_quad_split<8>(X, (int)M, ldx, codes, scales, zeros, (int)N, (int)K, Y, ldy, q, workspace, stream);
      return hipGetLastError() == hipSuccess ? 0 : 4;
    }
  }
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
  return launch_gemv_mt(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, workspace, workspace_bytes, stream);
}

}  // namespace w4a16
