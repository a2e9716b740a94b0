// Decode-shaped fused W4A16 matmul, 1 <= M <= 32 (gfx950).
//
// Y[m, n] = sum_g s[n,g] * sum_{k in g} X[m,k] * (q[n,k] - z[n,g])
// (Axe Corsa model card, "The Two-Stage Pipeline": dequantisation fused
// into the multiply, weights rebuilt in registers).
//
// Per wave and per group of 128 inputs, a 16-row tile of W meets a 16-row
// (M padded) tile of X on the BF16 matrix cores, v_mfma_f32_16x16x32_bf16:
//   * the packed codes are the B operand, turned into the exact BF16 values
//     128 + q by OR-ing each nibble into the mantissa of 128.0 (two ops per
//     pair of codes, no conversion instructions);
//   * the same A operand against a B of ones gives sum_{k in g} X[m,k];
//   * per group, in float32:  acc += s * (P - (128 + z) * Xsum),
//     the bias and the zero point removed with one fused multiply-add whose
//     product is exact.  No weight is ever rounded.
//
// Work split: a block owns 16 output rows and all of K; its S waves split
// the K groups evenly and their partial sums are added in a fixed order
// through LDS, so results are deterministic and no workspace is needed.
// Each lane streams 16 contiguous bytes (32 codes of one row) per group.

#include "common.h"

namespace w4a16 {
namespace {

constexpr int kMaxWaves = 16;

template <int MT, int U>
__global__ __launch_bounds__(1024) void gemv_mfma_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy) {
  __shared__ float red[kMaxWaves][MT * 4][kWave];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int S = blockDim.x / kWave;
  const int G = K / kGroup;
  const int col = lane & 15;  // output row of the tile (MFMA column)
  const int kq = lane >> 4;   // 32-input quarter of the group this lane feeds

  const int n = blockIdx.x * 16 + col;
  const int n_ld = n < N ? n : N - 1;
  const int gb = (G * wave) / S;
  const int ge = (G * (wave + 1)) / S;

  const u32x4* crow = reinterpret_cast<const u32x4*>(codes + (int64_t)n_ld * (K / 8)) + kq;
  const uint16_t* srow = scales + (int64_t)n_ld * G;
  const int32_t* zrow = zeros + (int64_t)n_ld * G;

  // A-operand rows: m = (lane & 15) + 16 * mt.
  const u32x4* xrow[MT];
  bool xvalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = col + 16 * mt;
    xvalid[mt] = m < M;
    xrow[mt] = reinterpret_cast<const u32x4*>(X + (int64_t)(xvalid[mt] ? m : 0) * ldx) + kq * 4;
  }

  const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g0 = gb; g0 < ge; g0 += U) {
    u32x4 cw[U];
    u32x4 xr[U][4][MT];
    float sc[U];
    float zb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u;
      if (g < ge) {
        cw[u] = __builtin_nontemporal_load(crow + g * 4);
        sc[u] = bf16_to_f32(srow[g]);
        zb[u] = (float)(128 + zrow[g]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xr[u][i][mt] = xvalid[mt] ? xrow[mt][g * 16 + i] : u32x4{0u, 0u, 0u, 0u};
        }
      } else {
        cw[u] = u32x4{0u, 0u, 0u, 0u};
        sc[u] = 0.f;
        zb[u] = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xr[u][i][mt] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 pg[MT], xs[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        pg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        xs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 b = codes_to_bias128_pairs(cw[u][i]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4 a = x_pairs_from_natural(xr[u][i][mt]);
          pg[mt] = mfma16x16x32(a, b, pg[mt]);
          xs[mt] = mfma16x16x32(a, ones, xs[mt]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float d = fmaf(-zb[u], xs[mt][r], pg[mt][r]);
          acc[mt][r] = fmaf(sc[u], d, acc[mt][r]);
        }
    }
  }

  if (S > 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][mt * 4 + r][lane] = acc[mt][r];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = red[0][mt * 4 + r][lane];
        for (int w = 1; w < S; ++w) v += red[w][mt * 4 + r][lane];
        acc[mt][r] = v;
      }
  }
  if (n >= N) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * kq + r;
      if (m < M) Y[(int64_t)m * ldy + n] = f32_to_bf16_rne(acc[mt][r]);
    }
}

int pick_waves(int G) {
  int s = G / 4;
  if (s < 1) s = 1;
  if (s > kMaxWaves) s = kMaxWaves;
  return s;
}

}  // namespace

int launch_gemv(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                int64_t ldy, hipStream_t stream) {
  const int G = (int)(K / kGroup);
  const int S = pick_waves(G);
  const dim3 grid((unsigned)((N + 15) / 16));
  const dim3 block(S * kWave);
  if (M <= 16)
    hipLaunchKernelGGL((gemv_mfma_kernel<1, 4>), grid, block, 0, stream, X, (int)M, ldx, codes,
                       scales, zeros, (int)N, (int)K, Y, ldy);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<2, 2>), grid, block, 0, stream, X, (int)M, ldx, codes,
                       scales, zeros, (int)N, (int)K, Y, ldy);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
