// Prefill-shaped fused W4A16 matmul on the BF16 matrix cores (gfx950).
//
// Same arithmetic as the decode kernel (Axe Corsa model card, "The Two-Stage
// Pipeline": dequantise inside the multiply): per group of 128 inputs the
// codes become exact BF16 operands 128 + q, the matrix cores produce
//   P[m,n]  = sum_{k in g} X[m,k] (128 + q[n,k])   and
//   Xs[m]   = sum_{k in g} X[m,k]                  (A against a B of ones),
// and the group is folded into the float32 accumulator with
//   acc += s[n,g] * (P - (128 + z[n,g]) * Xs).
// No weight is rounded to BF16, so the only rounding beyond float32
// accumulation is the final BF16 store.
//
// Tiling: a 256-thread block computes a 128 x 128 tile of Y; its four waves
// own 64 x 64 quadrants (4 x 4 MFMA 16x16x32 tiles).  One K step is one
// group: the block stages X[128 rows][128] (pair-permuted to match the code
// unpack) and the codes [128 rows][16 words] in LDS, the next group's tiles
// are fetched into registers while the current one is multiplied.

#include "common.h"

namespace w4a16 {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int kThreads = 256;
constexpr int XS_STRIDE = 136;  // bf16 per LDS row of X (128 + 8 pad)
constexpr int CS_STRIDE = 20;   // dwords per LDS row of codes (16 + 4 pad)
constexpr int X_CHUNKS = BM * 16 / kThreads;  // 16-byte X chunks per thread per group (8)
constexpr int C_CHUNKS = BN * 4 / kThreads;   // 16-byte code chunks per thread per group (2)

__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint16_t xs_lds[BM * XS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint32_t cs_lds[BN * CS_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int G = K / kGroup;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int64_t words_per_row = K / 8;

  // ---- global -> register staging.  Thread tid moves 16-byte chunk
  // (tid & 15) of X rows (tid >> 4) + 16 i, and 16-byte chunk (tid & 3) of
  // code rows (tid >> 2) + 64 i.
  const int xrow0 = tid >> 4, xpart = tid & 15;
  const u32x4* xsrc = reinterpret_cast<const u32x4*>(X + (int64_t)(m0 + xrow0) * ldx) + xpart;
  const int64_t xstep = 16 * ldx / 8;  // 16 rows, in 16-byte units
  const int xdst = xrow0 * XS_STRIDE + xpart * 8;
  const int crow0 = tid >> 2, cpart = tid & 3;
  const int64_t cstep = (int64_t)64 * words_per_row / 4;
  const u32x4* csrc = reinterpret_cast<const u32x4*>(codes + (int64_t)(n0 + crow0) * words_per_row) + cpart;
  const int cdst = crow0 * CS_STRIDE + cpart * 4;
  // rows of the code tile past N are clamped to the last row
  int crow_ok = 0;
#pragma unroll
  for (int i = 0; i < C_CHUNKS; ++i) crow_ok |= (n0 + crow0 + 64 * i < N) << i;
  const u32x4* clast = reinterpret_cast<const u32x4*>(codes + (int64_t)(N - 1) * words_per_row) + cpart;
  // per-lane output columns (one per 16-wide n tile) for scales / zero points
  const int ncol0 = n0 + wn * 64 + r16;

  u32x4 xreg[X_CHUNKS];
  u32x4 creg[C_CHUNKS];
  auto fetch = [&](int g) {
#pragma unroll
    for (int i = 0; i < X_CHUNKS; ++i)
      xreg[i] = (m0 + xrow0 + 16 * i < M) ? xsrc[i * xstep + g * 16] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < C_CHUNKS; ++i)
      creg[i] = __builtin_nontemporal_load(((crow_ok >> i) & 1) ? csrc + i * cstep + g * 4 : clast + g * 4);
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < X_CHUNKS; ++i)
      *reinterpret_cast<u32x4*>(&xs_lds[xdst + 16 * i * XS_STRIDE]) = x_pairs_from_natural(xreg[i]);
#pragma unroll
    for (int i = 0; i < C_CHUNKS; ++i)
      *reinterpret_cast<u32x4*>(&cs_lds[cdst + 64 * i * CS_STRIDE]) = creg[i];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};

  fetch(0);
  stash();
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    float sc[4], zb[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t gi = (int64_t)min(ncol0 + nt * 16, N - 1) * G + g;
      sc[nt] = bf16_to_f32(scales[gi]);
      zb[nt] = (float)(128 + zeros[gi]);
    }
    if (g + 1 < G) fetch(g + 1);

    f32x4 pg[4][4], xsum[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      xsum[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 4; ++b) pg[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // B fragments: lane (column r16, quarter q) holds words 4q..4q+3 of its row.
    u32x4 bw[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bw[nt] = *reinterpret_cast<const u32x4*>(&cs_lds[(wn * 64 + nt * 16 + r16) * CS_STRIDE + 4 * q]);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      u32x4 af[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        af[mt] = *reinterpret_cast<const u32x4*>(
            &xs_lds[(wm * 64 + mt * 16 + r16) * XS_STRIDE + 32 * q + 8 * kc]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const u32x4 b = codes_to_bias128_pairs(bw[nt][kc]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) pg[mt][nt] = mfma16x16x32(af[mt], b, pg[mt][nt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) xsum[mt] = mfma16x16x32(af[mt], ones, xsum[mt]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float d = fmaf(-zb[nt], xsum[mt][r], pg[mt][nt][r]);
          acc[mt][nt][r] = fmaf(sc[nt], d, acc[mt][nt][r]);
        }
    if (g + 1 < G) {
      __syncthreads();
      stash();
      __syncthreads();
    }
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = n0 + wn * 64 + nt * 16 + r16;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + mt * 16 + 4 * q + r;
        if (m < M) Y[(int64_t)m * ldy + n] = f32_to_bf16_rne(acc[mt][nt][r]);
      }
    }
}

}  // namespace

int launch_gemm(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                int64_t ldy, hipStream_t stream) {
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (grid.y > 65535u) return 3;
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, stream, X, (int)M, ldx, codes, scales,
                     zeros, (int)N, (int)K, Y, ldy);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
