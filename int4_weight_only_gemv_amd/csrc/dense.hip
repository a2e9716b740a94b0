// Dense BF16 comparisons for the fused W4A16 path (gfx950).
//
// Zeno AGI, "Weight-only vs mixed precision": its table of offline versus
// fused dequantisation and "7. The Marlin Kernel" (the naive three-kernel
// pipeline) describe the alternatives to dequantising inside the multiply,
// and "1. The Basic Recipe" the dense BF16 layer the INT4 path replaces.
// These kernels put numbers on them at the same shapes:
//   * dequant_bf16_kernel: the offline expansion of packed weights to dense
//     BF16 (also the middle kernel of the naive pipeline);
//   * dense_gemv_kernel: a dense BF16 linear layer at decode sizes, VALU dot
//     products streaming BF16 weights (HBM-bound like the fused decode);
//   * dense_gemm_kernel: a dense BF16 linear layer at prefill sizes on the
//     matrix cores, the fused GEMM's tiling without the INT4 work.

#include "common.h"

namespace w4a16 {
namespace {

// ---------------------------------------------------------------------------
// Offline expansion: w = BF16_RNE(fl32(fl32(q - z) * s)), one thread per code
// word (eight weights, one 16-byte store)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void dequant_bf16_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const int32_t* __restrict__ zeros, int64_t N, int64_t K, uint16_t* __restrict__ W,
    int64_t ldw) {
  const int64_t words = K / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N * words) return;
  const int64_t n = t / words, w = t - n * words;
  const int64_t G = K / kGroup, gi = n * G + w / (kGroup / 8);
  const uint32_t word = codes[t];
  const float s = bf16_to_f32(scales[gi]);
  const int z = zeros[gi];
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q0 = (int)((word >> (8 * i)) & 15u), q1 = (int)((word >> (8 * i + 4)) & 15u);
    const uint32_t lo = f32_to_bf16_rne(__fmul_rn((float)(q0 - z), s));
    const uint32_t hi = f32_to_bf16_rne(__fmul_rn((float)(q1 - z), s));
    out[i] = lo | (hi << 16);
  }
  *reinterpret_cast<u32x4*>(W + n * ldw + 8 * w) = out;
}

// ---------------------------------------------------------------------------
// Dense decode: Y[m, n] = sum_k X[m, k] W[n, k], M <= kDenseMaxM
// ---------------------------------------------------------------------------
//
// A block of 4 waves owns R consecutive rows of W; the waves split K in
// 512-input chunks (wave w takes chunks w, w + 4, ...).  Per chunk a lane
// holds 8 inputs: the activations once, then 16 bytes of each of the R rows,
// all R loads issued before the products (R x 1 KiB in flight per wave);
// v_dot2_f32_bf16 multiplies BF16 pairs exactly and accumulates in fp32.
// Partial sums reduce across the lanes (butterfly) and the waves (LDS, fixed
// order).

constexpr int kDenseWaves = 4;
constexpr int kDenseChunk = 8 * kWave;  // inputs per wave per chunk

template <int M, int R>
__global__ __launch_bounds__(kDenseWaves * 64) void dense_gemv_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const uint16_t* __restrict__ W, int64_t ldw,
    int N, int K, uint16_t* __restrict__ Y, int64_t ldy) {
  __shared__ float red[kDenseWaves][R * M];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int row0 = (int)blockIdx.x * R;
  const u32x4* wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wrow[r] = reinterpret_cast<const u32x4*>(W + (int64_t)min(row0 + r, N - 1) * ldw);
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  const int nchunks = (K + kDenseChunk - 1) / kDenseChunk;
  for (int c = wave; c < nchunks; c += kDenseWaves) {
    const int k = c * kDenseChunk + 8 * lane;
    if (k < K) {
      u32x4 wv[R], xv[M];
#pragma unroll
      for (int r = 0; r < R; ++r) wv[r] = __builtin_nontemporal_load(wrow[r] + k / 8);
#pragma unroll
      for (int m = 0; m < M; ++m) xv[m] = *reinterpret_cast<const u32x4*>(X + (int64_t)m * ldx + k);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][m] = dot2(wv[r][j], xv[m][j], acc[r][m]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int mask = 32; mask >= 1; mask >>= 1) v += __shfl_xor(v, mask);
      acc[r][m] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][r * M + m] = acc[r][m];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * M; i += blockDim.x) {
    const int r = i / M, m = i - r * M;
    if (row0 + r >= N) continue;
    float v = red[0][i];
#pragma unroll
    for (int w = 1; w < kDenseWaves; ++w) v += red[w][i];
    Y[(int64_t)m * ldy + row0 + r] = f32_to_bf16_rne(v);
  }
}

// ---------------------------------------------------------------------------
// Dense prefill on the matrix cores: the fused GEMM's 256 x 256 block tile
// (8 waves of 128 x 64, 16x16x32 BF16 tiles), both operands BF16 rows of 32
// inputs per K step moved global -> LDS (global_load_lds_dwordx4) into four
// stages, four steps ahead, one barrier per step, 16-byte chunks swizzled by
// (row >> 1) & 3.
// ---------------------------------------------------------------------------

constexpr int BM = 256, BN = 256, WM = 128, WN = 64, MT = WM / 16, NT = WN / 16;
constexpr int KS = 32;
constexpr int kGemmThreads = 512;
constexpr int STAGE = BM * KS * 2;                        // bytes per operand per stage
constexpr int LOADS = STAGE / 1024 / (kGemmThreads / 64); // 1-KiB copies per wave per operand
constexpr int kXcds = 8;
static_assert(LOADS == 2, "copy split");

__global__ __launch_bounds__(kGemmThreads) void dense_gemm_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint16_t* __restrict__ W,
    int64_t ldw, int N, int K, uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE], xs1[STAGE], xs2[STAGE], xs3[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ws0[STAGE], ws1[STAGE], ws2[STAGE], ws3[STAGE];

  const int T = m_tiles * n_tiles;
  int t = blockIdx.x;
  if (T % kXcds == 0) t = (t % kXcds) * (T / kXcds) + t / kXcds;
  const int m0 = (t / n_tiles) * BM;
  const int n0 = (t % n_tiles) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int steps = K / KS;

  // copies: lane -> row lane / 4, 16-byte slot lane % 4 holding the row's
  // chunk slot ^ ((row >> 1) & 3); copy j of wave w fills rows 16 (2w + j)..
  // Rows past M (N) read the last row and are never stored.
  const uint32_t swz = (uint32_t)(((lane & 3) ^ ((lane >> 3) & 3)) * 16);
  const char* xblk = reinterpret_cast<const char*>(X + (int64_t)m0 * ldx);
  const char* wblk = reinterpret_cast<const char*>(W + (int64_t)n0 * ldw);
  uint32_t xoffs[LOADS], woffs[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int r = 16 * (LOADS * wave + j) + (lane >> 2);
    xoffs[j] = (uint32_t)(min(m0 + r, M - 1) - m0) * (uint32_t)(ldx * 2) + swz;
    woffs[j] = (uint32_t)(min(n0 + r, N - 1) - n0) * (uint32_t)(ldw * 2) + swz;
  }
  const int dst0 = 16 * LOADS * wave * (KS * 2);
  auto copy = [&](uint8_t* xd, uint8_t* wd, int s) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      __builtin_amdgcn_global_load_lds(xblk + (xoffs[j] + (uint32_t)(s * KS * 2)),
                                       (lds_void*)&xd[dst0 + j * 16 * (KS * 2)], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(wblk + (woffs[j] + (uint32_t)(s * KS * 2)),
                                       (lds_void*)&wd[dst0 + j * 16 * (KS * 2)], 16, 0, 0);
    }
  };

  // fragments: A row tile mt = X rows wm 128 + 16 mt + r16, B column tile nt =
  // W rows wn 64 + 16 nt + r16; chunk q of the step (inputs 8q .. 8q+7)
  const int arow = wm * WM + r16, brow = wn * WN + r16;
  const int aoff = arow * (KS * 2) + ((q ^ ((arow >> 1) & 3)) * 16);
  const int boff = brow * (KS * 2) + ((q ^ ((brow >> 1) & 3)) * 16);
  u32x4 af[MT], bf[NT];
  auto read_b = [&](const uint8_t* ws) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bf[nt] = *reinterpret_cast<const u32x4*>(&ws[boff + nt * 16 * (KS * 2)]);
  };
  auto read_a = [&](const uint8_t* xs, int mt) {
    af[mt] = *reinterpret_cast<const u32x4*>(&xs[aoff + mt * 16 * (KS * 2)]);
  };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: steps 0..3 in flight, step 0's fragments in registers
  copy(xs0, ws0, 0);
  copy(xs1, ws1, min(1, steps - 1));
  copy(xs2, ws2, min(2, steps - 1));
  copy(xs3, ws3, min(3, steps - 1));
  wait_vmcnt<3 * 2 * LOADS>();
  block_barrier();
  read_b(ws0);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) read_a(xs0, mt);

  // One K step at position ST of a period of four (operands in stage ST,
  // fragments already in registers).  After the barrier stage ST is free, so
  // it takes step s + 4; the fragments of step s + 1 are read while the
  // matrix cores work: B into fresh registers, each A row tile after its
  // products.
  auto step = [&](auto stage, int s) {
    constexpr int ST = decltype(stage)::value;
    uint8_t* xs_here = ST == 0 ? xs0 : (ST == 1 ? xs1 : (ST == 2 ? xs2 : xs3));
    uint8_t* ws_here = ST == 0 ? ws0 : (ST == 1 ? ws1 : (ST == 2 ? ws2 : ws3));
    uint8_t* xs_next = ST == 0 ? xs1 : (ST == 1 ? xs2 : (ST == 2 ? xs3 : xs0));
    uint8_t* ws_next = ST == 0 ? ws1 : (ST == 1 ? ws2 : (ST == 2 ? ws3 : ws0));
    wait_vmcnt<2 * 2 * LOADS>();   // step s + 1 landed, every read of stage ST done
    block_barrier();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(af[mt]));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(bf[nt]));
    copy(xs_here, ws_here, min(s + 4, steps - 1));
    u32x4 b[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) b[nt] = bf[nt];
    read_b(ws_next);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 a = af[mt];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x32(a, b[nt], acc[mt][nt]);
      read_a(xs_next, mt);
    }
  };
  int s = 0;
  for (; s + 4 <= steps; s += 4) {
    step(Ic<0>{}, s);
    step(Ic<1>{}, s + 1);
    step(Ic<2>{}, s + 2);
    step(Ic<3>{}, s + 3);
  }
  // K = 128 k': steps is a multiple of four
  wait_vmcnt<0>();

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + wn * WN + nt * 16 + r16;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * WM + mt * 16 + 4 * q + r;
        if (m < M) Y[(int64_t)m * ldy + n] = f32_to_bf16_rne(acc[mt][nt][r]);
      }
    }
}

template <int M>
void launch_dense_gemv_m(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw, int N,
                         int K, uint16_t* Y, int64_t ldy, hipStream_t stream) {
  constexpr int R = M <= 2 ? 8 : 4;
  hipLaunchKernelGGL((dense_gemv_kernel<M, R>), dim3((unsigned)((N + R - 1) / R)),
                     dim3(kDenseWaves * kWave), 0, stream, X, ldx, W, ldw, N, K, Y, ldy);
}

}  // namespace

int launch_dequant_bf16(const uint32_t* codes, const uint16_t* scales, const int32_t* zeros,
                        int64_t N, int64_t K, uint16_t* W, int64_t ldw, hipStream_t stream) {
  const int64_t threads = N * (K / 8);
  hipLaunchKernelGGL(dequant_bf16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, codes, scales, zeros, N, K, W, ldw);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int launch_dense_gemv(const uint16_t* X, int64_t M, int64_t ldx, const uint16_t* W, int64_t ldw,
                      int64_t N, int64_t K, uint16_t* Y, int64_t ldy, hipStream_t stream) {
  const int n = (int)N, k = (int)K;
  switch (M) {
    case 1: launch_dense_gemv_m<1>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
    case 2: launch_dense_gemv_m<2>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
    case 3: launch_dense_gemv_m<3>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
    case 4: launch_dense_gemv_m<4>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
    case 5: launch_dense_gemv_m<5>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
    case 6: launch_dense_gemv_m<6>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
    case 7: launch_dense_gemv_m<7>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
    default: launch_dense_gemv_m<8>(X, ldx, W, ldw, n, k, Y, ldy, stream); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int launch_dense_gemm(const uint16_t* X, int64_t M, int64_t ldx, const uint16_t* W, int64_t ldw,
                      int64_t N, int64_t K, uint16_t* Y, int64_t ldy, hipStream_t stream) {
  const int64_t mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  if (mt * nt >= ((int64_t)1 << 31)) return 3;
  // per-lane 32-bit byte offsets within a tile's rows
  if ((BM - 1) * ldx * 2 + K * 2 >= ((int64_t)1 << 32) || (BN - 1) * ldw * 2 + K * 2 >= ((int64_t)1 << 32))
    return 3;
  hipLaunchKernelGGL(dense_gemm_kernel, dim3((unsigned)(mt * nt)), dim3(kGemmThreads), 0, stream, X,
                     (int)M, ldx, W, ldw, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
