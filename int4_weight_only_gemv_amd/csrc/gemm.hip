// Prefill-shaped fused W4A16 matmul on the BF16 matrix cores (gfx950).
//
// Same arithmetic as the decode kernels (Axe Corsa model card, "The
// Two-Stage Pipeline": dequantise inside the multiply): per group of 128
// inputs the codes become exact BF16 operands 128 + q, the matrix cores
// produce
//   P[m,n]  = sum_{k in g} X[m,k] (128 + q[n,k])   and
//   Xs[m]   = sum_{k in g} X[m,k]                  (A against a B of ones),
// and the group is folded into the float32 accumulator with
//   acc += s[n,g] * (P - (128 + z[n,g]) * Xs).
// No weight is rounded to BF16, so the only rounding beyond float32
// accumulation is the final BF16 store.
//
// Tiling: a 512-thread block (8 waves, 4 along M x 2 along N) computes a
// 256 x 128 tile of Y; each wave owns 64 x 64 (4 x 4 MFMA 16x16x32 tiles).
// A K step is half a group (64 inputs).  X[256][64] and the codes
// [128][8 words] of a step go straight from global memory to LDS
// (global_load_lds_dwordx4, no register staging) into one of three LDS
// stages, two steps ahead of the matrix cores, with one barrier per step.
// X rows are stored with their 16-byte chunks XOR-swizzled by row so the
// A-fragment reads spread over the LDS banks.  Codes are unpacked in natural
// k order, so X needs no permutation.  Tiles are handed to the 8 XCDs in
// contiguous runs with N fastest, so blocks that share X rows share an L2.

#include "common.h"

namespace w4a16 {
namespace {

constexpr int BM = 256;
constexpr int BN = 128;
constexpr int KS = 64;                 // inputs per K step (half a group)
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kStages = 3;
constexpr int X_STAGE = BM * KS * 2;   // bytes of X per stage (32 KiB)
constexpr int C_STAGE = BN * KS / 2;   // bytes of codes per stage (4 KiB)
constexpr int X_LOADS = X_STAGE / 1024 / kWaves;  // 1-KiB wave loads of X per wave per step (4)
constexpr int C_WAVES = C_STAGE / 1024;           // waves that also load one KiB of codes (4)
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void;

template <int V>
struct StageIdx {
  static constexpr int value = V;
};
static_assert(kStages == 3, "the main loop is unrolled over three stages");

// Eight codes of one word -> BF16 operands 128 + q in natural k order:
// dword j holds (code 2j, code 2j+1).
__device__ __forceinline__ u32x4 codes_to_bias128_natural(uint32_t w) {
  const uint32_t even = w & 0x0F0F0F0Fu;          // bytes q0 q2 q4 q6
  const uint32_t odd = (w >> 4) & 0x0F0F0F0Fu;    // bytes q1 q3 q5 q7
  const uint32_t lo = __builtin_amdgcn_perm(odd, even, 0x05010400u);  // q0 q1 q2 q3
  const uint32_t hi = __builtin_amdgcn_perm(odd, even, 0x07030602u);  // q4 q5 q6 q7
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(kExpBytes, lo, 0x04010400u);  // (q0, q1)
  r[1] = __builtin_amdgcn_perm(kExpBytes, lo, 0x04030402u);  // (q2, q3)
  r[2] = __builtin_amdgcn_perm(kExpBytes, hi, 0x04010400u);  // (q4, q5)
  r[3] = __builtin_amdgcn_perm(kExpBytes, hi, 0x04030402u);  // (q6, q7)
  return r;
}

// Wait until at most n vector-memory operations of this wave are in flight.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  // one LDS object per stage, so the compiler can tell the copies into one
  // stage from the reads of another and never waits for unrelated copies
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[X_STAGE], xs1[X_STAGE], xs2[X_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t cs0[C_STAGE], cs1[C_STAGE], cs2[C_STAGE];

  // XCD-aware tile order: consecutive block ids land on different XCDs, so
  // give XCD x the contiguous run of tiles [x T/8, (x+1) T/8), N fastest.
  const int T = m_tiles * n_tiles;
  int t = blockIdx.x;
  if (T % kXcds == 0) t = (t % kXcds) * (T / kXcds) + t / kXcds;
  const int m0 = (t / n_tiles) * BM;
  const int n0 = (t % n_tiles) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int G = K / kGroup;
  const int steps = 2 * G;
  const int64_t words_per_row = K / 8;

  // ---- direct-to-LDS copies.  X: wave load j of wave w fills tile rows
  // 8 (X_LOADS w + j) .. +7; lane -> row + lane/8, LDS chunk slot lane%8,
  // which holds global chunk slot ^ (row & 7).
  const uint16_t* xsrc[X_LOADS];
  int xoff[X_LOADS];
#pragma unroll
  for (int j = 0; j < X_LOADS; ++j) {
    const int row = 8 * (X_LOADS * wave + j) + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    xsrc[j] = X + (int64_t)min(m0 + row, M - 1) * ldx + chunk * 8;
    xoff[j] = 8 * (X_LOADS * wave + j) * (KS * 2);
  }
  // codes: wave w < C_WAVES fills code rows 32 w .. +31 (32 B each)
  const uint32_t* csrc = codes + (int64_t)min(n0 + 32 * wave + (lane >> 1), N - 1) * words_per_row +
                         (lane & 1) * 4;
  const int coff = 32 * wave * (KS / 2);
  auto issue = [&](int s, uint8_t* xdst, uint8_t* cdst) {
#pragma unroll
    for (int j = 0; j < X_LOADS; ++j)
      __builtin_amdgcn_global_load_lds(xsrc[j] + s * KS, (lds_void*)&xdst[xoff[j]], 16, 0, 0);
    if (wave < C_WAVES)
      __builtin_amdgcn_global_load_lds(csrc + s * (KS / 8), (lds_void*)&cdst[coff], 16, 0, 0);
  };

  // this lane's output columns (one per 16-wide n tile) for scales / zeros
  const int ncol0 = n0 + wn * 64 + r16;
  int64_t meta[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) meta[nt] = (int64_t)min(ncol0 + nt * 16, N - 1) * G;
  uint32_t sraw[4];
  int zraw[4];
  auto fetch_meta = [&](int g) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sraw[nt] = scales[meta[nt] + g];
      zraw[nt] = zeros[meta[nt] + g];
    }
  };

  // LDS read addresses: A row (wm 64 + mt 16 + r16), logical chunk 2q + kc
  // (inputs 16q + 8kc .. +7 of the step); B row (wn 64 + nt 16 + r16),
  // words 2q, 2q + 1.
  int aoff[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = wm * 64 + mt * 16 + r16;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) aoff[mt][kc] = row * (KS * 2) + (((2 * q + kc) ^ (row & 7)) * 16);
  }
  int boff[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) boff[nt] = (wn * 64 + nt * 16 + r16) * (KS / 2) + q * 8;

  f32x4 acc[4][4], pg[4][4], xsum[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    xsum[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      pg[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};

  fetch_meta(0);
  issue(0, xs0, cs0);
  if (steps > 1) issue(1, xs1, cs1);

  // one K step on LDS stage ST (= s mod 3); copies for step s + 2 go to
  // stage (ST + 2) mod 3, which every wave finished reading at step s - 1
  auto step = [&](auto stage, int s) {
    constexpr int ST = decltype(stage)::value;
    uint8_t* xs = ST == 0 ? xs0 : (ST == 1 ? xs1 : xs2);
    uint8_t* cs = ST == 0 ? cs0 : (ST == 1 ? cs1 : cs2);
    uint8_t* xn = ST == 0 ? xs2 : (ST == 1 ? xs0 : xs1);
    uint8_t* cn = ST == 0 ? cs2 : (ST == 1 ? cs0 : cs1);
    // step s landed in LDS once only the next step's copies are in flight
    if (s + 1 < steps) {
      if (wave < C_WAVES) wait_vmcnt<X_LOADS + 1>(); else wait_vmcnt<X_LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    // scale/zero of this step's group, fetched before the next copies so the
    // in-order vmcnt waits above never wait on the copies just issued
    if (s > 0 && !(s & 1)) fetch_meta(s / 2);
    if (s + 2 < steps) issue(s + 2, xn, cn);

    u32x2 bw[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bw[nt] = *reinterpret_cast<const u32x2*>(&cs[boff[nt]]);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      u32x4 af[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) af[mt] = *reinterpret_cast<const u32x4*>(&xs[aoff[mt][kc]]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const u32x4 b = codes_to_bias128_natural(bw[nt][kc]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) pg[mt][nt] = mfma16x16x32(af[mt], b, pg[mt][nt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) xsum[mt] = mfma16x16x32(af[mt], ones, xsum[mt]);
    }

    if (s & 1) {  // group complete: fold it into the accumulator
      float sc[4], zb[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        sc[nt] = bf16_to_f32(sraw[nt]);
        zb[nt] = (float)(128 + zraw[nt]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float d = fmaf(-zb[nt], xsum[mt][r], pg[mt][nt][r]);
            acc[mt][nt][r] = fmaf(sc[nt], d, acc[mt][nt][r]);
          }
          pg[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        xsum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  for (int s0 = 0; s0 < steps; s0 += kStages) {
    step(StageIdx<0>{}, s0);
    if (s0 + 1 < steps) step(StageIdx<1>{}, s0 + 1);
    if (s0 + 2 < steps) step(StageIdx<2>{}, s0 + 2);
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
  const int64_t mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  if (mt * nt >= ((int64_t)1 << 31)) return 3;
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)(mt * nt)), dim3(kThreads), 0, stream, X, (int)M,
                     ldx, codes, scales, zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
