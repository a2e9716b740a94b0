// Prefill-shaped fused W4A16 matmul on the BF16 matrix cores (gfx950).
//
// Y[m,n] = sum_g s[n,g] * sum_{k in g} X[m,k] (q[n,k] - z[n,g])  (Axe Corsa
// model card, "The Two-Stage Pipeline": dequantise inside the multiply).
//
// Operands.  Codes become exact BF16 values 128 + q (each nibble placed in
// the mantissa of BF16 128.0), so no weight is ever rounded.  Per group the
// matrix cores add sum_k X (128 + q) into the accumulator; the same A
// operand against a B of ones gives Xs[m] = sum_{k in g} X[m,k].
//
// One accumulator, rescaled per group.  The accumulator T is kept in units
// of the current group's scale:
//     end of group g:  T <- (T - (128 + z[n,g]) Xs[m]) * s[n,g] / s[n,g+1]
// and after the last group the factor is s[n,G-1] itself, so T = Y.  The
// scale ratios come from the hardware reciprocal (1 ulp) and one float32
// multiply, a few 1e-7 relative each; the packer's scales are positive
// normal BF16 values.
//
// Tiling.  A 512-thread block (8 waves, 2 along M x 4 along N) computes a
// 256 x 256 tile of Y; each wave owns 128 x 64 (8 x 4 MFMA 16x16x32 tiles).
// The four waves that share 128 rows each compute the activation sums of two
// of the eight 16-row tiles and exchange them through LDS.  A K step is a
// quarter group (32 inputs).  X[256][32] and the codes [256][4 words] of a
// step go straight from global memory to LDS (global_load_lds_dwordx4) into
// one of four LDS stages, three steps ahead of the matrix cores, with one
// barrier per step.  X rows (64 bytes) are stored with their 16-byte chunks
// XOR-swizzled by (row >> 1) & 3, so the eight rows that one 128-byte LDS
// cycle of a 16-byte-per-lane read serves fall on eight distinct bank groups.
// Codes are unpacked in natural k order, so X needs no permutation.  Tiles go
// to the 8 XCDs in contiguous runs with N fastest, so blocks that share X rows
// share an L2.

#include "common.h"

namespace w4a16 {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int WM = 128, WN = 64;       // wave tile
constexpr int MT = WM / 16, NT = WN / 16;
constexpr int KS = 32;                 // inputs per K step (a quarter group)
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kStages = 4;
constexpr int X_STAGE = BM * KS * 2;   // bytes of X per stage (16 KiB)
constexpr int C_STAGE = BN * KS / 2;   // bytes of codes per stage (4 KiB)
constexpr int X_LOADS = X_STAGE / 1024 / kWaves;  // 1-KiB wave copies of X per wave per step
constexpr int kXcds = 8;
constexpr int XS_TILES = MT / 4;       // activation-sum tiles computed by each wave
constexpr int C_WAVES = C_STAGE / 1024;          // 1-KiB code copies per step (each made by two waves)
constexpr int kSteps = kGroup / KS;               // K steps per group
static_assert(X_LOADS == 2 && C_WAVES == 4, "copy split");
static_assert(kStages == kSteps, "stage and position in the group are both s mod 4");

typedef __attribute__((address_space(3))) void lds_void;

template <int V>
struct Ic {
  static constexpr int value = V;
};

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

// Wait until at most n vector-memory operations of this wave are in flight
// and all of its LDS operations are done (so LDS writes made before the
// following barrier are visible to the whole block after it).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// Wait until the copies of the step at group position ST have landed.  Every
// step, each wave issues L copies (for the step three ahead, clamped to the
// last step) and, at position 0, the 2 NT scale/zero loads of the next group
// (clamped to the last group) before them.  The memory counter retires in
// issue order, so the wait may leave in flight exactly what was issued after
// this step's copies: the next two steps' copies and, at positions 1 and 2,
// the scale/zero loads.  No load is conditional, so the counts are fixed.
template <int L, int ST>
__device__ __forceinline__ void wait_step() {
  constexpr int kMeta = 2 * NT;
  if (ST == 1 || ST == 2) wait_vmcnt<2 * L + kMeta>(); else wait_vmcnt<2 * L>();
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  // one LDS object per stage, so the compiler can tell the copies into one
  // stage from the reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[X_STAGE], xs1[X_STAGE], xs2[X_STAGE], xs3[X_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t cs0[C_STAGE], cs1[C_STAGE], cs2[C_STAGE], cs3[C_STAGE];
  __shared__ __attribute__((aligned(16))) float xsum_lds[BM];

  // XCD-aware tile order: consecutive block ids land on different XCDs, so
  // give XCD x the contiguous run of tiles [x T/8, (x+1) T/8), N fastest.
  const int T = m_tiles * n_tiles;
  int t = blockIdx.x;
  if (T % kXcds == 0) t = (t % kXcds) * (T / kXcds) + t / kXcds;
  const int m0 = (t / n_tiles) * BM;
  const int n0 = (t % n_tiles) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int G = K / kGroup;
  const int steps = kSteps * G;

  // ---- direct-to-LDS copies, addressed as a block-uniform base plus a
  // 32-bit per-lane byte offset (the launcher keeps these below 2^32).
  // X: copy j of wave w fills tile rows 16 (2w + j) .. +15 (64 B each);
  // lane -> row + lane/4, LDS chunk slot lane%4, which holds global chunk
  // slot ^ ((row >> 1) & 3) (= (lane >> 3) & 3).  Codes: wave w fills code
  // rows 64 (w % 4) .. +63, one 16-byte row per lane; waves 4..7 repeat the
  // copies of waves 0..3 (the same bytes to the same LDS rows), so every wave
  // issues the same three copies per step and one set of memory-counter
  // waits holds for all of them.  Rows past M (N) read the last row and are
  // never stored.
  const char* xblk = reinterpret_cast<const char*>(X + (int64_t)m0 * ldx);
  const int xrow0 = 16 * X_LOADS * wave + (lane >> 2);
  uint32_t xoffs[X_LOADS];
#pragma unroll
  for (int j = 0; j < X_LOADS; ++j)
    xoffs[j] = (uint32_t)(min(m0 + xrow0 + 16 * j, M - 1) - m0) * (uint32_t)(ldx * 2) +
               (uint32_t)(((lane & 3) ^ ((lane >> 3) & 3)) * 16);
  const int xoff0 = 16 * X_LOADS * wave * (KS * 2);
  const char* cblk = reinterpret_cast<const char*>(codes + (int64_t)n0 * (K / 8));
  const uint32_t coffs =
      (uint32_t)(min(n0 + 64 * (wave & (C_WAVES - 1)) + lane, N - 1) - n0) * (uint32_t)(K / 2);
  const int coff = 64 * (wave & (C_WAVES - 1)) * (KS / 2);
  // copies of K step t (the caller clamps t to the last step, so the copy
  // count per step never changes and the memory-counter waits stay fixed)
  auto issue = [&](uint8_t* xdst, uint8_t* cdst, int t) {
#pragma unroll
    for (int j = 0; j < X_LOADS; ++j)
      __builtin_amdgcn_global_load_lds(xblk + (xoffs[j] + (uint32_t)(t * KS * 2)),
                                       (lds_void*)&xdst[xoff0 + j * 16 * (KS * 2)], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(cblk + (coffs + (uint32_t)(t * (KS / 2))), (lds_void*)&cdst[coff], 16, 0, 0);
  };

  // this lane's output columns (one per 16-wide n tile) for scales / zeros:
  // column ncol + 16 nt, clamped to N - 1; element offsets from the block's
  // first column
  const int ncol = n0 + wn * WN + r16;
  const uint16_t* sblk = scales + (int64_t)n0 * G;
  const int32_t* zblk = zeros + (int64_t)n0 * G;
  uint32_t moffs[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) moffs[nt] = (uint32_t)(min(ncol + 16 * nt, N - 1) - n0) * (uint32_t)G;
  uint32_t s_cur[NT], s_nxt[NT];
  int z_cur[NT], z_nxt[NT];

  // LDS read offsets: A row (wm 128 + mt 16 + r16), logical chunk q (inputs
  // 8q .. 8q+7 of the step); B row (wn 64 + nt 16 + r16), word q.  Rows r
  // and r + 16 share the swizzle ((r >> 1) & 3).
  const int arow = wm * WM + r16;
  const int aoff = arow * (KS * 2) + ((q ^ ((arow >> 1) & 3)) * 16);
  const int boff = (wn * WN + r16) * (KS / 2) + q * 4;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 xpart[XS_TILES];  // this wave's share of the group's activation sums
  const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    s_cur[nt] = sblk[moffs[nt]];
    z_cur[nt] = zblk[moffs[nt]];
    s_nxt[nt] = s_cur[nt];
    z_nxt[nt] = z_cur[nt];
  }
  issue(xs0, cs0, 0);   // steps >= 4
  issue(xs1, cs1, 1);
  issue(xs2, cs2, 2);

  // fold a finished group into the accumulator: remove bias and zero point,
  // move to the next group's scale (or, after the last group, apply it)
  auto group_end = [&](bool last) {
    float zb[NT], ratio[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      zb[nt] = (float)(128 + z_cur[nt]);
      const float sc = bf16_to_f32(s_cur[nt]);
      ratio[nt] = last ? sc : sc * __builtin_amdgcn_rcpf(bf16_to_f32(s_nxt[nt]));
      s_cur[nt] = s_nxt[nt];
      z_cur[nt] = z_nxt[nt];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 xs = *reinterpret_cast<const f32x4*>(&xsum_lds[wm * WM + mt * 16 + 4 * q]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][nt][r] = fmaf(-zb[nt], xs[r], acc[mt][nt][r]) * ratio[nt];
    }
  };

  // One K step: stage ST = s mod 4 = position of the step in its group.
  // Copies for step s + 3 go to stage (ST + 3) mod 4, which every wave
  // finished reading at step s - 1.
  auto step = [&](auto stage, int s) {
    constexpr int ST = decltype(stage)::value;
    uint8_t* xs = ST == 0 ? xs0 : (ST == 1 ? xs1 : (ST == 2 ? xs2 : xs3));
    uint8_t* cs = ST == 0 ? cs0 : (ST == 1 ? cs1 : (ST == 2 ? cs2 : cs3));
    uint8_t* xn = ST == 0 ? xs3 : (ST == 1 ? xs0 : (ST == 2 ? xs1 : xs2));
    uint8_t* cn = ST == 0 ? cs3 : (ST == 1 ? cs0 : (ST == 2 ? cs1 : cs2));
    const int g = s / kSteps;
    wait_step<X_LOADS + 1, ST>();
    __builtin_amdgcn_s_barrier();
    if (ST == 0) {
      // the previous group's activation sums are in LDS: fold it in
      if (s > 0) group_end(false);
      // next group's scale/zero (the last group's again after the last),
      // issued before this step's copies, as wait_step counts them
      const int gn = min(g + 1, G - 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s_nxt[nt] = sblk[moffs[nt] + gn];
        z_nxt[nt] = zblk[moffs[nt] + gn];
      }
    }
    issue(xn, cn, min(s + 3, steps - 1));

    u32x4 b[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      b[nt] = codes_to_bias128_natural(*reinterpret_cast<const uint32_t*>(&cs[boff + nt * 16 * (KS / 2)]));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 af = *reinterpret_cast<const u32x4*>(&xs[aoff + mt * 16 * (KS * 2)]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x32(af, b[nt], acc[mt][nt]);
    }
    // this wave's share of the activation sums: its own two 16-row tiles,
    // re-read from LDS so no matrix-core op sits under a per-wave branch
#pragma unroll
    for (int i = 0; i < XS_TILES; ++i) {
      const u32x4 af = *reinterpret_cast<const u32x4*>(&xs[aoff + (wn * XS_TILES + i) * 16 * (KS * 2)]);
      xpart[i] = mfma16x16x32(af, ones, ST == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : xpart[i]);
    }
    if (ST == kSteps - 1) {
      // publish this wave's activation sums.  Every column of the ones
      // product holds the same sums, so all 16 lanes of a row group store
      // identical values to the same place; keeping the store outside any
      // lane-dependent branch keeps the matrix-core op that feeds it from
      // being moved under a partial exec mask.
#pragma unroll
      for (int i = 0; i < XS_TILES; ++i)
        *reinterpret_cast<f32x4*>(&xsum_lds[wm * WM + (wn * XS_TILES + i) * 16 + 4 * q]) = xpart[i];
    }
  };

  for (int s0 = 0; s0 < steps; s0 += kSteps) {
    step(Ic<0>{}, s0);
    step(Ic<1>{}, s0 + 1);
    step(Ic<2>{}, s0 + 2);
    step(Ic<3>{}, s0 + 3);
  }
  wait_vmcnt<0>();   // the clamped copies past the last step
  __syncthreads();   // last group's activation sums
  group_end(true);

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

}  // namespace

int launch_gemm(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                int64_t ldy, hipStream_t stream) {
  const int64_t mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
  if (mt * nt >= ((int64_t)1 << 31)) return 3;
  // per-lane 32-bit byte offsets within a tile's rows of X and of the codes
  if ((BM - 1) * ldx * 2 + K * 2 >= ((int64_t)1 << 32) || BN * (K / 2) >= ((int64_t)1 << 32)) return 3;
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)(mt * nt)), dim3(kThreads), 0, stream, X, (int)M,
                     ldx, codes, scales, zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
