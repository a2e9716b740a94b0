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
// One accumulator, rescaled per group, in a per-column unit that stays near
// one.  Group g's scale is split as s = u * 4^E with E = floor(log4 |s|)
// (clamped to kEmin..kEmax) and u = s * 4^-E, so |u| lies in [1, 4) for
// every normal scale.  The power of four goes into the B operand exactly:
// its BF16 exponent byte becomes 0x43 + E, so B = 4^E (128 + q), still an
// exact value, and the per-lane byte costs nothing in the unpack.  The
// accumulator T is kept in units of the current group's u:
//     end of group g:  T <- (T - 4^E (128 + z[n,g]) Xs[m]) * u_g / u_{g+1}
// and after the last group the factor is u_{G-1} itself, so T = Y.  The
// ratio of two units lies in (1/4, 4), so no sequence of scales can drive T
// out of range: tiny groups after large ones (down to the smallest normal
// BF16 scale), zero scales (the group then contributes at most 4^kEmin of
// the running unit, and the unit is kept), subnormal and negative scales
// all give the per-group result.  The unit ratio is a correctly rounded
// float32 division, one rounding per group.
//
// Tiling.  A 512-thread block (8 waves, 2 along M x 4 along N) computes a
// 256 x 256 tile of Y; each wave owns 128 x 64 (8 x 4 MFMA 16x16x32 tiles).
// (With few such tiles, 256-thread blocks of 128 x 128, waves of 64 x 64,
// three blocks per CU, or 128-thread blocks of 64 x 128.)  The waves that share a row half each compute the
// activation sums of two of its 16-row tiles (from A fragments they read
// anyway) and exchange them through LDS.  A K step is a quarter
// group (32 inputs): X[BM][32] of a step goes straight from global memory to
// LDS (global_load_lds_dwordx4) into one of four stages, issued four steps
// ahead; the codes of a whole group ([BN][64 bytes]) go the same way into
// one of two group buffers, a group ahead; one barrier per step.  The next
// step's A fragment of a row tile is read right after the row's products,
// so the LDS reads run under the matrix-core work.  16-byte
// chunks of each 64-byte LDS row are XOR-swizzled by (row >> 1) & 3, so the
// rows that one LDS cycle of a 16-byte-per-lane read serves fall on distinct
// bank groups.  Codes are unpacked in natural k order, so X needs no
// permutation.  Each lane loads the scales and zero points of one column of
// its wave per 128-input block; lane permutes spread the factors to the
// accumulator layout.  Groups of 32 or 64 inputs (two or four per block) end
// with the same rescale, every one or two K steps.  Tiles go to the 8 XCDs in contiguous runs with N fastest, so
// blocks that share X rows share an L2.

#include "common.h"

namespace w4a16 {
namespace {

constexpr int KS = 32;                 // inputs per K step (a quarter group)
constexpr int kSteps = kGroup / KS;    // K steps per group
constexpr int C_ROW = kGroup / 2;      // bytes of codes per column per group (64)
constexpr int kXcds = 8;

// Range of the power-of-four exponent E folded into the B operands: the
// exponent bytes 0x43 + E stay within 0x07 .. 0x7B, so B = 4^E (128 + q)
// (and 4^E (256 + 16 h) for the high nibble of 8-bit codes) are normal BF16
// values, and 4^E (128 + z) stays finite for any int32 z.
constexpr int kEmin = -60, kEmax = 56;

// Split of a group's scale (BF16 bits) into unit and exponent: E = floor(
// log4 |s|) clamped to kEmin .. kEmax, u = s 4^-E (|u| in [1, 4) for normal
// scales inside the clamp).  A zero scale keeps the previous unit (its group
// then adds at most 4^kEmin (128 + q) per input, in that unit).
__device__ __forceinline__ void split_scale(uint32_t sbits, float u_prev, int& E, float& u) {
  const int e2 = (int)((sbits >> 7) & 0xFFu);   // biased exponent of the scale
  E = min(max((e2 - 127) >> 1, kEmin), kEmax);
  const float s = bf16_to_f32(sbits);
  u = s == 0.f ? u_prev : __builtin_ldexpf(s, -2 * E);
}

// XCD-aware tile order: consecutive block ids land on different XCDs, so
// XCD x gets the contiguous run of tiles [x T/8, (x+1) T/8), N fastest.
__device__ __forceinline__ int tile_of(int bid, int T) {
  return T % kXcds == 0 ? (bid % kXcds) * (T / kXcds) + bid / kXcds : bid;
}

// Block tile BM x BN on (BM / WM) x (BN / WN) waves, each computing a
// WM x WN wave tile of 16x16 MFMA tiles.  The 256 x 256 tile (8 waves of
// 128 x 64) is the main one; 128 x 128 (4 waves of 64 x 64) keeps the CUs
// busy when there are few large tiles.
template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int MT = WM / 16, NT = WN / 16;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int X_STAGE = BM * KS * 2;   // bytes of X per stage, four stages
  static constexpr int C_GROUP = BN * C_ROW;    // bytes of codes per group, two buffers
  static constexpr int X_LOADS = X_STAGE / 1024 / kWaves;  // 1-KiB X copies per wave per step
  static constexpr int C_LOADS = C_GROUP / 1024 / kWaves;  // 1-KiB code copies per wave per group
  static constexpr int XS_TILES = MT / WAVES_N;  // activation-sum tiles computed by each wave
  static_assert(WAVES_M == 1 || WAVES_M == 2, "wm = wave % WAVES_M");
  static_assert(X_LOADS == 2 && (C_LOADS == 2 || C_LOADS == 4), "copy split");
  static_assert(XS_TILES == 2, "two activation-sum tiles per wave");
};
using TileBig = TileCfg<256, 256, 128, 64>;
using TileSmall = TileCfg<128, 128, 64, 64>;
using TileTiny = TileCfg<64, 128, 64, 64>;

// Memory operations each wave issues, in this order: at block position 0,
// the next block's scale and zero-point loads and C_LOADS code copies; at every
// step, X_LOADS copies of X for the step four ahead.  Nothing is
// conditional (indices are clamped to the last block / step), so the
// in-order memory counter gives fixed waits.  At the step at position ST
// the wait is for the X copies of the following step; what may stay in
// flight is everything issued after them: two more steps of X copies and,
// at positions 1 and 2, the block-start loads.  At position 3 the wait also
// covers the next block's code copies (issued before the awaited X copies).
template <class C, int ST, int CL>
__device__ __forceinline__ void wait_step() {
  constexpr int kBlockStart = 2 + CL;   // CL: code copies per wave per block
  if (ST == 1 || ST == 2) wait_vmcnt<2 * C::X_LOADS + kBlockStart>(); else wait_vmcnt<2 * C::X_LOADS>();
}

// GS: K steps per quantisation group (1, 2 or 4: groups of 32, 64 or 128
// inputs).  Codes always move in blocks of 128 inputs (four steps); a block
// holds kSteps / GS groups.
// W8: the W8A16 variant (8-bit codes, byte j of word i is k = 4i + j, groups
// of 128).  A code q = 16 h + l feeds two products on the same A fragment:
// B = 128 + l (the INT4 operand) and B = 256 + 16 h (8 h placed in mantissa
// bits 3..6 under the same exponent byte with the exponent's low bit set),
// both exact, so the accumulator gathers sum x q + 384 Xsum and the fold
// removes 384 + z.  Code rows are 128 bytes per block in LDS, their 16-byte
// chunks XOR-swizzled by row & 7.
// SPLIT: the block runs one run of Kl inputs of its tile (X, codes, scales
// and zeros already offset to the run's start; K stays the row length of the
// packed matrix) and stores the float32 partial tile to part[BM][BN] (its own
// slab) instead of the BF16 tile to Y.  bid is the tile's block index.
template <class C, int GS, bool W8 = false, bool SPLIT = false>
__device__ __forceinline__ void gemm_tile(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles, int bid, int Kl,
    float* __restrict__ part) {
  static_assert(GS == 1 || GS == 2 || GS == 4, "groups of 32, 64 or 128 inputs");
  constexpr int GPB = kSteps / GS;   // groups per 128-input block
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, MT = C::MT, NT = C::NT;
  static_assert(!W8 || GS == kSteps, "8-bit codes use groups of 128");
  constexpr int C_ROW_B = W8 ? 2 * C_ROW : C_ROW;            // code bytes per column per block
  constexpr int X_STAGE = C::X_STAGE, C_GROUP = BN * C_ROW_B;
  constexpr int X_LOADS = C::X_LOADS, C_LOADS = C_GROUP / 1024 / C::kWaves, XS_TILES = C::XS_TILES;
  static_assert(C_LOADS == 2 || C_LOADS == 4, "copy split");
  constexpr int CR_COPY = 1024 / C_ROW_B;                    // code rows per 1-KiB copy
  // one LDS object per buffer, so the compiler can tell the copies into one
  // buffer from the reads of another.  The X stages' larger alignment places
  // them first, below 64 KiB, where their addresses fit the immediate offset
  // of the LDS reads.
  __shared__ __attribute__((aligned(4096))) uint8_t xs0[X_STAGE], xs1[X_STAGE], xs2[X_STAGE], xs3[X_STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t cg0[C_GROUP], cg1[C_GROUP];
  // activation sums of a group, double-buffered by group parity (a group's
  // sums are read after the barrier that follows their store, and the next
  // store into the same buffer comes two groups later)
  __shared__ __attribute__((aligned(16))) float xsum_lds[2][BM];

  const int t = tile_of(bid, m_tiles * n_tiles);
  const int m0 = (t / n_tiles) * BM;
  const int n0 = (t % n_tiles) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int r16 = lane & 15, q = lane >> 4;
  const int G = Kl / kGroup;          // 128-input blocks (of the run)
  const int GR = (K / kGroup) * GPB;  // quantisation groups per row
  const int steps = kSteps * G;

  // ---- direct-to-LDS copies, addressed as a block-uniform base plus a
  // 32-bit per-lane byte offset (the launcher keeps these below 2^32).  A
  // copy instruction fills 64 consecutive 16-byte LDS slots, four per row:
  // lane -> row lane/4, slot lane%4, and slot p of row r holds the row's
  // 16-byte chunk p ^ ((r >> 1) & 3) (= (lane >> 3) & 3), so that reads of
  // one chunk from consecutive rows spread over the LDS banks.
  //   X, per step: rows of 32 inputs (64 B); copy j of wave w fills tile
  //   rows 16 (2w + j) .. +15.
  //   Codes, per group: rows of 128 codes (64 B, chunk = step); copy j of
  //   wave w fills code rows 16 (2w + j) .. +15.
  // Rows past M (N) read the last row and are never stored.
  const uint32_t swz = (uint32_t)(((lane & 3) ^ ((lane >> 3) & 3)) * 16);
  const char* xblk = reinterpret_cast<const char*>(X + (int64_t)m0 * ldx);
  const char* cblk = reinterpret_cast<const char*>(codes + (int64_t)n0 * (K / (W8 ? 4 : 8)));
  uint32_t xoffs[X_LOADS], coffs[C_LOADS];
#pragma unroll
  for (int j = 0; j < X_LOADS; ++j)
    xoffs[j] = (uint32_t)(min(m0 + 16 * (X_LOADS * wave + j) + (lane >> 2), M - 1) - m0) * (uint32_t)(ldx * 2) + swz;
#pragma unroll
  for (int j = 0; j < C_LOADS; ++j) {
    if constexpr (W8) {
      // lane -> code row (8 per copy) lane / 8, LDS slot lane % 8, which
      // holds the row's 16-byte chunk slot ^ (row & 7)
      const int row = CR_COPY * (C_LOADS * wave + j) + (lane >> 3);
      coffs[j] = (uint32_t)(min(n0 + row, N - 1) - n0) * (uint32_t)K + (uint32_t)((((lane & 7) ^ (row & 7))) * 16);
    } else {
      coffs[j] = (uint32_t)(min(n0 + 16 * (C_LOADS * wave + j) + (lane >> 2), N - 1) - n0) * (uint32_t)(K / 2) + swz;
    }
  }
  const int xdst0 = 16 * X_LOADS * wave * (KS * 2);
  const int cdst0 = CR_COPY * C_LOADS * wave * C_ROW_B;
  // X copies of K step t (clamped by the caller)
  auto copy_x = [&](uint8_t* dst, int t) {
#pragma unroll
    for (int j = 0; j < X_LOADS; ++j)
      __builtin_amdgcn_global_load_lds(xblk + (xoffs[j] + (uint32_t)(t * KS * 2)),
                                       (lds_void*)&dst[xdst0 + j * 16 * (KS * 2)], 16, 0, 0);
  };
  // code copies of group g (clamped by the caller)
  auto copy_codes = [&](uint8_t* dst, int g) {
#pragma unroll
    for (int j = 0; j < C_LOADS; ++j)
      __builtin_amdgcn_global_load_lds(cblk + (coffs[j] + (uint32_t)(g * C_ROW_B)),
                                       (lds_void*)&dst[cdst0 + j * 1024], 16, 0, 0);
  };

  // Scales and zero points: lane l of a wave fetches those of the wave's
  // column l (its WN = 64 columns, one per lane; clamped to N - 1), one
  // load of each per 128-input block (the block's GPB groups are adjacent
  // in memory), as 32-bit byte offsets from a block-uniform base (the
  // launcher checks the range) so the loads take a scalar base.  The
  // per-column factors are then moved to the lanes of the accumulator
  // layout (column r16 + 16 nt) by lane permutes.
  static_assert(WN == 64, "one metadata column per lane");
  const uint16_t* sblk = scales + (int64_t)n0 * GR;
  const int32_t* zblk = zeros + (int64_t)n0 * GR;
  const uint32_t moff = (uint32_t)(min(n0 + wn * WN + lane, N - 1) - n0) * (uint32_t)GR;
  // block b's scales of this lane's column, two per dword, and zero points
  uint32_t s_cur[(GPB + 1) / 2], s_nxt[(GPB + 1) / 2];
  int z_cur[GPB], z_nxt[GPB];
  auto ld_meta = [&](int b) {
    const uint32_t e = moff + (uint32_t)(b * GPB);
    const char* sp = reinterpret_cast<const char*>(sblk) + e * 2u;
    const char* zp = reinterpret_cast<const char*>(zblk) + e * 4u;
    if constexpr (GPB == 1) {
      s_nxt[0] = *reinterpret_cast<const uint16_t*>(sp);
      z_nxt[0] = *reinterpret_cast<const int32_t*>(zp);
    } else if constexpr (GPB == 2) {
      s_nxt[0] = *reinterpret_cast<const uint32_t*>(sp);
      const int2 z = *reinterpret_cast<const int2*>(zp);
      z_nxt[0] = z.x;
      z_nxt[1] = z.y;
    } else {
      const uint2 sv = *reinterpret_cast<const uint2*>(sp);
      s_nxt[0] = sv.x;
      s_nxt[1] = sv.y;
      const int4 z = *reinterpret_cast<const int4*>(zp);
      z_nxt[0] = z.x;
      z_nxt[1] = z.y;
      z_nxt[2] = z.z;
      z_nxt[3] = z.w;
    }
  };
  auto scale_of = [](const uint32_t* sv, int i) { return (i & 1) ? (sv[i >> 1] >> 16) : (sv[i >> 1] & 0xFFFFu); };

  // LDS read offsets.  A: row (wm 128 + mt 16 + r16), chunk q (inputs
  // 8q .. 8q+7 of the step).  B: code row (wn 64 + nt 16 + r16), chunk =
  // step position, word q.  Rows r and r + 16 share the swizzle.
  const int arow = wm * WM + r16;
  const int aoff = arow * (KS * 2) + ((q ^ ((arow >> 1) & 3)) * 16);
  const int brow = wn * WN + r16;
  const int bswz = (brow >> 1) & 3;
  const int boff = W8 ? brow * C_ROW_B + (q & 1) * 8 : brow * C_ROW + q * 4;
  // Row tiles in a wave-dependent order: register row tile j is row tile
  // rowt(j), so that the tiles whose activation sums this wave computes
  // (XS_TILES wn ..) come first and their A fragments are af[0 ..].
  const int rot = wn * XS_TILES;
  auto rowt = [&](int j) { return (j + rot) & (MT - 1); };

  f32x4 acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 xpart[XS_TILES];  // this wave's share of the group's activation sums
  const u32x4 ones = {kOnePair, kOnePair, kOnePair, kOnePair};

  // This lane's metadata column: the unit u and exponent E of the current
  // group (see split_scale), and per n tile the B exponent bytes of the
  // current group for the accumulator layout's column r16 + 16 nt.
  float u_col = 1.f;
  int e_col = 0;
  uint32_t eb[NT];
  // Groups of 128: the transition is prepared a step ahead (off the
  // critical path of the step that applies it), except on the 128 x 128
  // tiles at three waves per SIMD, whose register budget has no room for it.
  constexpr bool kPrep = GS == kSteps && (W8 || BM != TileSmall::BM);
  // A group transition, prepared (per metadata column, in this lane) ahead
  // of the step that applies it: the finished group's bias + zero point
  // times its 4^E, the unit ratio, and the next group's unit and exponent.
  float zl_p, rl_p, u_p;
  int e_p;
  auto spread_exponent = [&](int e) {
    const int ebl = (int)((uint32_t)(0x43 + e) * 0x01010101u);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) eb[nt] = (uint32_t)__builtin_amdgcn_ds_bpermute((r16 + 16 * nt) * 4, ebl);
  };
  // the first group of the row: its unit and exponent
  auto group_begin = [&](uint32_t s_first) {
    split_scale(s_first, 1.f, e_col, u_col);
    spread_exponent(e_col);
  };
  // prepare the end of the current group (zero point z_fin) and the move to
  // the group with scale s_next, or, when last, the final application of the
  // current unit; the current state does not change
  auto prep_transition = [&](int z_fin, uint32_t s_next, bool last) {
    zl_p = __builtin_ldexpf((float)z_fin + (W8 ? 384.f : 128.f), 2 * e_col);
    rl_p = u_col;
    u_p = u_col;
    e_p = e_col;
    if (!last) {
      split_scale(s_next, u_col, e_p, u_p);
      rl_p = u_col / u_p;
    }
  };
  // apply the prepared transition: lane permutes move the column factors to
  // the accumulator layout (column r16 + 16 nt), then the bias and zero
  // point leave the accumulator and it moves to the next unit; the next
  // group's exponent bytes follow the same way
  auto apply_transition = [&](const float* xbuf, bool last) {
    float zb[NT], ratio[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int src = (r16 + 16 * nt) * 4;
      zb[nt] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(zl_p)));
      ratio[nt] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(rl_p)));
    }
    if (!last) {
      u_col = u_p;
      e_col = e_p;
      spread_exponent(e_col);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 xs = *reinterpret_cast<const f32x4*>(&xbuf[wm * WM + rowt(mt) * 16 + 4 * q]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][nt][r] = fmaf(-zb[nt], xs[r], acc[mt][nt][r]) * ratio[nt];
    }
  };
  // fold a finished group into the accumulator in one go (transitions inside
  // a 128-input block, and the last group)
  auto group_end = [&](int z_fin, uint32_t s_next, bool last, const float* xbuf) {
    prep_transition(z_fin, s_next, last);
    apply_transition(xbuf, last);
  };

  // Operand fragments of one K step, read from LDS one step ahead of use:
  // the raw code words of the 4 column tiles (chunk `pos` of the group
  // buffer) and A of the 8 row tiles.
  // (8-bit codes: two words, inputs 8q .. 8q+7 of the step, from chunk
  // 2 pos + q / 2 of the 128-byte row)
  u32x4 af[MT];
  uint32_t bw[NT][W8 ? 2 : 1];
  auto read_b = [&](const uint8_t* cg, int pos) {
    if constexpr (W8) {
      const int bo = boff + (((2 * pos + (q >> 1)) ^ (brow & 7)) * 16);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint2 v = *reinterpret_cast<const uint2*>(&cg[bo + nt * 16 * C_ROW_B]);
        bw[nt][0] = v.x;
        bw[nt][1] = v.y;
      }
    } else {
      const int bo = boff + ((pos ^ bswz) * 16);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bw[nt][0] = *reinterpret_cast<const uint32_t*>(&cg[bo + nt * 16 * C_ROW]);
    }
  };
  // per-lane A read offsets of the row tiles, kept in registers (opaque to
  // the compiler) so that each read is one instruction: the stage buffer's
  // address goes into its immediate offset
  uint32_t aoffs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    aoffs[mt] = (uint32_t)(aoff + rowt(mt) * 16 * (KS * 2));
    asm volatile("" : "+v"(aoffs[mt]));
  }
  auto read_a = [&](const uint8_t* xs, int mt) {
    af[mt] = *reinterpret_cast<const u32x4*>(&xs[aoffs[mt]]);
  };
  auto read_frags = [&](const uint8_t* xs, const uint8_t* cg, int pos) {
    read_b(cg, pos);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) read_a(xs, mt);
  };

  // prologue: group 0's scale/zero and codes, steps 0..3 of X in flight,
  // step 0's fragments in registers (steps >= 4)
  ld_meta(0);   // block 0's, moved to the current set at step 0
  auto prologue = [&](uint8_t* cg_first) {   // group 0's code buffer
    copy_codes(cg_first, 0);
    copy_x(xs0, 0);
    copy_x(xs1, 1);
    copy_x(xs2, 2);
    copy_x(xs3, 3);
    wait_vmcnt<3 * X_LOADS>();
    block_barrier();
    read_frags(xs0, cg_first, 0);
  };
  // (two static calls rather than one with a selected pointer, so the
  // compiler still tells the two code buffers apart)
  if (G & 1) prologue(cg1); else prologue(cg0);
  // block 0's metadata landed before the prologue's barrier: the first
  // group's unit and B exponent
  group_begin(scale_of(s_nxt, 0));

  // One K step s at group position ST = s mod 4 of a group using code
  // buffer GP, whose X sits in stage ST; its fragments
  // are already in registers.  After the barrier stage ST is free (its reads
  // finished before it), so it takes the X of step s + 4; at position 0 the
  // other code buffer (read last two steps ago) takes the next group's
  // codes.  Meanwhile the fragments of step s + 1 are read while the matrix
  // cores work on step s.
  auto step = [&](auto stage, auto parity, int s) {
    constexpr int ST = decltype(stage)::value;
    constexpr int GP = decltype(parity)::value;
    uint8_t* xs_here = ST == 0 ? xs0 : (ST == 1 ? xs1 : (ST == 2 ? xs2 : xs3));
    uint8_t* xs_next = ST == 0 ? xs1 : (ST == 1 ? xs2 : (ST == 2 ? xs3 : xs0));
    uint8_t* cg_here = GP == 0 ? cg0 : cg1;
    uint8_t* cg_other = GP == 0 ? cg1 : cg0;
    const int g = s / kSteps;
    wait_step<C, ST, C_LOADS>();   // step s + 1 landed, every read of stage ST done
    block_barrier();
    // pin this step's fragments here, so the compiler cannot pull their uses
    // up into the previous step next to the reads that produced them
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(af[mt]));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int w = 0; w < (W8 ? 2 : 1); ++w) asm volatile("" : "+v"(bw[nt][w]));
    if (ST == 0) {
      // the previous block's last group: its activation sums are in LDS
      if (s > 0) {
        if constexpr (kPrep)
          apply_transition(xsum_lds[GP ^ 1], false);   // prepared at the previous step
        else
          group_end(z_cur[GPB - 1], scale_of(s_nxt, 0), false, xsum_lds[GS == kSteps ? GP ^ 1 : 1]);
      }
#pragma unroll
      for (int i = 0; i < (GPB + 1) / 2; ++i) s_cur[i] = s_nxt[i];
#pragma unroll
      for (int i = 0; i < GPB; ++i) z_cur[i] = z_nxt[i];
      // next block's scales/zeros and codes (the last block's again after
      // the last), issued before this step's X copies, as wait_step counts
      // them
      const int gn = min(g + 1, G - 1);
      ld_meta(gn);
      copy_codes(cg_other, gn);
    } else if (ST % GS == 0) {
      // a group inside the block ends
      constexpr int i = ST / GS;
      group_end(z_cur[i - 1], scale_of(s_cur, i), false, xsum_lds[(i - 1) & 1]);
    } else if (kPrep && ST == kSteps - 1) {
      // the next block's metadata landed with this step's wait: prepare the
      // transition the next step applies (after the last group it is unused)
      prep_transition(z_cur[0], scale_of(s_nxt, 0), false);
    }
    copy_x(xs_here, min(s + 4, steps - 1));

    // this wave's share of the activation sums: its own row tiles, the
    // first XS_TILES register row tiles
#pragma unroll
    for (int i = 0; i < XS_TILES; ++i)
      xpart[i] = mfma16x16x32(af[i], ones, ST % GS == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : xpart[i]);
    u32x4 b[NT], bh[W8 ? NT : 1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (W8) {
        // low nibbles l -> bytes l; high nibbles h -> bytes 0x80 | 8 h (BF16
        // 0x43, 0x80 | 8h = 256 + 16 h; under 0x43 + E both scale by 4^E)
        const uint32_t l0 = bw[nt][0] & 0x0F0F0F0Fu, h0 = ((bw[nt][0] >> 1) & 0x78787878u) | 0x80808080u;
        const uint32_t l1 = bw[nt][1] & 0x0F0F0F0Fu, h1 = ((bw[nt][1] >> 1) & 0x78787878u) | 0x80808080u;
        const uint32_t e = eb[nt];
        b[nt] = u32x4{__builtin_amdgcn_perm(e, l0, 0x04010400u), __builtin_amdgcn_perm(e, l0, 0x04030402u),
                      __builtin_amdgcn_perm(e, l1, 0x04010400u), __builtin_amdgcn_perm(e, l1, 0x04030402u)};
        bh[nt] = u32x4{__builtin_amdgcn_perm(e, h0, 0x04010400u), __builtin_amdgcn_perm(e, h0, 0x04030402u),
                       __builtin_amdgcn_perm(e, h1, 0x04010400u), __builtin_amdgcn_perm(e, h1, 0x04030402u)};
      } else {
        b[nt] = codes_to_bias128_natural(bw[nt][0], eb[nt]);
      }
    }
    // the next step's fragments (past the last step: a harmless re-read):
    // code words into the registers just freed, each A row tile after its
    // products
    if (ST == kSteps - 1) read_b(cg_other, 0); else read_b(cg_here, ST + 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 a = af[mt];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[mt][nt] = mfma16x16x32(a, b[nt], acc[mt][nt]);
        if constexpr (W8) acc[mt][nt] = mfma16x16x32(a, bh[nt], acc[mt][nt]);
      }
      read_a(xs_next, mt);
    }
    if constexpr (ST == 0) {
      // scheduling hint for the step that carries the block's first rescale:
      // alternate one matrix op with four vector ops, so the rescale and the
      // unpack interleave with the products instead of preceding them all
      // (+1-6% on the 8B-shaped layers at M = 4096; eight per op: no gain)
#pragma unroll
      for (int i = 0; i < 34; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
      }
    }
    if (ST % GS == GS - 1) {
      // publish this wave's activation sums of the group.  Every column of the ones
      // product holds the same sums, so all 16 lanes of a row group store
      // identical values to the same place; keeping the store outside any
      // lane-dependent branch keeps the matrix-core op that feeds it from
      // being moved under a partial exec mask.
#pragma unroll
      for (int i = 0; i < XS_TILES; ++i)
        *reinterpret_cast<f32x4*>(&xsum_lds[GS == kSteps ? GP : (ST / GS) & 1][wm * WM + (wn * XS_TILES + i) * 16 + 4 * q]) = xpart[i];
    }
  };
  auto group = [&](auto parity, int g) {
    step(Ic<0>{}, parity, kSteps * g);
    step(Ic<1>{}, parity, kSteps * g + 1);
    step(Ic<2>{}, parity, kSteps * g + 2);
    step(Ic<3>{}, parity, kSteps * g + 3);
  };

  // groups run in pairs (code buffer 0, then 1); an odd count starts with
  // the second half of a pair
  for (int g = -(G & 1); g < G; g += 2) {
    if (g >= 0) group(Ic<0>{}, g);
    group(Ic<1>{}, g + 1);
  }
  wait_vmcnt<0>();   // the clamped copies past the last step
  __syncthreads();   // last group's activation sums (odd parity: see above)
  group_end(z_cur[GPB - 1], 0u, true, xsum_lds[1]);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + wn * WN + nt * 16 + r16;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * WM + rowt(mt) * 16 + 4 * q + r;
        if constexpr (SPLIT) {
          if (m < M) part[(m - m0) * BN + (n - n0)] = acc[mt][nt][r];
        } else {
          if (m < M) Y[(int64_t)m * ldy + n] = f32_to_bf16_rne(acc[mt][nt][r]);
        }
      }
    }
}

// One kernel per tile shape, templated on the steps per group.
template <int GS>
__global__ __launch_bounds__(TileBig::kThreads) void gemm_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  gemm_tile<TileBig, GS>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, m_tiles, n_tiles, (int)blockIdx.x, K,
                         nullptr);
}

// three blocks per CU: the register budget of three waves per SIMD (without
// it the compiler keeps the accumulators in AGPRs at one wave per SIMD)
template <int GS>
__global__ __launch_bounds__(TileSmall::kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gemm_small_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  gemm_tile<TileSmall, GS>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, m_tiles, n_tiles, (int)blockIdx.x, K,
                           nullptr);
}

// 128 x 128 tiles for groups of 32 or 64 inputs and for 8-bit codes: two
// waves per SIMD, so that the more frequent rescale or the second set of B
// operands has the registers it needs
template <int GS, bool W8>
__global__ __launch_bounds__(TileSmall::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_small2_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  gemm_tile<TileSmall, GS, W8>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, m_tiles, n_tiles, (int)blockIdx.x,
                               K, nullptr);
}

// 64 x 128 tiles on two waves of 64 x 64, for layers whose 128 x 128 tiles
// would still leave CUs idle (two waves per SIMD: at three the compiler
// moves values into AGPRs)
template <int GS>
__global__ __launch_bounds__(TileTiny::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tiny_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K,
    uint16_t* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  gemm_tile<TileTiny, GS>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, m_tiles, n_tiles, (int)blockIdx.x, K,
                          nullptr);
}

// K split over ksplit equal runs of whole 128-input blocks (groups of 128)
// for the R tiles of block index t_full .. t_full + R - 1 (all tiles, or
// those past the last whole round of CUs): block b computes split tile
// r = b % R over run b / R and stores its float32 partial tile to the slab
// part + (run R + r) BM BN; split_reduce_kernel then adds the runs in order.
template <class C>
__device__ __forceinline__ void gemm_split_tile(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K, int m_tiles,
    int n_tiles, int t_full, int R, int ksplit, float* __restrict__ part) {
  const int r = (int)blockIdx.x % R, ks = (int)blockIdx.x / R, Kl = K / ksplit;
  const int64_t kb = (int64_t)ks * Kl;
  gemm_tile<C, kSteps, false, true>(X + kb, M, ldx, codes + kb / 8, scales + kb / kGroup, zeros + kb / kGroup, N,
                                    K, nullptr, 0, m_tiles, n_tiles, t_full + r, Kl,
                                    part + ((int64_t)ks * R + r) * (C::BM * C::BN));
}

__global__ __launch_bounds__(TileBig::kThreads) void gemm_split_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K, int m_tiles,
    int n_tiles, int t_full, int R, int ksplit, float* __restrict__ part) {
  gemm_split_tile<TileBig>(X, M, ldx, codes, scales, zeros, N, K, m_tiles, n_tiles, t_full, R, ksplit, part);
}

__global__ __launch_bounds__(TileSmall::kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gemm_small_split_kernel(
    const uint16_t* __restrict__ X, int M, int64_t ldx, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int N, int K, int m_tiles,
    int n_tiles, int t_full, int R, int ksplit, float* __restrict__ part) {
  gemm_split_tile<TileSmall>(X, M, ldx, codes, scales, zeros, N, K, m_tiles, n_tiles, t_full, R, ksplit, part);
}

// The split tiles' outputs: Y = BF16 of the sum of the ksplit partial slabs
// in run order (fixed, so the result is deterministic); four consecutive
// outputs of a tile row per thread, stored where they fall inside Y.
template <int BM, int BN>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int ksplit, int R,
                                                           int t_full, int m_tiles, int n_tiles, int M, int N,
                                                           uint16_t* __restrict__ Y, int64_t ldy) {
  constexpr int TILE = BM * BN;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)R * (TILE / 4)) return;
  const int r = (int)(idx / (TILE / 4)), e = (int)(idx - (int64_t)r * (TILE / 4)) * 4;
  const int t = tile_of(t_full + r, m_tiles * n_tiles);
  const int m = (t / n_tiles) * BM + e / BN, n = (t % n_tiles) * BN + e % BN;
  if (m >= M) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)r * TILE + e);
  for (int k = 1; k < ksplit; ++k) v += *reinterpret_cast<const f32x4*>(part + ((int64_t)k * R + r) * TILE + e);
  uint16_t* y = Y + (int64_t)m * ldy + n;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (n + i < N) y[i] = f32_to_bf16_rne(v[i]);
}

}  // namespace

namespace {
template <class C, int GS, bool W8 = false>
int launch_tiles(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                 const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                 int64_t ldy, hipStream_t stream, int ksplit = 1, float* part = nullptr, int64_t t_full = 0) {
  const int64_t mt = (M + C::BM - 1) / C::BM, nt = (N + C::BN - 1) / C::BN;
  if (mt * nt >= ((int64_t)1 << 31)) return 3;
  // per-lane 32-bit byte offsets within a tile's rows of X, of the codes and
  // of the zero points
  if ((C::BM - 1) * ldx * 2 + K * 2 >= ((int64_t)1 << 32) || C::BN * (W8 ? K : K / 2) >= ((int64_t)1 << 32) ||
      C::BN * (K / (KS * GS)) * 4 >= ((int64_t)1 << 32))
    return 3;
  const dim3 grid((unsigned)(mt * nt)), block(C::kThreads);
  if (ksplit > 1) {
    // tiles of block index < t_full whole (the same kernel as unsplit, on a
    // grid of t_full blocks), the other R split over ksplit runs through the
    // float32 partial slabs in `part`
    if constexpr (GS == kSteps && !W8 && C::BM != TileTiny::BM) {
      const int64_t R = mt * nt - t_full;
      if (t_full > 0) {
        if constexpr (C::BM == TileBig::BM)
          hipLaunchKernelGGL(gemm_kernel<GS>, dim3((unsigned)t_full), block, 0, stream, X, (int)M, ldx, codes,
                             scales, zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
        else
          hipLaunchKernelGGL(gemm_small_kernel<GS>, dim3((unsigned)t_full), block, 0, stream, X, (int)M, ldx,
                             codes, scales, zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
      }
      const dim3 sgrid((unsigned)(R * ksplit));
      if constexpr (C::BM == TileBig::BM)
        hipLaunchKernelGGL(gemm_split_kernel, sgrid, block, 0, stream, X, (int)M, ldx, codes, scales, zeros,
                           (int)N, (int)K, (int)mt, (int)nt, (int)t_full, (int)R, ksplit, part);
      else
        hipLaunchKernelGGL(gemm_small_split_kernel, sgrid, block, 0, stream, X, (int)M, ldx, codes, scales,
                           zeros, (int)N, (int)K, (int)mt, (int)nt, (int)t_full, (int)R, ksplit, part);
      const int64_t threads = R * (C::BM * C::BN / 4);
      hipLaunchKernelGGL((split_reduce_kernel<C::BM, C::BN>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                         stream, part, ksplit, (int)R, (int)t_full, (int)mt, (int)nt, (int)M, (int)N, Y, ldy);
      return hipGetLastError() == hipSuccess ? 0 : 4;
    } else {
      return 3;
    }
  }
  if constexpr (C::BM == TileBig::BM)
    hipLaunchKernelGGL(gemm_kernel<GS>, grid, block, 0, stream, X, (int)M, ldx, codes, scales,
                       zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
  else if constexpr (C::BM == TileSmall::BM && GS == kSteps && !W8)
    hipLaunchKernelGGL(gemm_small_kernel<GS>, grid, block, 0, stream, X, (int)M, ldx, codes, scales,
                       zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
  else if constexpr (C::BM == TileSmall::BM)
    hipLaunchKernelGGL((gemm_small2_kernel<GS, W8>), grid, block, 0, stream, X, (int)M, ldx, codes,
                       scales, zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
  else
    hipLaunchKernelGGL(gemm_tiny_kernel<GS>, grid, block, 0, stream, X, (int)M, ldx, codes, scales,
                       zeros, (int)N, (int)K, Y, ldy, (int)mt, (int)nt);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
}  // namespace

namespace {
// Groups of 128: 256 x 256 tiles when there are at least three per four
// CUs.  On whole layers the 128 x 128 tiles run at ~560-610 TFLOP/s and the
// large ones at ~750-770, so smaller tiles win only when the large ones would
// leave a quarter of the CUs idle (at 192 large tiles the two are level).
// Between 128 x 128 and 64 x 128 tiles the one whose block count fills the
// rounds of CUs better wins, ties to the larger tile (measured on the
// 8B-shaped layers, M = 512 .. 4096).
// With a workspace, K may instead be split over KS = 2, 4 or 8 runs of at
// least 1024 inputs (float32 partial tiles of at most kGemmSplitMaxBytes,
// added by a further launch).  When the large tiles fill the CUs: the tiles
// past the last whole round, if splitting them KS = 2 or 4 ways makes them
// take at most half a round (384 tiles: one round of whole tiles, then 128
// tiles over 2 runs).  Otherwise, every tile: the smallest KS whose 256 x 256
// blocks fill at least three quarters of the rounds of CUs, else the smallest
// whose 128 x 128 blocks do.  Measured on the 8B-shaped layers (M = 512: 425
// -> 306 us for the four; down 174 -> 85 us, o 55 -> 42 us; M = 1024: down 205
// -> 140 us, o 64 -> 59; M = 2048: down 303 -> 254 us).
constexpr int64_t kGemmSplitMaxBytes = (int64_t)128 << 20;

struct GemmPlan {
  int cfg;         // 0: 256 x 256, 1: 128 x 128, 2: 64 x 128
  int ksplit;      // runs of K (1: no split)
  int64_t t_full;  // tiles (by block index) computed whole; the rest are split
  int64_t ws_bytes;
};

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, bool split) {
  const int64_t cus = device_cu_count();
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  auto fill = [&](int64_t t) { return (double)t / (double)(((t + cus - 1) / cus) * cus); };
  const int64_t big = tiles(TileBig::BM, TileBig::BN), small = tiles(TileSmall::BM, TileSmall::BN);
  auto ok = [&](int ks, int64_t split_tiles, int64_t tile) {
    return K % (kGroup * ks) == 0 && K / ks >= 1024 && (int64_t)ks * split_tiles * tile * 4 <= kGemmSplitMaxBytes;
  };
  constexpr int64_t kBig = (int64_t)TileBig::BM * TileBig::BN, kSmall = (int64_t)TileSmall::BM * TileSmall::BN;
  if (4 * big >= 3 * cus) {
    const int64_t rem = big % cus;
    if (split && big > cus && rem > 0)
      for (int ks : {2, 4})
        if (ok(ks, rem, kBig) && ((rem * ks + cus - 1) / cus) * 2 <= ks)
          return GemmPlan{0, ks, big - rem, ks * rem * kBig * 4};
    return GemmPlan{0, 1, 0, 0};
  }
  if (split) {
    for (int ks : {2, 4, 8})
      if (ok(ks, big, kBig) && fill(big * ks) >= 0.75) return GemmPlan{0, ks, 0, ks * big * kBig * 4};
    for (int ks : {2, 4, 8})
      if (ok(ks, small, kSmall) && fill(small * ks) >= 0.75 && fill(small * ks) > fill(small) + 1e-9)
        return GemmPlan{1, ks, 0, ks * small * kSmall * 4};
  }
  if (fill(tiles(TileTiny::BM, TileTiny::BN)) > fill(small) + 1e-9) return GemmPlan{2, 1, 0, 0};
  return GemmPlan{1, 1, 0, 0};
}

int launch_gemm_g128(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                     const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                     int64_t ldy, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  GemmPlan p = gemm_plan(M, N, K, workspace != nullptr);
  if (p.ksplit > 1 && workspace_bytes < p.ws_bytes) p = gemm_plan(M, N, K, false);
  float* part = reinterpret_cast<float*>(workspace);
  if (p.cfg == 0)
    return launch_tiles<TileBig, kSteps>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream, p.ksplit, part,
                                         p.t_full);
  if (p.cfg == 2)
    return launch_tiles<TileTiny, kSteps>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream);
  return launch_tiles<TileSmall, kSteps>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream, p.ksplit, part,
                                         p.t_full);
}
}  // namespace

// Workspace with which launch_gemm may split K for this shape (groups of
// 128; 0: none needed).
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) { return gemm_plan(M, N, K, true).ws_bytes; }

// group: 32, 64 or 128 inputs per quantisation group (checked by the caller)
int launch_gemm(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, int group,
                uint16_t* Y, int64_t ldy, hipStream_t stream, void* workspace, int64_t workspace_bytes) {
  // Groups of 32 or 64: a rescale every one or two steps; 256 x 256 tiles
  // would spill their accumulators, so 128 x 128 tiles at two waves per
  // SIMD, or 64 x 128 tiles when those fill the rounds of CUs better.
  if (group != kGroup) {
    const int64_t cus = device_cu_count();
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    auto fill = [&](int64_t t) { return (double)t / (double)(((t + cus - 1) / cus) * cus); };
    const bool tiny =
        fill(tiles(TileTiny::BM, TileTiny::BN)) > fill(tiles(TileSmall::BM, TileSmall::BN)) + 1e-9;
    if (group == 32)
      return tiny ? launch_tiles<TileTiny, 1>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream)
                  : launch_tiles<TileSmall, 1>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream);
    return tiny ? launch_tiles<TileTiny, 2>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream)
                : launch_tiles<TileSmall, 2>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream);
  }
  return launch_gemm_g128(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, workspace, workspace_bytes, stream);
}

// W8A16 variant, any M >= 1 (checked by the caller): 128 x 128 tiles
int launch_gemm_int8(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                     const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                     int64_t ldy, hipStream_t stream) {
  return launch_tiles<TileSmall, kSteps, true>(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, stream);
}

}  // namespace w4a16
