// Decode of a chain of dependent W4A16 linears in one persistent launch
// (gfx950).
//
// A decoder's weight stream is a chain: each linear's input is formed from
// the previous linear's output (in a decoder layer: qkv, o, gate_up,
// down).  Launched one linear at a time, every launch pays the
// dispatch, the ramp until its first loads return and the tail of its last
// blocks, about 1.5-3 us each, and nothing streams in between ("Weight-Only
// Quantization and Mixed Precision", "7. The Marlin Kernel": round trips
// between separate kernels eat the benefit).  Here one block per CU runs the
// whole chain.  Wave 0 is the control wave; waves 1..15 stream weights:
//
//   for each linear l:
//     all waves stage X_l in LDS: formed from the previous output by the
//       linear's glue (as is, SwiGLU of [gate | up], or single-key attention:
//       each head's value vector), times the optional producer weight,
//       rounded to BF16, stored pair-permuted with the activation sums of
//       every 32 inputs (consecutive lanes read consecutive 8-input octets
//       with coherent 64-bit loads, several octets' loads in flight);
//     the streaming waves take the block's rows of W_l, four rows x 2048
//       inputs per item, with the exact operands 128 + q and the per-group
//       fold of the decode kernel (s (P - (128 + z) Xsum), v_dot2_f32_bf16);
//       each keeps two items in flight in registers, and its load cursor runs
//       on into the next linears, so the weight stream continues through
//       the steps below;
//     the control wave adds the K slices of each row in LDS in a fixed
//       order, stores Y_l in BF16 (a producer of exactly [gate | up] for a
//       SwiGLU input owns gate and up rows k, K' + k and also stores that
//       input, formed once, in the workspace's glue region), waits for its
//       stores and meets the other blocks at a grid barrier while the
//       streaming waves wait at a block barrier with their loads in flight.
//
// The outputs pass between blocks (and the XCDs' separate L2 caches) as
// agent-scope atomic stores (32-bit) and loads (32- and 64-bit), coherent across the
// device without the L2 write-back and invalidation an agent-scope fence
// costs (measured on MI355X: 5.3 against 1.7 us per barrier).  The barrier
// is two-level: blocks arrive on 16 counters on separate cache lines, the
// last of each group on a top counter, and the last of all publishes the
// next generation into 8 copies that the blocks poll (one flat counter: 3.7
// us).  The grid is one block per CU, all resident at once (the block's
// registers fill a CU), launched normally (a cooperative launch costs ~20 us
// more).  Every barrier wait is bounded: a block that waits longer than the
// plan's spin limit records a timeout in the workspace status word and goes
// on, so every launch ends.  Results are deterministic.

#include "chain.h"
#include "common.h"

#include <atomic>

#include "w4a16.h"

namespace w4a16 {

namespace {

constexpr int kChainWaves = 16;
constexpr int kChainThreads = kChainWaves * 64;
constexpr int kChainSlice = 2048;     // inputs per wave item: 64 lanes x 32
constexpr int kRing = 2;              // weight items in flight per streaming wave
constexpr int kStageU = 2;            // input octets per thread and staging pass

constexpr int kGroups = kChainGroups, kGenCopies = kChainGenCopies;
constexpr int kTopWord = kChainTopWord, kStatusWord = kChainStatusWord, kGenWord0 = kChainGenWord0;

// Coherent accesses through global-address-space pointers: the pointers
// come from descriptors in memory, and as generic pointers the loads would be
// flat loads, which also count on the LDS counter and serialise the staging.
typedef __attribute__((address_space(1))) unsigned g_u32;
typedef __attribute__((address_space(1))) const unsigned g_cu32;
typedef __attribute__((address_space(1))) const uint64_t g_cu64;

__device__ __forceinline__ unsigned ld_coherent(const unsigned* p) {
  return __hip_atomic_load((g_cu32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(unsigned* p, unsigned v) {
  __hip_atomic_store((g_u32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ld_coherent64(const uint64_t* p) {
  return __hip_atomic_load((g_cu64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float lo16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four BF16 values of a 64-bit word, in order.
__device__ __forceinline__ void unpack4(uint64_t w, float* v) {
  v[0] = lo16((unsigned)w);
  v[1] = hi16((unsigned)w);
  v[2] = lo16((unsigned)(w >> 32));
  v[3] = hi16((unsigned)(w >> 32));
}

// The 8 inputs 8o .. 8o+7 of activation row m as formed by the linear's glue
// (before the producer weight), in two steps so that a thread can issue the
// loads of several octets before it waits for the first: fetch_octet loads
// the raw BF16 words (consecutive lanes take consecutive octets, so every
// load instruction of a wave covers one contiguous run of the previous
// output: two coherent 64-bit loads per octet and source, rows 16-byte
// aligned), form_octet applies the glue.  Single-key attention reads whole
// octets when heads are a multiple of 8 inputs and the value block starts at
// a multiple of 4; otherwise form_octet reads it element by element.
// Staging kind of an input its producer already formed (SwiGLU and the
// producer weight applied, rounded to BF16) into the workspace's glue region.
constexpr int kGlued = 4;

__device__ __forceinline__ bool attn_octets(const ChainDesc& d) {
  return d.head_dim % 8 == 0 && d.v_offset % 4 == 0;
}

template <int KIND>
__device__ __forceinline__ void fetch_octet(const ChainDesc& d, const ChainDesc* prev, const uint16_t* X0,
                                            int64_t ldx, const uint16_t* glue, int m, int o, uint64_t w[4]) {
  const int k0 = 8 * o;
  if constexpr (KIND == kGlued) {
    const uint64_t* row = reinterpret_cast<const uint64_t*>(glue + (int64_t)m * d.K);
    w[0] = ld_coherent64(row + 2 * o);
    w[1] = ld_coherent64(row + 2 * o + 1);
  } else if constexpr (KIND == W4A16_CHAIN_X0) {
    const uint64_t* p = reinterpret_cast<const uint64_t*>(X0 + (int64_t)m * ldx + k0);
    w[0] = p[0];
    w[1] = p[1];
  } else {
    const uint64_t* row = reinterpret_cast<const uint64_t*>(prev->y + (int64_t)m * prev->ldy);
    if constexpr (KIND == W4A16_CHAIN_PREV) {
      w[0] = ld_coherent64(row + 2 * o);
      w[1] = ld_coherent64(row + 2 * o + 1);
    } else if constexpr (KIND == W4A16_CHAIN_SWIGLU) {
      w[0] = ld_coherent64(row + 2 * o);
      w[1] = ld_coherent64(row + 2 * o + 1);
      w[2] = ld_coherent64(row + d.K / 4 + 2 * o);
      w[3] = ld_coherent64(row + d.K / 4 + 2 * o + 1);
    } else {   // W4A16_CHAIN_ATTN1 with whole octets (attn_octets)
      const int h = k0 / d.head_dim;
      const int src = d.v_offset + (h / d.group) * d.head_dim + (k0 - h * d.head_dim);   // multiple of 4
      w[0] = ld_coherent64(row + src / 4);
      w[1] = ld_coherent64(row + src / 4 + 1);
    }
  }
}

// KIND: the glue, or -1 for single-key attention read element by element
template <int KIND>
__device__ __forceinline__ void form_octet(const ChainDesc& d, const ChainDesc* prev, int m, int o,
                                           const uint64_t w[4], float v[8]) {
  if constexpr (KIND == W4A16_CHAIN_SWIGLU) {
    float g[8], u[8];
    unpack4(w[0], g);
    unpack4(w[1], g + 4);
    unpack4(w[2], u);
    unpack4(w[3], u + 4);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = g[t] * __builtin_amdgcn_rcpf(1.f + __expf(-g[t])) * u[t];
  } else if constexpr (KIND >= 0) {
    unpack4(w[0], v);
    unpack4(w[1], v + 4);
  } else {
    const unsigned* row32 = reinterpret_cast<const unsigned*>(prev->y + (int64_t)m * prev->ldy);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int k = 8 * o + t;
      const int h = k / d.head_dim;
      const int e = d.v_offset + (h / d.group) * d.head_dim + (k - h * d.head_dim);
      const unsigned x = ld_coherent(row32 + e / 2);
      v[t] = (e & 1) ? hi16(x) : lo16(x);
    }
  }
}

// Block barrier without a wait on vector memory (the compiler may not move
// memory accesses across it; loads in flight stay in flight).
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Grid barrier, arrival half: the block's stores are complete (every wave
// waited for its stores, then the block synchronised), thread 0 arrives on its group's counter, the last
// of a group on the top counter, and the last of all resets the counters and
// publishes the next generation.  Returns true in the thread that published.
__device__ __forceinline__ bool grid_arrive(unsigned* bar, unsigned nblocks, unsigned gen) {
  if (threadIdx.x != 0) return false;
  const unsigned g = blockIdx.x % kGroups;
  const unsigned gsize = (nblocks - g + kGroups - 1) / kGroups;
  const unsigned groups = nblocks < (unsigned)kGroups ? nblocks : (unsigned)kGroups;
  const unsigned a = __hip_atomic_fetch_add(bar + 16 * g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a != gsize - 1) return false;
  st_coherent(bar + 16 * g, 0u);
  const unsigned t = __hip_atomic_fetch_add(bar + kTopWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t != groups - 1) return false;
  st_coherent(bar + kTopWord, 0u);
#pragma unroll
  for (int j = 0; j < kGenCopies; ++j) st_coherent(bar + kGenWord0 + 16 * j, gen + 1u);
  return true;
}

// Grid barrier, waiting half (thread 0; bounded), then the block follows.
__device__ __forceinline__ void grid_wait(unsigned* bar, unsigned gen, bool published, int spin_limit) {
  if (threadIdx.x == 0 && !published) {
    const unsigned* w = bar + kGenWord0 + 16 * (blockIdx.x % kGenCopies);
    int spins = 0;
    while (ld_coherent(w) == gen) {
      if (++spins > spin_limit) {
        st_coherent(bar + kStatusWord, (unsigned)W4A16_CHAIN_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  block_sync_lds();
}

typedef const __attribute__((address_space(4))) ChainDesc CDesc;

template <int M>
__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainDesc* __restrict__ descs, int n_linears,
                                                              const uint16_t* __restrict__ X0, int64_t ldx,
                                                              unsigned* __restrict__ bar, int spin_limit,
                                                              int max_k, int max_rows) {
  constexpr int R = 4;                          // rows per item
  constexpr int MP = M == 1 ? 1 : 2;            // values per lane after the group step
  constexpr int S = kChainWaves - 1;            // streaming waves
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // X of the current linear, pair-permuted, [m][chunk c = 64 slice + lane][i]
  // stored as [m][slice][i][lane] (16 bytes per lane and i: conflict-free reads)
  const int xsl = max_k / kChainSlice + 1;                                      // slice slots per row of X
  u32x4* xs = reinterpret_cast<u32x4*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)M * xsl * 4 * 64 * 16);   // [m][chunk]
  float* red = xsum + (size_t)M * (max_k / 32);                                  // [slice][row][m]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sw = wave - 1;
  uint16_t* glue = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(bar) + kChainHeaderBytes);                      // index of a streaming wave (waves 1 .. 15)
  const unsigned nblocks = gridDim.x;
  const int b = blockIdx.x;
  unsigned gen = 0;
  if (threadIdx.x == 0) gen = ld_coherent(bar + kGenWord0 + 16 * (blockIdx.x % kGenCopies));

  // descriptors read through the constant address space: wave-uniform
  // scalar loads, which wait on their own counter (a vector load here would
  // make the next wait drain the weight stream)
  CDesc* cdesc = (CDesc*)descs;
  // the block's rows of a linear: nb batches of R from row0 on; a paired
  // linear (pair > 0) has nb / 2 batches of gate rows from row0 and as many
  // of up rows from pair + row0, in that order
  auto block_rows = [&](int per_block, int rem, int pair, int& row0, int& nb) {
    nb = (per_block + (b < rem ? 1 : 0)) * (pair > 0 ? 2 : 1);
    row0 = R * (b * per_block + min(b, rem));
  };
  auto row_of = [&](int pair, int row0, int nb, int li) {   // global row of block-local row li
    return (pair > 0 && li >= R * (nb / 2)) ? pair + row0 + (li - R * (nb / 2)) : row0 + li;
  };

  // The weight stream of a streaming wave: its items of every linear in
  // chain order (item sw + k S of each linear, k = 0, 1, ...: a 4-row batch
  // and a 2048-input slice), kRing loads ahead of the products, in kRing
  // register buffers.  The cursor (cl, ck) names the next entry to load; it
  // runs ahead into the following linears, so the stream goes on through the
  // reduction, the grid barrier and the staging of the next input.  Entries
  // past the chain's end load the workspace header instead (valid memory,
  // values unused).  At a linear's start every load has landed, and the
  // buffers are rotated so that buffer 0 holds its first item; within the
  // linear each product then waits only for its own buffer.
  u32x4 cb[kRing][R];
  uint16_t sb[kRing];
  int zb[kRing];
  auto items_of = [&](int l) {
    const int nb = (cdesc[l].batches_per_block + (b < cdesc[l].batches_rem ? 1 : 0)) * (cdesc[l].pair > 0 ? 2 : 1);
    return nb * cdesc[l].slices;
  };
  auto entries_of = [&](int l) {
    const int items = items_of(l);
    return sw < items ? (items - sw + S - 1) / S : 0;
  };
  int cl = 0, ck = 0;
  auto settle = [&]() {
    while (cl < n_linears && ck >= entries_of(cl)) {
      cl += 1;
      ck = 0;
    }
  };
  auto stream_load = [&](int buf) {
    const u32x4* cbase = reinterpret_cast<const u32x4*>(bar) + lane;
    const uint16_t* sbase = reinterpret_cast<const uint16_t*>(bar);
    const int32_t* zbase = reinterpret_cast<const int32_t*>(bar);
    int64_t vrow = 0, G = 0;
    int rowb = 0, nmax = 0, c4 = lane >> 2;
    const int it = sw + ck * S;
    if (cl < n_linears && it < items_of(cl)) {
      const int K = cdesc[cl].K, slices = cdesc[cl].slices;
      int row0, nb;
      block_rows(cdesc[cl].batches_per_block, cdesc[cl].batches_rem, cdesc[cl].pair, row0, nb);
      const int batch = it / slices, sl = it - batch * slices;
      const int c = min(sl * 64 + lane, K / 32 - 1);   // inactive lanes read valid memory
      vrow = K / 32;
      G = K / kGroup;
      rowb = row_of(cdesc[cl].pair, row0, nb, batch * R);   // a batch never straddles the halves
      nmax = cdesc[cl].N - 1;
      c4 = c / 4;
      cbase = reinterpret_cast<const u32x4*>(cdesc[cl].codes) + c;
      sbase = cdesc[cl].scales;
      zbase = cdesc[cl].zeros;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) cb[buf][j] = __builtin_nontemporal_load(cbase + (int64_t)min(rowb + j, nmax) * vrow);
    const int64_t mi = (int64_t)min(rowb + (lane & 3), nmax) * G + c4;
    sb[buf] = sbase[mi];
    zb[buf] = zbase[mi];
    ck += 1;
    settle();
  };

  if (wave > 0) {
    settle();
    static_for<0, kRing>([&](auto j) { stream_load(decltype(j)::value); });
  }
  int phase = 0;   // buffer of the oldest entry in flight

  for (int l = 0; l < n_linears; ++l) {
    const ChainDesc d = descs[l];
    const ChainDesc* prev = l > 0 ? descs + (l - 1) : nullptr;
    int row0, nb;
    block_rows(d.batches_per_block, d.batches_rem, d.pair, row0, nb);
    const int items = nb * d.slices;
    // a paired producer: wave 0 fetches the next producer weight of its
    // first two passes of gate-row pairs now, while it has nothing in flight
    const int half = R * (nb / 2);
    const uint16_t* gnext = d.pair > 0 ? descs[l + 1].gamma : nullptr;
    uint32_t gpre[2] = {0x3F803F80u, 0x3F803F80u};   // BF16 (1, 1) without a producer weight
    if (wave == 0 && gnext) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = lane + 64 * q;
        if (e < (half / 2) * M) gpre[q] = *reinterpret_cast<const uint32_t*>(gnext + row0 + 2 * (e / M));
      }
    }

    // ---- stage X_l: octets (8 inputs) of the activation rows, kStageU per
    // thread and pass with all their loads issued first; the four lanes of a
    // 32-input chunk add their sums
    const int octs = d.K / 8;
    // every block reads the whole input at the same moment: each starts at
    // its own 32-input chunk (block-dependent rotation) so that the blocks
    // spread over the memory channels
    const int shift = 4 * ((b * 37) % (octs / 4));
    auto octet_of = [&](int e, int& m, int& o) {
      m = e / octs;
      o = e - m * octs + shift;
      if (o >= octs) o -= octs;
    };
    auto stage = [&](auto kind_c) {
      constexpr int KIND = decltype(kind_c)::value;
      for (int e0 = threadIdx.x; e0 < M * octs; e0 += kStageU * kChainThreads) {
        uint64_t w[kStageU][4];
        u32x4 gw[kStageU];
        static_for<0, kStageU>([&](auto uu) {
          constexpr int u = decltype(uu)::value;
          const int e = e0 + u * kChainThreads;
          if (e < M * octs) {
            int m, o;
            octet_of(e, m, o);
            if constexpr (KIND >= 0) fetch_octet<KIND>(d, prev, X0, ldx, glue, m, o, w[u]);
            if (KIND != kGlued && d.gamma) gw[u] = *reinterpret_cast<const u32x4*>(d.gamma + 8 * o);
          }
        });
        static_for<0, kStageU>([&](auto uu) {
          constexpr int u = decltype(uu)::value;
          const int e = e0 + u * kChainThreads;
          if (e < M * octs) {
            int m, o;
            octet_of(e, m, o);
            float v[8];
            form_octet<KIND>(d, prev, m, o, w[u], v);
            if (KIND != kGlued && d.gamma) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                v[2 * j] *= lo16(gw[u][j]);
                v[2 * j + 1] *= hi16(gw[u][j]);
              }
            }
            u32x4 raw;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              raw[j] = (uint32_t)f32_to_bf16_rne(v[2 * j]) | ((uint32_t)f32_to_bf16_rne(v[2 * j + 1]) << 16);
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) sum = dot2(raw[j], kOnePair, sum);
            sum += dpp<kDppXor1>(sum);
            sum += dpp<kDppXor2>(sum);
            const int c = o >> 2, i = o & 3, sl = c >> 6, ln = c & 63;
            xs[((size_t)(m * xsl + sl) * 4 + i) * 64 + ln] = x_pairs_from_natural(raw);
            if (i == 0) xsum[m * (max_k / 32) + c] = sum;
          }
        });
      }
    };
    if (d.input == W4A16_CHAIN_X0) stage(Ic<W4A16_CHAIN_X0>{});
    else if (d.input == W4A16_CHAIN_PREV) stage(Ic<W4A16_CHAIN_PREV>{});
    else if (d.input == W4A16_CHAIN_SWIGLU) {
      if (d.glued) stage(Ic<kGlued>{});
      else stage(Ic<W4A16_CHAIN_SWIGLU>{});
    }
    else if (attn_octets(d)) stage(Ic<W4A16_CHAIN_ATTN1>{});
    else stage(Ic<-1>{});
    block_sync_lds();

    // ---- the block's rows: items (4-row batch, 2048-input slice)
    auto compute = [&](int buf, int it) {
      const int batch = it / d.slices, sl = it - batch * d.slices;
      const int chunks = d.K / 32;
      const int c = sl * 64 + lane;
      const bool active = c < chunks;
      u32x4 xp[M][4];
      float xsg[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 v = xs[((size_t)(m * xsl + sl) * 4 + i) * 64 + lane];
          if (!active) v = u32x4{0u, 0u, 0u, 0u};
          xp[m][i] = v;
        }
        if (active) s = xsum[m * (max_k / 32) + c];
        s += dpp<kDppXor1>(s);
        xsg[m] = s + dpp<kDppXor2>(s);
      }
      float P[R][M];
#pragma unroll
      for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int m = 0; m < M; ++m) P[j][m] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 q = codes_to_bias128_pairs(cb[buf][j][i]);
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) P[j][m] = dot2(q[jj], xp[m][i][jj], P[j][m]);
        }
      }
      // sum over the four lanes of a group, lane l keeping row l % 4 ...
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
        const float s = bf16_to_f32(sb[buf]);
        const float zb128 = (float)zb[buf] + 128.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float q = pick(up, h[1][m] + dpp<kDppXor1>(h[1][m]), h[0][m] + dpp<kDppXor1>(h[0][m]));
          // ... and removes the bias and zero point of that (row, group)
          part[m] = s * fmaf(-zb128, xsg[m], q);
        }
#pragma unroll
        for (int m = M; m < MP; ++m) part[m] = 0.f;
      }
      // then over the 16 groups of the slice (lane bits 2..5)
      lane_tree_sum<MP, MP == 1 ? 0 : 1>(part, lane);
      int m;
      if (tree_result<MP, MP == 1 ? 0 : 1>(lane, m) && m < M)
        red[((size_t)sl * max_rows + batch * R + (lane & 3)) * M + m] = part[0];
    };
    if (wave > 0) {
      // the prefetched items have landed behind the staging loads (or are
      // waited for here, in waves that staged nothing)
      wait_vmcnt<0>();
      // rotate the ring so that buffer 0 holds the oldest entry
      static_for<1, kRing>([&](auto rr) {
        constexpr int r = decltype(rr)::value;
        if (phase == r) {
          u32x4 tc[kRing][R];
          uint16_t ts[kRing];
          int tz[kRing];
#pragma unroll
          for (int j = 0; j < kRing; ++j) {
#pragma unroll
            for (int q = 0; q < R; ++q) tc[j][q] = cb[(j + r) % kRing][q];
            ts[j] = sb[(j + r) % kRing];
            tz[j] = zb[(j + r) % kRing];
          }
#pragma unroll
          for (int j = 0; j < kRing; ++j) {
#pragma unroll
            for (int q = 0; q < R; ++q) cb[j][q] = tc[j][q];
            sb[j] = ts[j];
            zb[j] = tz[j];
          }
        }
      });
      int it = sw;
      for (; it + (kRing - 1) * S < items; it += kRing * S) {
        static_for<0, kRing>([&](auto jj) {
          constexpr int j = decltype(jj)::value;
          compute(j, it + j * S);
          stream_load(j);
        });
      }
      // the last, partial round: its buffers are refilled, the rest keep
      // entries of the following linears, and the oldest entry is then in
      // buffer `phase`
      phase = 0;
      static_for<0, kRing - 1>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        if (it + j * S < items) {
          compute(j, it + j * S);
          stream_load(j);
          phase = j + 1;
        }
      });
    }
    block_sync_lds();

    // ---- wave 0: the K slices of each row in a fixed order, BF16 store of
    // row pairs as coherent 32-bit stores (rows start at a multiple of 4; an
    // odd last row of the linear updates its half of the word atomically),
    // then the grid barrier; the streaming waves wait at the block barrier
    // with their next loads in flight
    if (wave == 0 && d.pair > 0) {
      // paired rows, per pass a pair of gate rows r, r + 1 and their up rows:
      // the four outputs stored, and the next input k = row0 + r, r + 1
      // formed from the stored BF16 values (silu(g) u times the next
      // producer weight, the float32 steps of the SwiGLU staging, rounded to
      // BF16) into the glue region [m][pair]
      auto row_value = [&](int r, int m) {
        float v = red[(size_t)r * M + m];
        for (int sl = 1; sl < d.slices; ++sl) v += red[((size_t)sl * max_rows + r) * M + m];
        return (uint32_t)f32_to_bf16_rne(v);
      };
      auto swiglu = [&](uint32_t gb, uint32_t ub, float gamma) {
        const float g = bf16_to_f32(gb), u = bf16_to_f32(ub);
        float v = g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
        if (gnext) v *= gamma;
        return (uint32_t)f32_to_bf16_rne(v);
      };
      unsigned* gwords = reinterpret_cast<unsigned*>(glue);
      int q = 0;
      for (int e = lane; e < (half / 2) * M; e += 64, ++q) {
        const int r = 2 * (e / M), m = e - (e / M) * M;
        const uint32_t g0 = row_value(r, m), g1 = row_value(r + 1, m);
        const uint32_t u0 = row_value(half + r, m), u1 = row_value(half + r + 1, m);
        uint16_t* yrow = d.y + (int64_t)m * d.ldy;
        st_coherent(reinterpret_cast<unsigned*>(yrow + row0 + r), g0 | (g1 << 16));
        st_coherent(reinterpret_cast<unsigned*>(yrow + d.pair + row0 + r), u0 | (u1 << 16));
        const uint32_t gw = q == 0   ? gpre[0]
                            : q == 1 ? gpre[1]
                                     : (gnext ? *reinterpret_cast<const uint32_t*>(gnext + row0 + r) : 0x3F803F80u);
        st_coherent(gwords + ((int64_t)m * d.pair + row0 + r) / 2,
                    swiglu(g0, u0, lo16(gw)) | (swiglu(g1, u1, hi16(gw)) << 16));
      }
    } else if (wave == 0) {
      const int rows = min(R * nb, d.N - row0);
      auto row_value = [&](int r, int m) {
        float v = red[(size_t)r * M + m];
        for (int sl = 1; sl < d.slices; ++sl) v += red[((size_t)sl * max_rows + r) * M + m];
        return (uint32_t)f32_to_bf16_rne(v);
      };
      for (int e = lane; e < ((rows + 1) / 2) * M; e += 64) {
        const int r = 2 * (e / M), m = e - (e / M) * M;
        unsigned* yw = reinterpret_cast<unsigned*>(d.y + (int64_t)m * d.ldy + row0 + r);
        if (r + 1 < rows) {
          st_coherent(yw, row_value(r, m) | (row_value(r + 1, m) << 16));
        } else {
          __hip_atomic_fetch_and(yw, 0xFFFF0000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_fetch_or(yw, row_value(r, m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (l + 1 < n_linears) {
      // the block's stores (all in wave 0) are complete before it arrives:
      // a block barrier does not wait for global stores
      bool published = false;
      if (wave == 0) {
        wait_vmcnt<0>();
        published = grid_arrive(bar, nblocks, gen);
      }
      grid_wait(bar, gen, published, spin_limit);
      gen += 1u;
    }
  }
}

}  // namespace

// Launch one chain (the caller has validated the plan): M = 1 or 2, one
// block per CU.
int launch_chain(const void* descs, int n_linears, int M, const uint16_t* X0, int64_t ldx, unsigned* bar,
                 int spin_limit, int max_k, int max_rows, int grid, size_t lds_bytes, hipStream_t stream) {
  const ChainDesc* dd = reinterpret_cast<const ChainDesc*>(descs);
  if (M == 1) {
    static bool attr1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<1>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    if (!attr1) return 4;
    hipLaunchKernelGGL(chain_kernel<1>, dim3(grid), dim3(kChainThreads), lds_bytes, stream, dd, n_linears, X0, ldx,
                       bar, spin_limit, max_k, max_rows);
  } else {
    static bool attr2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_kernel<2>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    if (!attr2) return 4;
    hipLaunchKernelGGL(chain_kernel<2>, dim3(grid), dim3(kChainThreads), lds_bytes, stream, dd, n_linears, X0, ldx,
                       bar, spin_limit, max_k, max_rows);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// ---------------------------------------------------------------------------
// The same launch for callers that cannot allocate: barrier state and
// descriptors in a file-scope device array of fixed size (one copy per GPU,
// kept until the process ends; calls that overlap on one GPU race).
// ---------------------------------------------------------------------------

namespace {

constexpr int64_t kScratchBytes = kChainDescOffset + (int64_t)W4A16_CHAIN_NOALLOC_MAX_LINEARS * sizeof(ChainDesc);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each device, looked up once per device with
// that device current (the array's name is a host-side stand-in).
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// the barrier state must start at zero: a fill kernel (no memset node)
__global__ void clear_words_kernel(unsigned* p, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) p[i] = 0u;
}

}  // namespace

int launch_chain_noalloc(const ChainDesc* d, int n_linears, int M, const uint16_t* X0, int64_t ldx, int max_k,
                         int max_rows, int grid, size_t lds_bytes, int* status, hipStream_t stream) {
  char* ws = static_cast<char*>(scratch_address());
  if (!ws) return 4;
  // descriptors: the host copy (the caller's stack) must be consumed before
  // this call returns, so the copy is waited for
  if (hipMemcpyAsync(ws + kChainDescOffset, d, (size_t)n_linears * sizeof(ChainDesc), hipMemcpyHostToDevice,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return 4;
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, reinterpret_cast<unsigned*>(ws),
                     (int)(kChainHeaderBytes / 4));
  if (hipGetLastError() != hipSuccess) return 4;
  if (int st = launch_chain(ws + kChainDescOffset, n_linears, M, X0, ldx, reinterpret_cast<unsigned*>(ws),
                            W4A16_CHAIN_SPIN_LIMIT, max_k, max_rows, grid, lds_bytes, stream))
    return st;
  if (status) {
    unsigned v = 0;
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpy(&v, ws + kChainStatusWord * 4, 4, hipMemcpyDeviceToHost) != hipSuccess)
      return 4;
    *status = (int)v;
  }
  return 0;
}

}  // namespace w4a16
