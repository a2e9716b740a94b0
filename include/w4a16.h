/*
 * w4a16.h -- C ABI of the fused INT4 weight-only (W4A16) matmul library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (Axe Corsa model card, "The Two-Stage Pipeline"):
 *
 *     Y[m, n] = sum_k X[m, k] * w_hat[n, k],
 *     w_hat[n, k] = (q[n, k] - z[n, g]) * s[n, g],   g = k / 128,
 *
 * with q an unsigned 4-bit code, s a BF16 scale and z an INT32 zero point,
 * one (s, z) pair per group of 128 consecutive input channels ("What the
 * Tensor Types Tell You").  X and Y are BF16.  Dequantisation happens in
 * registers inside the multiply, so only the packed codes and the group
 * metadata are read from memory ("Quantization I: int8, int4, the basics",
 * "Concept": dequantise tile by tile inside the multiply).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers (memory of the current HIP device) unless a
 *   comment says otherwise.  The caller allocates and frees every buffer; the
 *   library allocates no memory at run time.  Its only global state is a
 *   per-device record of the architecture check and the fixed device array
 *   of w4a16_chain_run_noalloc.
 * - BF16 values are passed as their uint16_t bit patterns.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *   default stream).  It returns once the work is enqueued; buffers must stay
 *   alive until the stream has passed the work.
 * - Argument checks are synchronous and happen before anything is launched;
 *   on any error nothing is written.  Launch failures return W4A16_ERR_HIP.
 *   Faults inside a kernel surface at the caller's next synchronisation.
 * - Inputs are finite; non-finite weights or activations give undefined
 *   (but memory-safe) results.
 * - The matmuls accept any finite BF16 scale -- zero, negative and subnormal
 *   ones included, which the packers never write but a container read in
 *   place may hold -- and any int32 zero point, in any sequence along a row,
 *   with the accuracy stated for each entry point.
 * - Every size (M, N, K, T) must be below W4A16_MAX_DIM = 2^30; larger
 *   sizes return W4A16_ERR_UNSUPPORTED.
 * - The kernels are built for gfx950 only: an entry point whose arguments
 *   pass the checks returns W4A16_ERR_UNSUPPORTED when the current HIP
 *   device is not a gfx950 GPU (or there is no device).
 * - Results are deterministic: the same inputs give the same bits.  (The
 *   paths that split K over blocks, and the chain, count arrivals with
 *   atomics but add their partial sums in a fixed order.)
 *
 * Storage layout of a packed weight matrix with N outputs and K inputs
 * (K a multiple of 128):
 *   codes  uint32_t [N][K/8]  nibble j (bits 4j..4j+3) of word i of row n is
 *                             q[n, 8i + j]; read as bytes (little endian)
 *                             each byte holds two consecutive codes, low
 *                             nibble first -- the two-codes-per-byte stream of
 *                             the compressed-tensors format ("What the Tensor
 *                             Types Tell You").  16-byte aligned.  The
 *                             same bytes viewed as int64 [N][K/16] are that
 *                             format's I64 container, so such a container
 *                             is consumed in place (no copy, no repacking).
 *   scales uint16_t [N][K/128] BF16 scale bits.
 *   zeros  int32_t  [N][K/128] zero points, not clamped to 0..15.
 * That is 4 + 16/128 + 32/128 = 4.375 bits per weight (Axe Corsa model card,
 * "Storage Cost").  The *_grouped entry points take groups of 32 or 64
 * inputs as well (scales and zeros then [N][K/group]; K stays a multiple of
 * 128).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_GROUP 128
#define W4A16_ABI_VERSION 10
#define W4A16_GEMV_MAX_M 32
#define W4A16_DENSE_GEMV_MAX_M 8
#define W4A16_INT8_GEMV_MAX_M 4
#define W4A16_INT8_GEMV_MAX_K 32768
#define W4A16_MAX_DIM ((int64_t)1 << 30)
/* Limits of the matrix-core GEMMs (32-bit per-tile offsets): ldx (and ldw of
   the dense GEMM) below W4A16_GEMM_MAX_LD, K below W4A16_GEMM_MAX_K. */
#define W4A16_GEMM_MAX_LD ((int64_t)1 << 23)
#define W4A16_GEMM_MAX_K ((int64_t)1 << 25)

enum {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad leading dimension */
  W4A16_ERR_MISALIGNED = 2,  /* a pointer or leading dimension breaks an alignment rule */
  W4A16_ERR_UNSUPPORTED = 3, /* the current device is not gfx950, or a size beyond a documented limit */
  W4A16_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
};

/* W4A16_ABI_VERSION of the loaded library. */
int w4a16_abi_version(void);

/* Static description of a status code (never NULL). */
const char* w4a16_strerror(int status);

/*
 * w4a16_pack -- group-wise asymmetric round-to-nearest quantise and pack
 * (Axe Corsa model card, "The Two-Stage Pipeline": asymmetric INT4, one
 * scale and one zero point per group of 128 consecutive weights;
 * "Quantization I", "Concept": zero point, rounding, clipping).
 *
 *   W      BF16 [N][ldw], row n holds the K input weights of output n.
 *   awq_s  optional float [K]; if not NULL the quantiser input is the
 *          float32 product W[n,k] * awq_s[k] (the AWQ rescaled weight
 *          W' = W diag(s), "Stage 1: Activation-Aware Weight Scaling").
 *   codes, scales, zeros  outputs in the layout above.
 *
 * Per group of 128 values w (float32 arithmetic, round to nearest even, no
 * fused multiply-add, denormals kept):
 *   D = max - min;  t = D / 15;  s = BF16 of t rounded toward zero;
 *   if s is zero or subnormal: s = BF16 toward zero of max(|min|, |max|),
 *       and 1.0 if that is still zero or subnormal;
 *   z = round_half_away_from_zero(-min / s)            (int32, unclamped);
 *   q = clamp(round_half_away_from_zero(w / s) + z, 0, 15).
 * The minimum of every group maps to code 0 and, when the group straddles
 * zero, the maximum to code 15: all 16 codes are used.
 *
 * Requires N >= 1, K >= 128, K % 128 == 0, ldw >= K; codes 16-byte aligned.
 * Results are bit-exact and independent of the launch configuration.
 */
int w4a16_pack(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
               const float* awq_s, uint32_t* codes, uint16_t* scales,
               int32_t* zeros, void* stream);

/*
 * w4a16_pack_symmetric -- the symmetric INT4 variant ("Quantization I",
 * "Concept", and the Axe Corsa model card, "The Two-Stage Pipeline", name it
 * and argue it wastes range; the formula on the pages is lost, this is the
 * reading used).  Same arguments, rules and output layout as w4a16_pack;
 * per group of 128 values w (float32, as above):
 *   A = max |w|;  s = BF16 of A / 7 rounded toward zero;
 *   if s is zero or subnormal: s = BF16 toward zero of A, and 1.0 if that
 *       is still zero or subnormal;
 *   z = 8;  q = clamp(round_half_away_from_zero(w / s) + 8, 0, 15).
 * Codes are 1..15 (signed -7..7 around the zero point 8), so every matmul
 * entry point consumes the result unchanged.  Bit-exact.
 */
int w4a16_pack_symmetric(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                         const float* awq_s, uint32_t* codes, uint16_t* scales,
                         int32_t* zeros, void* stream);

/*
 * w4a16_gemv -- decode-shaped fused dequantise-multiply, 1 <= M <= 32.
 *
 *   X      BF16 [M][ldx] activations (never quantised).
 *   codes, scales, zeros  a packed matrix with N outputs and K inputs.
 *   Y      BF16 [M][ldy] output, Y = X * w_hat^T.
 *
 * Products are accumulated in float32 and rounded once to BF16 (nearest
 * even) on store.  Requires 1 <= M <= 32, N >= 1, K >= 128, K % 128 == 0,
 * ldx >= K, ldy >= N; X 16-byte aligned and ldx % 8 == 0; codes 16-byte
 * aligned.  Y must not overlap the inputs.
 *
 * Accuracy (every matmul entry point).  No weight is rounded: per group the
 * kernels form s * (sum_k x (128 + q) - (128 + z) sum_k x) from exact
 * integer-valued BF16 operands in float32.  Besides half a BF16 ulp from the
 * store, an output therefore carries float32 rounding relative to
 * sum_g |s_g| (128 + |z_g|) |sum_{k in g} x_k|: far below the store's
 * rounding for ordinary groups, but for a group whose weights all
 * dequantise to zero (every q = z, such as the packer's all-zero groups,
 * scale 1.0) an absolute residue of order 2^-22 |s| 128 |sum x| that the
 * group's zero weights do not bound.
 */
int w4a16_gemv(const uint16_t* X, int64_t M, int64_t ldx,
               const uint32_t* codes, const uint16_t* scales,
               const int32_t* zeros, int64_t N, int64_t K,
               uint16_t* Y, int64_t ldy, void* stream);

/*
 * w4a16_gemv_workspace_bytes -- the workspace with which w4a16_gemv_ws may
 * split the K inputs of a row over several blocks for this shape (decode at
 * 9 <= M <= 32 with rows of more than 4096 inputs, at 3 <= M <= 8 with
 * rows of more than 8192 inputs); 0 when the shape needs none.  The size depends on the current device (its compute-unit count).
 * Returns W4A16_ERR_INVALID_ARG for shapes w4a16_gemv rejects.
 */
int w4a16_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t* bytes);

/*
 * w4a16_gemv_ws -- w4a16_gemv with a caller-owned workspace: same
 * arguments, layout, accuracy and limits, plus
 *
 *   workspace        device memory, 64-byte aligned, zero-filled before
 *                    its first use, not overlapping X, Y or the packed
 *                    matrix (W4A16_ERR_INVALID_ARG otherwise); may be NULL
 *                    with workspace_bytes 0.
 *   workspace_bytes  its size.
 *
 * With at least w4a16_gemv_workspace_bytes() bytes the decode kernel may
 * split K over blocks, whose float32 partial sums meet in the workspace (a
 * fixed summation order: results are deterministic, and may differ from
 * the unsplit kernel's in the last bits).  With less, or none, the call is
 * w4a16_gemv.  Each call leaves the workspace's counters at zero, so one
 * workspace serves any sequence of calls of any shapes on one stream; calls
 * that may run at the same time (other streams, concurrent graphs) need
 * workspaces of their own.
 */
int w4a16_gemv_ws(const uint16_t* X, int64_t M, int64_t ldx,
                  const uint32_t* codes, const uint16_t* scales,
                  const int32_t* zeros, int64_t N, int64_t K,
                  uint16_t* Y, int64_t ldy, void* workspace,
                  int64_t workspace_bytes, void* stream);

/*
 * w4a16_gemm -- prefill-shaped fused dequantise-multiply on the BF16 matrix
 * cores, any M >= 1 (tuned for M >= 256).  Same arguments, layout, accuracy
 * and alignment rules as w4a16_gemv, without the limit on M.  The
 * dequantised weights feed the matrix cores as exact integer-valued BF16
 * operands times a power of four, and the rest of each group's scale is
 * applied in float32, so no weight is ever rounded and consecutive groups'
 * scales may differ by any factor (a zero scale's group contributes at most
 * 2^-120 (128 + q) x per input, relative to the running unit of its row's
 * earlier scales).  Also requires ldx < W4A16_GEMM_MAX_LD,
 * K < W4A16_GEMM_MAX_K and ceil(M/64) * ceil(N/128) < 2^31, otherwise
 * W4A16_ERR_UNSUPPORTED.
 */
int w4a16_gemm(const uint16_t* X, int64_t M, int64_t ldx,
               const uint32_t* codes, const uint16_t* scales,
               const int32_t* zeros, int64_t N, int64_t K,
               uint16_t* Y, int64_t ldy, void* stream);

/*
 * w4a16_gemm_workspace_bytes -- the workspace with which w4a16_gemm_ws may
 * split the K inputs of each output tile over 2, 4 or 8 blocks for this
 * shape (when the shape has too few large output tiles to fill the device's
 * compute units, typically M up to ~2048; at most 128 MiB); 0 when it
 * splits nothing.  The size depends on the current device (its compute-unit
 * count).  Returns W4A16_ERR_INVALID_ARG for shapes w4a16_gemm rejects.
 */
int w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t* bytes);

/*
 * w4a16_gemm_ws -- w4a16_gemm with a caller-owned workspace: same
 * arguments, layout, limits and accuracy rules, plus
 *
 *   workspace        device memory, 16-byte aligned, not overlapping X, Y or
 *                    the packed matrix (W4A16_ERR_INVALID_ARG otherwise);
 *                    any contents (it holds float32 partial outputs during
 *                    the call); may be NULL with workspace_bytes 0.
 *   workspace_bytes  its size.
 *
 * With at least w4a16_gemm_workspace_bytes() bytes the product may split K:
 * each run's float32 partial tile goes to the workspace and a second launch
 * adds the runs in a fixed order and rounds once to BF16, so results are
 * deterministic (they may differ from the unsplit product's in the last
 * bit).  With less, or none, the call is w4a16_gemm.  Calls that may run at
 * the same time need workspaces of their own.
 */
int w4a16_gemm_ws(const uint16_t* X, int64_t M, int64_t ldx,
                  const uint32_t* codes, const uint16_t* scales,
                  const int32_t* zeros, int64_t N, int64_t K,
                  uint16_t* Y, int64_t ldy, void* workspace,
                  int64_t workspace_bytes, void* stream);

/*
 * w4a16_pack_grouped, w4a16_gemv_grouped, w4a16_gemm_grouped -- the same
 * three operations with a group of `group` consecutive inputs per scale and
 * zero point, group = 32, 64 or 128 (the group sizes "Quantization I",
 * "Concept", and Zeno AGI, "Weight-only vs mixed precision" (its summary of
 * common settings) name; 128 gives exactly w4a16_pack / w4a16_gemv /
 * w4a16_gemm).  scales and zeros are [N][K/group]; K must still be a
 * multiple of 128.  The quantiser rules of w4a16_pack apply per group; the
 * matmuls keep the accuracy rules of w4a16_gemv / w4a16_gemm (and the GEMM
 * limits of w4a16_gemm: w4a16_gemv_grouped runs the GEMM for M > 8).  For
 * group 32 and 64 the matmuls also require scales and zeros 16-byte aligned.
 * Any other group value: W4A16_ERR_INVALID_ARG.
 */
int w4a16_pack_grouped(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                       const float* awq_s, int64_t group, uint32_t* codes,
                       uint16_t* scales, int32_t* zeros, void* stream);
int w4a16_gemv_grouped(const uint16_t* X, int64_t M, int64_t ldx,
                       const uint32_t* codes, const uint16_t* scales,
                       const int32_t* zeros, int64_t N, int64_t K, int64_t group,
                       uint16_t* Y, int64_t ldy, void* stream);
int w4a16_gemm_grouped(const uint16_t* X, int64_t M, int64_t ldx,
                       const uint32_t* codes, const uint16_t* scales,
                       const int32_t* zeros, int64_t N, int64_t K, int64_t group,
                       uint16_t* Y, int64_t ldy, void* stream);

/*
 * w4a16_pack_int8, w4a16_gemv_int8, w4a16_gemm_int8 -- the W8A16 variant (Zeno AGI, "Weight-
 * only vs mixed precision", its precision matrix: 8-bit weights, 16-bit
 * activations).  Codes are 8-bit, four per word: codes uint32_t [N][K/4],
 * byte j of word i of row n is q[n, 4i + j] (the byte stream is q row by
 * row); scales and zeros as above (groups of 128).  The quantiser is
 * w4a16_pack's with 255 steps: t = D / 255 and q = clamp(..., 0, 255).
 * w4a16_gemv_int8 is the decode product for 1 <= M <= W4A16_INT8_GEMV_MAX_M
 * and K <= W4A16_INT8_GEMV_MAX_K (larger K: W4A16_ERR_UNSUPPORTED), with the
 * accuracy and alignment rules of w4a16_gemv; each code's two nibbles feed
 * the matrix product as exact BF16 operands, so no weight is rounded.
 * w4a16_gemm_int8 is the prefill product on the matrix cores, any M >= 1,
 * with the rules and limits of w4a16_gemm.
 */
int w4a16_pack_int8(const uint16_t* W, int64_t N, int64_t K, int64_t ldw,
                    const float* awq_s, uint32_t* codes, uint16_t* scales,
                    int32_t* zeros, void* stream);
int w4a16_gemv_int8(const uint16_t* X, int64_t M, int64_t ldx,
                    const uint32_t* codes, const uint16_t* scales,
                    const int32_t* zeros, int64_t N, int64_t K,
                    uint16_t* Y, int64_t ldy, void* stream);
int w4a16_gemm_int8(const uint16_t* X, int64_t M, int64_t ldx,
                    const uint32_t* codes, const uint16_t* scales,
                    const int32_t* zeros, int64_t N, int64_t K,
                    uint16_t* Y, int64_t ldy, void* stream);

/*
 * w4a16_awq_importance -- per-input-channel activation magnitude from a
 * calibration batch, importance[k] = (1/T) sum_t |Xcal[t, k]| (the reading
 * of the importance score in the Axe Corsa model card, "Stage 1").
 *   Xcal  BF16 [T][ldx];  importance  float [K].
 * Summed in float64 in a fixed order, rounded once to float32.
 * Requires T >= 1, K >= 1, ldx >= K.
 */
int w4a16_awq_importance(const uint16_t* Xcal, int64_t T, int64_t K,
                         int64_t ldx, float* importance, void* stream);

/*
 * w4a16_awq_scale -- AWQ smoothing scale s[k] = importance[k] ** alpha
 * (Axe Corsa model card, "Stage 1"), evaluated in float64 and rounded to
 * float32.  alpha in [0, 1]; importance must be positive.
 */
int w4a16_awq_scale(const float* importance, int64_t K, float alpha,
                    float* s, void* stream);

/*
 * w4a16_awq_fold -- absorb X' = diag(s)^-1 X into the producer's
 * per-channel weight and bias (Axe Corsa model card, "Stage 1": the
 * division is folded into the preceding LayerNorm, so it costs nothing at
 * run time):  gamma[k] = BF16_rne(gamma[k] / s[k]), and beta likewise when
 * beta is not NULL.  In place.  Requires K >= 1.
 */
int w4a16_awq_fold(const float* s, int64_t K, uint16_t* gamma,
                   uint16_t* beta, void* stream);

/*
 * w4a16_scale_channels -- the producer's per-channel multiply with a folded
 * weight: Xout[m, k] = BF16_rne(X[m, k] * gamma[k]) (float32 product).
 * Used to form the activations X' that meet AWQ-rescaled weights.
 * Requires M >= 1, K >= 1, ldx >= K, ldo >= K.  Xout may equal X.
 */
int w4a16_scale_channels(const uint16_t* X, int64_t M, int64_t K,
                         int64_t ldx, const uint16_t* gamma, uint16_t* Xout,
                         int64_t ldo, void* stream);

/*
 * w4a16_awq_search_error -- the objective of AWQ's exponent search (Axe
 * Corsa model card, "Stage 1: Activation-Aware Weight Scaling"; cyankiwi
 * Quantization docs, "The Baseline: AWQ": a light grid search over the
 * exponent, scored by the layer's output error): the relative L2 distance
 *   err[0] = sqrt( sum_{m,n} (Y[m,n] - Yref[m,n])^2 / sum_{m,n} Yref[m,n]^2 )
 * between two BF16 outputs Y [M][ldy] and Yref [M][ldr] (for example the
 * quantised layer's and the dense layer's).  Sums in float64 in a fixed
 * order (deterministic); an all-zero Yref gives inf or NaN.  err is one
 * double in device memory, 8-byte aligned.  Runs as one workgroup: meant for
 * calibration, not the inference path.  Requires M, N >= 1, ldy >= N,
 * ldr >= N.
 */
int w4a16_awq_search_error(const uint16_t* Y, int64_t ldy, const uint16_t* Yref,
                           int64_t ldr, int64_t M, int64_t N, double* err,
                           void* stream);

/*
 * Decode of a chain of dependent linears in one persistent launch.
 *
 * A decoder's weight stream is a chain: each linear's input is formed from
 * the previous linear's output.  Run one launch per linear, each launch pays
 * its dispatch, ramp and tail and nothing streams in between (Zeno AGI,
 * "Weight-only vs mixed precision", "7. The Marlin Kernel": round trips
 * between kernels eat the benefit of the fused matmul).  w4a16_chain_run
 * runs a whole chain in one launch: one block per CU (all resident), the rows
 * of each linear spread over all blocks, a grid barrier between consecutive
 * linears, the next linear's first weights already streaming through it.
 *
 * Linear l computes Y_l = X_l * w_hat_l^T (the arithmetic and accuracy of
 * w4a16_gemv, groups of 128) with X_l [M][K_l] formed from the previous
 * stored output Y_{l-1} (BF16) by its input kind, times gamma when given
 * (float32 product), rounded once to BF16 (nearest even):
 *   W4A16_CHAIN_X0      X_l[m,k] = X0[m,k] (the chain's input);
 *   W4A16_CHAIN_PREV    X_l[m,k] = Y_{l-1}[m,k];
 *   W4A16_CHAIN_SWIGLU  X_l[m,k] = silu(Y_{l-1}[m,k]) * Y_{l-1}[m,K+k], the
 *                       previous output holding [gate | up];
 *                       silu(g) = g / (1 + exp(-g)) in float32;
 *   W4A16_CHAIN_ATTN1   attention over a one-token context (the softmax of a
 *                       single score is 1, so each head returns its value
 *                       vector): X_l[m, h*head_dim + d] =
 *                       Y_{l-1}[m, v_offset + (h / group)*head_dim + d].
 * gamma is the producer's per-input-channel weight into which an AWQ scale is
 * folded (Axe Corsa model card, "Stage 1: Activation-Aware Weight Scaling").
 */
enum {
  W4A16_CHAIN_X0 = 0,
  W4A16_CHAIN_PREV = 1,
  W4A16_CHAIN_SWIGLU = 2,
  W4A16_CHAIN_ATTN1 = 3
};
#define W4A16_CHAIN_MAX_M 2
#define W4A16_CHAIN_MAX_LINEARS 1024
#define W4A16_CHAIN_MAX_K 32768
#define W4A16_CHAIN_SPIN_LIMIT (1 << 22)   /* default polls of a barrier wait */
#define W4A16_CHAIN_TIMEOUT 1              /* status: a barrier wait gave up */

/* One linear of a chain (host memory; the pointers are device pointers). */
typedef struct {
  const uint32_t* codes;    /* packed matrix, N outputs, K inputs, groups of 128 */
  const uint16_t* scales;
  const int32_t* zeros;
  const uint16_t* gamma;    /* optional BF16 [K] producer weight, NULL for none; 16-byte aligned */
  uint16_t* Y;              /* BF16 [M][ldy] output; 16-byte aligned, ldy % 8 == 0 */
  int64_t N, K, ldy;
  int32_t input;            /* W4A16_CHAIN_*; linear 0 must take W4A16_CHAIN_X0 */
  int32_t v_offset, head_dim, group;   /* W4A16_CHAIN_ATTN1 only */
} w4a16_chain_linear;

/* What w4a16_chain_prepare hands to w4a16_chain_run: plain data, caller
   owned.  spin_limit may be lowered by the caller (it bounds every barrier
   wait; W4A16_CHAIN_SPIN_LIMIT polls of about 50 ns by default). */
typedef struct {
  void* workspace;
  int32_t n_linears, M, grid, max_k, max_rows, k0;
  int32_t spin_limit, reserved;
  int64_t lds_bytes;
} w4a16_chain_plan;

/* Device workspace bytes for a chain of n_linears (barrier state, status
   word, a 128 KiB region where a linear whose output is exactly [gate | up]
   of a SwiGLU input leaves that input formed, the descriptors). */
int w4a16_chain_workspace_bytes(int n_linears, int64_t* bytes);

/*
 * w4a16_chain_prepare -- check a chain (host array of n_linears linears),
 * write its descriptors into `workspace` (device memory, 256-byte aligned,
 * at least w4a16_chain_workspace_bytes; it must stay allocated while the
 * plan is used, and not be shared by two plans run concurrently) and fill
 * *plan.  Synchronous: returns after the copy on `stream` completed, so the
 * host array may be freed.  Requires 1 <= M <= W4A16_CHAIN_MAX_M, every K a
 * multiple of 128 up to W4A16_CHAIN_MAX_K, inputs consistent with the
 * previous linear's N (PREV: K <= N_{l-1}; SWIGLU: 2K <= N_{l-1}; ATTN1:
 * K % head_dim == 0 and the gathered values inside N_{l-1}), outputs not
 * overlapping any input; the LDS the plan needs must fit a CU (status 3).
 */
int w4a16_chain_prepare(const w4a16_chain_linear* linears, int n_linears, int64_t M,
                        void* workspace, int64_t workspace_bytes,
                        w4a16_chain_plan* plan, void* stream);

/*
 * w4a16_chain_run -- run a prepared chain on X0 (BF16 [M][ldx], 16-byte
 * aligned, ldx % 8 == 0, ldx >= the largest K of the linears that take
 * W4A16_CHAIN_X0), asynchronously on `stream`, in one launch of one block
 * per compute unit (all resident at once).
 * Every Y_l is written.  Deterministic.
 */
int w4a16_chain_run(const w4a16_chain_plan* plan, const uint16_t* X0, int64_t ldx, void* stream);

/*
 * w4a16_chain_status -- synchronise `stream`, then report the plan's status
 * word and clear the workspace's barrier state: 0, or W4A16_CHAIN_TIMEOUT if
 * a barrier wait of a run since the last call gave up (that run's outputs
 * are not valid, and the barrier state must be cleared by this call before
 * the next run).  Synchronous.
 */
int w4a16_chain_status(const w4a16_chain_plan* plan, int* status, void* stream);

/*
 * w4a16_chain_run_noalloc -- prepare and run a chain in one call without
 * allocating or taking a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid it).  Same chain rules and results as w4a16_chain_prepare +
 * w4a16_chain_run; the barrier state, the SwiGLU input region and the
 * descriptors live in a fixed device array inside the library (about 155
 * KiB, one per GPU, kept until the process ends), so
 * at most W4A16_CHAIN_NOALLOC_MAX_LINEARS linears (more:
 * W4A16_ERR_UNSUPPORTED), and calls that overlap on one GPU race (the
 * caller serialises them, e.g. on one stream).  The descriptors are copied
 * from the call's own stack and the copy is waited for before the launch;
 * the chain then runs asynchronously.  If status is not NULL the call also
 * waits for the run and stores 0 or W4A16_CHAIN_TIMEOUT there.
 */
#define W4A16_CHAIN_NOALLOC_MAX_LINEARS 256
int w4a16_chain_run_noalloc(const w4a16_chain_linear* linears, int n_linears, int64_t M,
                            const uint16_t* X0, int64_t ldx, int* status, void* stream);

/*
 * w4a16_hbm_read_probe -- measurement helper, not part of the matmul path:
 * reads `bytes` of device memory at buf with fully coalesced 16-byte loads
 * (each wave instruction covers 1 KiB of consecutive bytes, several loads in
 * flight per lane) and discards the data (sink, one uint32 in device memory,
 * is written only for one particular XOR of the contents).  Timed over a
 * buffer much larger than the last-level cache it gives the streaming-read
 * ceiling the decode kernels are compared with, beside the specification's
 * peak.  Requires bytes >= 16, bytes % 16 == 0, buf 16-byte aligned.
 */
int w4a16_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Dense BF16 comparisons.  Not part of the fused path: they measure the
 * alternatives it is chosen over (Zeno AGI, "Weight-only vs mixed
 * precision": the table of offline versus fused dequantisation, the naive
 * three-kernel pipeline of "7. The Marlin Kernel", and the dense 16-bit
 * layer of "1. The Basic Recipe") at the same shapes.
 *
 * w4a16_dequantize_bf16 -- expand a packed matrix to dense BF16:
 *   W[n, k] = BF16_rne(fl32(fl32(q[n, k] - z[n, g]) * s[n, g])), g = k / 128,
 * i.e. the float32 product rounded once to BF16 (the pages fix no precision
 * for an offline expansion).  Unlike the fused kernels this rounds every
 * weight.  codes, scales, zeros as for w4a16_gemv; W BF16 [N][ldw] output,
 * 16-byte aligned, ldw % 8 == 0, ldw >= K.  Requires N >= 1, K >= 128,
 * K % 128 == 0, and |q - z| < 2^31.  Bit-exact.
 */
int w4a16_dequantize_bf16(const uint32_t* codes, const uint16_t* scales,
                          const int32_t* zeros, int64_t N, int64_t K,
                          uint16_t* W, int64_t ldw, void* stream);

/*
 * w4a16_dense_gemv -- dense BF16 decode-shaped Y = X * W^T,
 * 1 <= M <= W4A16_DENSE_GEMV_MAX_M (8).
 *   X  BF16 [M][ldx];  W  BF16 [N][ldw], row n the K input weights of
 *   output n;  Y  BF16 [M][ldy].
 * Exact BF16 products accumulated in float32, rounded once to BF16 (nearest
 * even).  Requires N >= 1, K >= 128, K % 128 == 0, ldx >= K, ldw >= K,
 * ldy >= N; X and W 16-byte aligned, ldx % 8 == 0, ldw % 8 == 0.
 */
int w4a16_dense_gemv(const uint16_t* X, int64_t M, int64_t ldx,
                     const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                     uint16_t* Y, int64_t ldy, void* stream);

/*
 * w4a16_dense_gemm -- dense BF16 prefill-shaped Y = X * W^T on the matrix
 * cores, any M >= 1.  Same arguments, accuracy and rules as
 * w4a16_dense_gemv without the limit on M; also requires ldx and ldw below
 * W4A16_GEMM_MAX_LD and ceil(M/256) * ceil(N/256) < 2^31, otherwise
 * W4A16_ERR_UNSUPPORTED.
 */
int w4a16_dense_gemm(const uint16_t* X, int64_t M, int64_t ldx,
                     const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                     uint16_t* Y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
