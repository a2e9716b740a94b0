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
 *   library allocates nothing and keeps no mutable global state.
 * - BF16 values are passed as their uint16_t bit patterns.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *   default stream).  It returns once the work is enqueued; buffers must stay
 *   alive until the stream has passed the work.
 * - Argument checks are synchronous and happen before anything is launched;
 *   on any error nothing is written.  Launch failures return W4A16_ERR_HIP.
 *   Faults inside a kernel surface at the caller's next synchronisation.
 * - Inputs are finite; non-finite weights or activations give undefined
 *   (but memory-safe) results.
 * - Results are deterministic: no atomics; the same inputs give the same bits.
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
#define W4A16_ABI_VERSION 6
#define W4A16_GEMV_MAX_M 32
#define W4A16_DENSE_GEMV_MAX_M 8
#define W4A16_INT8_GEMV_MAX_M 4
#define W4A16_INT8_GEMV_MAX_K 32768

enum {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad leading dimension */
  W4A16_ERR_MISALIGNED = 2,  /* a pointer or leading dimension breaks an alignment rule */
  W4A16_ERR_UNSUPPORTED = 3, /* no gfx950 device, or a size beyond a documented limit */
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
 */
int w4a16_gemv(const uint16_t* X, int64_t M, int64_t ldx,
               const uint32_t* codes, const uint16_t* scales,
               const int32_t* zeros, int64_t N, int64_t K,
               uint16_t* Y, int64_t ldy, void* stream);

/*
 * w4a16_gemm -- prefill-shaped fused dequantise-multiply on the BF16 matrix
 * cores, any M >= 1 (tuned for M >= 256).  Same arguments, layout, accuracy
 * and alignment rules as w4a16_gemv, without the limit on M.  The
 * dequantised weights feed the matrix cores as exact small integers and the
 * group scale is applied in float32, so no weight is ever rounded.
 */
int w4a16_gemm(const uint16_t* X, int64_t M, int64_t ldx,
               const uint32_t* codes, const uint16_t* scales,
               const int32_t* zeros, int64_t N, int64_t K,
               uint16_t* Y, int64_t ldy, void* stream);

/*
 * w4a16_pack_grouped, w4a16_gemv_grouped, w4a16_gemm_grouped -- the same
 * three operations with a group of `group` consecutive inputs per scale and
 * zero point, group = 32, 64 or 128 (the group sizes "Quantization I",
 * "Concept", and Zeno AGI, "Weight-only vs mixed precision" (its summary of
 * common settings) name; 128 gives exactly w4a16_pack / w4a16_gemv /
 * w4a16_gemm).  scales and zeros are [N][K/group]; K must still be a
 * multiple of 128.  The quantiser rules of w4a16_pack apply per group; the
 * matmuls keep the accuracy rules of w4a16_gemv / w4a16_gemm.  For group 32
 * and 64 the matmuls also require scales and zeros 16-byte aligned.
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
 * with the rules of w4a16_gemm.
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
 * w4a16_dense_gemv without the limit on M.
 */
int w4a16_dense_gemm(const uint16_t* X, int64_t M, int64_t ldx,
                     const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                     uint16_t* Y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
