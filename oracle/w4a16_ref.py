"""Plain, slow CPU oracle for the fused W4A16 weight-only matmul.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP library and never reads
anything the library produced except for the values it is compared against.

What it computes, and where each step comes from (page titles and sections of
the source pages):

* Group-wise asymmetric INT4 quantisation, one BF16 scale and one INT32 zero
  point per group of 128 consecutive K-weights -- Axe Corsa model card,
  "The Two-Stage Pipeline" (asymmetric scheme, groups of 128) and "What the
  Tensor Types Tell You" (BF16 scales, I32 zero points, packed INT4 codes).
* The scale/zero/code rule is the affine min/max round-to-nearest quantiser
  ("Quantization I: int8, int4, the basics", "Concept": a zero point shifts
  the range, rounding maps nearby reals to one code, clipping maps extremes
  to the boundary).  Where the pages leave a choice open (fp32 arithmetic,
  BF16 rounding of the scale toward zero, rounding half away from zero, the
  unclamped integer zero point, degenerate groups, nibble order) the oracle
  follows the readings listed in the design notes; each function states its
  reading.
* Dequantisation w_hat = (q - z_g) * s_g -- Axe Corsa model card, "The
  Two-Stage Pipeline", inverse mapping equation.
* Y = X . W_hat^T accumulated in fp64 (the exact result up to fp64 rounding;
  the product accumulates in fp32 and stores BF16).
* AWQ: s_i = importance_i ** alpha, W' = W . diag(s), X' = diag(s)^-1 X folded
  into the producer -- Axe Corsa model card, "Stage 1: Activation-Aware Weight
  Scaling".
* Comparisons outside the fused path: the dense BF16 weights an offline
  dequantisation would store, and the dense BF16 product -- Zeno AGI,
  "Weight-only vs mixed precision" (offline-versus-fused table, "7. The
  Marlin Kernel").

Every function is deliberately unoptimised: explicit bit manipulation,
explicit rounding, float64 products.  Vectorisation over whole arrays with
numpy is used only to apply the same per-element definition everywhere.
"""

from __future__ import annotations

import numpy as np

GROUP = 128          # Axe Corsa model card, "The Two-Stage Pipeline": 128 weights per group
# Smaller groups the pages name as common settings ("Quantization I",
# "Concept"; Zeno AGI, "Weight-only vs mixed precision", its summary of
# settings): the same rules per group of 32 or 64.
GROUPS = (32, 64, 128)


def _group_of(K: int, n_groups: int) -> int:
    """Group size of a packed matrix from its shapes (K inputs, n_groups
    scales per row)."""
    if n_groups < 1 or K % n_groups or K // n_groups not in GROUPS:
        raise ValueError(f"K={K} with {n_groups} groups per row is not a group of {GROUPS}")
    return K // n_groups
QMAX = 15            # 16 representable unsigned INT4 codes, 0..15
QMAX8 = 255          # W8A16 variant: 256 unsigned INT8 codes, 0..255
FLT_MIN = np.float32(2.0 ** -126)


# ---------------------------------------------------------------------------
# BF16 <-> FP32 bit conversions (BF16 = upper 16 bits of an IEEE binary32)
# ---------------------------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rtz(x) -> np.ndarray:
    """float32 -> BF16 bits, rounding toward zero: keep the upper 16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 -> BF16 bits, round to nearest, ties to even; NaN -> 0x7FC0."""
    xf = np.asarray(x, dtype=np.float32)
    u = xf.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    return np.where(np.isnan(xf), np.uint16(0x7FC0), r).astype(np.uint16)


def round_half_away(v) -> np.ndarray:
    """Round half away from zero, sign(v) * floor(|v| + 1/2), evaluated in
    float64 (exact for every float32 input).  Returns float64 integers."""
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    return np.sign(v64) * np.floor(np.abs(v64) + 0.5)


# ---------------------------------------------------------------------------
# Quantise (scale, zero point, codes) for one matrix, group by group
# ---------------------------------------------------------------------------

def group_scale_zero(w_groups: np.ndarray, qmax: int = QMAX):
    """Scale and zero point of each group.

    w_groups: float32 [..., 128], the quantiser input of each group.
    Returns (s_bits uint16 [...], s float32 [...], z int64 [...]).

    Reading of the affine min/max rule (Quantization I, "Concept"; Axe Corsa
    model card, "The Two-Stage Pipeline": asymmetric, the grid floats to
    where the weights are, all 16 codes used):
      D = fl32(max - min); t = fl32(D / 15); s = bf16 of t rounded toward zero.
      Degenerate group (s zero or subnormal): s = bf16_rtz(max(|min|,|max|)),
      and 1.0 if that is still zero or subnormal.
      z = round_half_away(fl32(-min / s)), an unclamped integer (the zero point
      is an offset on the integer grid, "What the Tensor Types Tell You").
    """
    w = np.asarray(w_groups, dtype=np.float32)
    mn = w.min(axis=-1)
    mx = w.max(axis=-1)
    d = (mx - mn).astype(np.float32)
    t = (d / np.float32(qmax)).astype(np.float32)
    s_bits = f32_to_bf16_rtz(t)
    s = bf16_to_f32(s_bits)
    degenerate = s < FLT_MIN
    if np.any(degenerate):
        m = np.maximum(np.abs(mn), np.abs(mx)).astype(np.float32)
        alt_bits = f32_to_bf16_rtz(m)
        alt = bf16_to_f32(alt_bits)
        alt_bits = np.where(alt < FLT_MIN, np.uint16(0x3F80), alt_bits)  # 1.0
        s_bits = np.where(degenerate, alt_bits, s_bits).astype(np.uint16)
        s = bf16_to_f32(s_bits)
    neg_mn_over_s = (-mn / s).astype(np.float32)
    z = round_half_away(neg_mn_over_s).astype(np.int64)
    return s_bits, s, z


def group_codes(w_groups: np.ndarray, s: np.ndarray, z: np.ndarray, qmax: int = QMAX) -> np.ndarray:
    """Codes q = clamp(round_half_away(fl32(w / s)) + z, 0, 15), rounding
    against the stored BF16 scale (round-to-nearest on the grid used at
    dequantisation).  Clipping to the code range follows Quantization I,
    "Concept".  Returns uint8 [..., 128]."""
    w = np.asarray(w_groups, dtype=np.float32)
    ratio = (w / s[..., None]).astype(np.float32)
    r = round_half_away(ratio).astype(np.int64)
    q = np.clip(r + z[..., None], 0, qmax)
    return q.astype(np.uint8)


def quantize(W_bits: np.ndarray, awq_s: np.ndarray | None = None, group: int = GROUP):
    """Quantise a BF16 weight matrix W [N][K] (uint16 bits) group-wise, in
    groups of `group` consecutive inputs (32, 64 or 128).

    If awq_s (float32 [K]) is given, the quantiser input is
    fl32(W[n,k] * awq_s[k]) -- the AWQ rescaled weight W' = W . diag(s)
    (Axe Corsa model card, "Stage 1: Activation-Aware Weight Scaling").

    Returns (q uint8 [N][K], s_bits uint16 [N][K/group], z int32 [N][K/group]).
    """
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    if group not in GROUPS:
        raise ValueError(f"group must be one of {GROUPS}")
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = bf16_to_f32(W_bits)
    if awq_s is not None:
        w = (w * np.asarray(awq_s, dtype=np.float32)[None, :]).astype(np.float32)
    wg = w.reshape(N, K // group, group)
    s_bits, s, z = group_scale_zero(wg)
    q = group_codes(wg, s, z).reshape(N, K)
    if np.any(z > np.iinfo(np.int32).max) or np.any(z < np.iinfo(np.int32).min):
        raise OverflowError("zero point outside int32 (input outside the documented domain)")
    return q, s_bits.astype(np.uint16), z.astype(np.int32)


# ---------------------------------------------------------------------------
# W8A16 variant: the same asymmetric rules with 8-bit codes
# ---------------------------------------------------------------------------

def quantize_int8(W_bits: np.ndarray, awq_s: np.ndarray | None = None):
    """W8A16 (Zeno AGI, "Weight-only vs mixed precision", its precision
    matrix): the asymmetric min/max rules of `quantize` with 256 levels,
    D / 255 for the step and codes clamped to 0..255; groups of 128.
    Returns (q uint8 [N][K], s_bits uint16 [N][K/128], z int32 [N][K/128])."""
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = bf16_to_f32(W_bits)
    if awq_s is not None:
        w = (w * np.asarray(awq_s, dtype=np.float32)[None, :]).astype(np.float32)
    wg = w.reshape(N, K // GROUP, GROUP)
    s_bits, s, z = group_scale_zero(wg, QMAX8)
    q = group_codes(wg, s, z, QMAX8).reshape(N, K)
    return q, s_bits.astype(np.uint16), z.astype(np.int32)


def pack_codes_int8(q: np.ndarray) -> np.ndarray:
    """q uint8 [N][K] (0..255) -> words uint32 [N][K/4]: byte j of word i
    holds k = 4i + j, so the little-endian byte stream is q row by row."""
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    q4 = q.reshape(N, K // 4, 4)
    words = np.zeros((N, K // 4), dtype=np.uint32)
    for j in range(4):
        words |= (q4[:, :, j] & np.uint32(0xFF)) << np.uint32(8 * j)
    return words


def unpack_codes_int8(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint32)
    N, W4 = w.shape
    q = np.zeros((N, W4, 4), dtype=np.uint8)
    for j in range(4):
        q[:, :, j] = ((w >> np.uint32(8 * j)) & np.uint32(0xFF)).astype(np.uint8)
    return q.reshape(N, W4 * 4)


def quantize_pack_int8(W_bits: np.ndarray, awq_s: np.ndarray | None = None):
    q, s_bits, z = quantize_int8(W_bits, awq_s)
    return pack_codes_int8(q), s_bits, z


def dequantize_int8(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """w_hat = (q - z) * s in float64 for 8-bit codes, g = k // 128."""
    q = unpack_codes_int8(codes).astype(np.float64)
    N, K = q.shape
    s = bf16_to_f32(scales).astype(np.float64)
    z = np.asarray(zeros, dtype=np.int64).astype(np.float64)
    g = np.arange(K) // GROUP
    return (q - z[:, g]) * s[:, g]


def matmul_ref_int8(X_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                    zeros: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """Y[m,n] = sum_k X[m,k] * w_hat[n,k] in float64, 8-bit codes."""
    if rows is not None:
        codes, scales, zeros = codes[rows], scales[rows], zeros[rows]
    return bf16_to_f32(X_bits).astype(np.float64) @ dequantize_int8(codes, scales, zeros).T


# ---------------------------------------------------------------------------
# Symmetric variant: zero point fixed at the middle of the code range
# ---------------------------------------------------------------------------

SYM_ZERO = 8         # signed codes -7..7 stored as 1..15


def group_scale_symmetric(w_groups: np.ndarray):
    """Scale of each group for symmetric INT4.

    The pages name symmetric uniform quantisation and argue that it wastes
    range ("Quantization I: int8, int4, the basics", "Concept"; Axe Corsa
    model card, "The Two-Stage Pipeline"), but their formula is stripped.
    Reading: the grid is centred on zero and reaches the largest magnitude,
      A = max |w|; t = fl32(A / 7); s = bf16 of t rounded toward zero,
    with the asymmetric rule's fallback for a zero or subnormal s (s =
    bf16_rtz(A), then 1.0).  Codes are round_half_away(w / s) in -7..7,
    stored with zero point 8, so the dequantisation (q - z) s and every
    kernel are those of the asymmetric format.
    Returns (s_bits uint16 [...], s float32 [...])."""
    w = np.asarray(w_groups, dtype=np.float32)
    a = np.abs(w).max(axis=-1).astype(np.float32)
    t = (a / np.float32(7)).astype(np.float32)
    s_bits = f32_to_bf16_rtz(t)
    s = bf16_to_f32(s_bits)
    degenerate = s < FLT_MIN
    if np.any(degenerate):
        alt_bits = f32_to_bf16_rtz(a)
        alt = bf16_to_f32(alt_bits)
        alt_bits = np.where(alt < FLT_MIN, np.uint16(0x3F80), alt_bits)  # 1.0
        s_bits = np.where(degenerate, alt_bits, s_bits).astype(np.uint16)
        s = bf16_to_f32(s_bits)
    return s_bits, s


def quantize_symmetric(W_bits: np.ndarray, awq_s: np.ndarray | None = None):
    """Symmetric group-wise INT4 of a BF16 matrix W [N][K]: returns (q uint8
    [N][K] in 1..15, s_bits uint16 [N][K/128], z int32 [N][K/128] all 8).
    awq_s as for quantize()."""
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    w = bf16_to_f32(W_bits)
    if awq_s is not None:
        w = (w * np.asarray(awq_s, dtype=np.float32)[None, :]).astype(np.float32)
    wg = w.reshape(N, K // GROUP, GROUP)
    s_bits, s = group_scale_symmetric(wg)
    z = np.full(s_bits.shape, SYM_ZERO, dtype=np.int64)
    q = group_codes(wg, s, z).reshape(N, K)
    return q, s_bits.astype(np.uint16), z.astype(np.int32)


def quantize_pack_symmetric(W_bits: np.ndarray, awq_s: np.ndarray | None = None):
    q, s_bits, z = quantize_symmetric(W_bits, awq_s)
    return pack_codes(q), s_bits, z


# ---------------------------------------------------------------------------
# Packing: eight 4-bit codes per 32-bit word along K
# ---------------------------------------------------------------------------

def pack_codes(q: np.ndarray) -> np.ndarray:
    """q uint8 [N][K] (values 0..15) -> words uint32 [N][K/8].

    Nibble j (bits 4j..4j+3) of word i holds k = 8i + j.  In little-endian
    byte order each byte then holds two consecutive codes, low nibble first,
    the byte stream of the compressed-tensors packing (Axe Corsa model card,
    "What the Tensor Types Tell You": two INT4 values per byte).
    """
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    q8 = q.reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        words |= (q8[:, :, j] & np.uint32(0xF)) << np.uint32(4 * j)
    return words


def pack_codes_i64(q: np.ndarray) -> np.ndarray:
    """q uint8 [N][K] -> int64 [N][K/16], the compressed-tensors container
    (Axe Corsa model card, "What the Tensor Types Tell You": packed INT4
    codes held in I64 tensors, two values per byte): nibble j of word i is
    k = 16i + j, little endian."""
    q = np.asarray(q, dtype=np.uint64)
    N, K = q.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    q16 = q.reshape(N, K // 16, 16)
    words = np.zeros((N, K // 16), dtype=np.uint64)
    for j in range(16):
        words |= (q16[:, :, j] & np.uint64(0xF)) << np.uint64(4 * j)
    return words.view(np.int64)


def unpack_codes(words: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes: words uint32 [N][K/8] -> q uint8 [N][K]."""
    w = np.asarray(words, dtype=np.uint32)
    N, W8 = w.shape
    q = np.zeros((N, W8, 8), dtype=np.uint8)
    for j in range(8):
        q[:, :, j] = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8)
    return q.reshape(N, W8 * 8)


def quantize_pack(W_bits: np.ndarray, awq_s: np.ndarray | None = None, group: int = GROUP):
    """Quantise then pack: returns (codes uint32 [N][K/8], scales uint16
    [N][K/group] (BF16 bits), zeros int32 [N][K/group])."""
    q, s_bits, z = quantize(W_bits, awq_s, group)
    return pack_codes(q), s_bits, z


# ---------------------------------------------------------------------------
# Dequantise and multiply
# ---------------------------------------------------------------------------

def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """w_hat[n,k] = (q[n,k] - z[n,g]) * s[n,g] in float64, g = k // group
    (Axe Corsa model card, "The Two-Stage Pipeline", dequantisation
    equation), the group size read from the shapes.  Exact: the product has
    at most ~40 significant bits."""
    q = unpack_codes(codes).astype(np.float64)
    N, K = q.shape
    s = bf16_to_f32(scales).astype(np.float64)
    z = np.asarray(zeros, dtype=np.int64).astype(np.float64)
    g = np.arange(K) // _group_of(K, s.shape[1])
    return (q - z[:, g]) * s[:, g]


def matmul_ref(X_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray,
               zeros: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """Reference output Y[m,n] = sum_k X[m,k] * w_hat[n,k] in float64.

    X_bits: BF16 bits [M][K].  If `rows` is given, only those output columns n
    are computed (the result has shape [M][len(rows)]).
    """
    if rows is not None:
        codes, scales, zeros = codes[rows], scales[rows], zeros[rows]
    w_hat = dequantize(codes, scales, zeros)
    x = bf16_to_f32(X_bits).astype(np.float64)
    return x @ w_hat.T


# ---------------------------------------------------------------------------
# Dense BF16 comparisons: the offline expansion the pages warn against and
# the dense product the INT4 path is measured against
# ---------------------------------------------------------------------------

def dequantize_bf16(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """Dense BF16 weights of an offline dequantisation: w[n,k] =
    BF16_RNE(fl32(fl32(q - z) * s)), g = k // 128, as BF16 bits [N][K].

    The expansion itself is the "dequantise offline" alternative of Zeno AGI,
    "Weight-only vs mixed precision" (table of offline versus fused
    dequantisation) and the middle kernel of its naive three-kernel pipeline
    ("7. The Marlin Kernel").  Reading: the pages fix no precision for it;
    here the integer difference becomes float32 (exact below 2**24), one
    float32 multiply rounds to nearest even, and one more rounding to nearest
    even gives BF16.  The result is NOT the exact dequantised weight: it is
    what a dense BF16 model built from the packed weights holds."""
    q = unpack_codes(codes).astype(np.int64)
    N, K = q.shape
    s = bf16_to_f32(scales)
    z = np.asarray(zeros, dtype=np.int64)
    g = np.arange(K) // _group_of(K, s.shape[1])
    diff = (q - z[:, g]).astype(np.float32)
    prod = np.multiply(diff, s[:, g], dtype=np.float32)
    return f32_to_bf16_rne(prod)


def dense_matmul_ref(X_bits: np.ndarray, W_bits: np.ndarray,
                     rows: np.ndarray | None = None) -> np.ndarray:
    """Y[m,n] = sum_k X[m,k] * W[n,k] for BF16 X [M][K] and BF16 W [N][K],
    in float64 (the dense BF16 linear layer, Zeno AGI, "Weight-only vs mixed
    precision", "1. The Basic Recipe": weights and activations both 16-bit).
    If `rows` is given only those output columns are computed."""
    W = np.asarray(W_bits)
    if rows is not None:
        W = W[rows]
    x = bf16_to_f32(X_bits).astype(np.float64)
    w = bf16_to_f32(W).astype(np.float64)
    return x @ w.T


# ---------------------------------------------------------------------------
# AWQ (optional fold of the per-input-channel scale into the producer)
# ---------------------------------------------------------------------------

def awq_importance(Xcal_bits: np.ndarray) -> np.ndarray:
    """Per-input-channel importance = mean over calibration tokens of |X|.
    Reading of the stripped importance formula in the Axe Corsa model card,
    "Stage 1: Activation-Aware Weight Scaling" (per-channel activation
    magnitudes).  Float64 mean, returned as float64 [K]."""
    x = bf16_to_f32(Xcal_bits).astype(np.float64)
    return np.abs(x).mean(axis=0)


def awq_scale(importance: np.ndarray, alpha: float) -> np.ndarray:
    """s_i = importance_i ** alpha (Axe Corsa model card, "Stage 1"), in
    float64, rounded to float32."""
    imp = np.asarray(importance, dtype=np.float64)
    return np.power(imp, np.float64(alpha)).astype(np.float32)


def awq_fold(s: np.ndarray, gamma_bits: np.ndarray) -> np.ndarray:
    """Fold X' = diag(s)^-1 X into the producer's per-channel weight:
    gamma'[k] = bf16_rne(fl32(gamma[k] / s[k])) (Axe Corsa model card,
    "Stage 1": the division is absorbed into the preceding LayerNorm)."""
    g = bf16_to_f32(gamma_bits)
    return f32_to_bf16_rne((g / np.asarray(s, dtype=np.float32)).astype(np.float32))


def apply_channel_scale(X_bits: np.ndarray, gamma_bits: np.ndarray) -> np.ndarray:
    """The producer's output with a folded per-channel weight:
    X'[m,k] = bf16_rne(fl32(X[m,k] * gamma[k]))."""
    x = bf16_to_f32(X_bits)
    g = bf16_to_f32(gamma_bits)
    return f32_to_bf16_rne((x * g[None, :]).astype(np.float32))


def awq_search(W_bits: np.ndarray, Xcal_bits: np.ndarray, alphas, X_bits: np.ndarray | None = None):
    """AWQ's one-dimensional search over the exponent of s = importance^alpha
    (Axe Corsa model card, "Stage 1: Activation-Aware Weight Scaling";
    cyankiwi docs, "The Baseline: AWQ": a light grid search rather than
    training).  For each alpha: s from the calibration batch, the weights
    quantised as W' = W diag(s), the activations fed through the folded
    producer weight gamma' = bf16(1 / s) (producer weight 1), and the
    relative L2 error of the layer output against the dense BF16 product
    X W^T measured on X (default: the calibration batch).
    Reading: the pages name neither the grid nor the objective's norm; the
    objective is the layer-output error the AWQ pages describe, in L2.
    Returns (errors float64 [len(alphas)], index of the smallest)."""
    W_bits = np.asarray(W_bits, dtype=np.uint16)
    X_bits = Xcal_bits if X_bits is None else X_bits
    K = W_bits.shape[1]
    imp = awq_importance(Xcal_bits)
    y_dense = dense_matmul_ref(X_bits, W_bits)
    ones = np.full(K, 0x3F80, dtype=np.uint16)
    errs = []
    for a in alphas:
        s = awq_scale(imp, a)
        codes, scales, zeros = quantize_pack(W_bits, s)
        Xs = apply_channel_scale(X_bits, awq_fold(s, ones))
        y = matmul_ref(Xs, codes, scales, zeros)
        errs.append(np.linalg.norm(y - y_dense) / np.linalg.norm(y_dense))
    errs = np.asarray(errs, dtype=np.float64)
    return errs, int(np.argmin(errs))


# ---------------------------------------------------------------------------
# A chain of dependent decode linears (a decoder stack's weight stream)
# ---------------------------------------------------------------------------
#
# The weight stream of a whole decoder (BASELINE config 5: 40 layers of four
# INT4 linears) is a chain: each linear's input is formed from the output of
# the one before by the layer's glue.  Readings (the pages describe the
# linears and the AWQ fold, not the rest of the decoder):
# * outputs are stored in BF16 (round to nearest even of the exact product),
#   and each input is formed from the stored BF16 values;
# * "prev": the previous output as is (o -> gate_up: the residual add and the
#   normalisation are left out);
# * "swiglu": the previous output holds the gate then the up projection
#   ([gate | up], K each); x = silu(gate) * up with silu(g) = g / (1 + e^-g);
# * "attn1": attention over a context of one cached token: the softmax over a
#   single score is 1, so each query head's output is the value vector of its
#   key/value head; the previous output holds [q | k | v] and head h (of
#   head_dim inputs) reads v of key/value head h // group;
# * an optional per-input-channel producer weight gamma (the folded AWQ
#   1 / s, Axe Corsa model card, "Stage 1: Activation-Aware Weight Scaling")
#   multiplies x;
# * every formed input is rounded once to BF16 (nearest even).

def f64_to_bf16_rne(x) -> np.ndarray:
    """float64 -> BF16 bits, round to nearest even, one rounding (values in
    the normal BF16 range): x = m 2^e with 1/2 <= |m| < 1, keep 8 significant
    bits of m."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 256.0), e - 8)          # np.rint: ties to even
    return f32_to_bf16_rtz(r.astype(np.float32))     # r is exactly a BF16 value


def silu_ref(g) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in float64."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def chain_input(kind: str, y_prev_bits, K: int, params=None, gamma_bits=None,
                x0_bits=None) -> np.ndarray:
    """BF16 bits [M][K] of a chain linear's input (see the readings above).
    kind: "x0" (the chain's own input x0_bits), "prev", "swiglu" or "attn1"
    (params = (v_offset, head_dim, group))."""
    if kind == "x0":
        x = bf16_to_f32(np.asarray(x0_bits)[:, :K]).astype(np.float64)
    elif kind == "prev":
        x = bf16_to_f32(np.asarray(y_prev_bits)[:, :K]).astype(np.float64)
    elif kind == "swiglu":
        y = bf16_to_f32(np.asarray(y_prev_bits)).astype(np.float64)
        x = silu_ref(y[:, :K]) * y[:, K:2 * K]
    elif kind == "attn1":
        v_off, head_dim, group = params
        y = bf16_to_f32(np.asarray(y_prev_bits)).astype(np.float64)
        k = np.arange(K)
        src = v_off + (k // head_dim // group) * head_dim + k % head_dim
        x = y[:, src]
    else:
        raise ValueError(kind)
    if gamma_bits is not None:
        x = x * bf16_to_f32(gamma_bits).astype(np.float64)[None, :]
    return f64_to_bf16_rne(x)


def chain_ref(x0_bits, linears):
    """Run a chain.  linears: list of dicts with codes, scales, zeros (a packed
    matrix), kind, optional params and gamma (BF16 bits [K]).  Returns the
    list of (input BF16 bits [M][K], exact output float64 [M][N], stored
    output BF16 bits [M][N]) per linear."""
    out = []
    y_prev = None
    for L in linears:
        K = L["codes"].shape[1] * 8
        x = chain_input(L["kind"], y_prev, K, L.get("params"), L.get("gamma"), x0_bits)
        y = matmul_ref(x, L["codes"], L["scales"], L["zeros"])
        y_prev = f64_to_bf16_rne(y)
        out.append((x, y, y_prev))
    return out


# ---------------------------------------------------------------------------
# Parity gates on the floating-point output
# ---------------------------------------------------------------------------

REL_L2_TOL = 2e-3     # relative L2 error of the BF16 output
ELEM_TOL = 1e-2       # per element: |err| <= ELEM_TOL * (|ref| + 1)


def output_errors(y, y_ref):
    """Returns (relative L2 error, max over elements of |err| / (|ref|+1))."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = y - y_ref
    denom = np.linalg.norm(y_ref)
    rel = float(np.linalg.norm(err) / denom) if denom > 0 else float(np.linalg.norm(err))
    elem = float(np.max(np.abs(err) / (np.abs(y_ref) + 1.0))) if err.size else 0.0
    return rel, elem


def output_ok(y, y_ref) -> bool:
    rel, elem = output_errors(y, y_ref)
    return rel <= REL_L2_TOL and elem <= ELEM_TOL


def storage_bytes(N: int, K: int) -> int:
    """Bytes of the packed format: N*K/2 codes + 2 B scale + 4 B zero per
    group of 128 (Axe Corsa model card, "Storage Cost")."""
    return N * K // 2 + (N * K // GROUP) * (2 + 4)
