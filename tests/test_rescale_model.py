"""A float32 model of the prefill kernel's per-group rescale, on the CPU.

The matrix-core kernel keeps one accumulator per output and moves it from one
quantisation group's units to the next at every group end.  This file
models that arithmetic in numpy float32 (one rounding per group product, per
fused multiply-add and per multiply, as the kernel does) on weights whose
groups include the quantiser's special cases -- the smallest normal BF16
scale after ordinary groups, zero, constant and far-from-zero groups -- and
on packed matrices with zero, negative and subnormal scales.  It checks that

* the unit scheme the kernel uses (scale s = u 4^E, |u| in [1, 4), the power
  of four carried by the B operand's exponent byte) gives outputs within the
  parity bound of the oracle for all of them, and
* the earlier scheme (accumulator in units of the group's own scale, moved by
  s_g / s_{g+1}) overflows on the same inputs, so these inputs do catch a
  return to it.

The model is not the oracle: the oracle (oracle/w4a16_ref.py) supplies the
expected outputs; this file only checks the kernel's arithmetic design.
"""
import numpy as np
import pytest

import oracle as O
from synth import gen
from parity import assert_output_close

F32 = np.float32
K_EMIN, K_EMAX = -60, 56   # the kernel's clamp of E


def _groups(X_bits, codes, scales, zeros):
    """Per group: x [M][128] float64, codes q [N][128], s bits [N], z [N]."""
    x = O.bf16_to_f32(X_bits).astype(np.float64)
    q = O.unpack_codes(codes)
    G = scales.shape[1]
    for g in range(G):
        sl = slice(128 * g, 128 * (g + 1))
        yield x[:, sl], q[:, sl].astype(np.float64), scales[:, g], zeros[:, g].astype(np.float64)


def _split(sbits, u_prev):
    """E = floor(log4 |s|) clamped, u = s 4^-E; a zero scale keeps u_prev."""
    e2 = ((sbits.astype(np.int64) >> 7) & 0xFF)
    E = np.clip((e2 - 127) >> 1, K_EMIN, K_EMAX)
    s = O.bf16_to_f32(sbits).astype(np.float64)
    u = np.where(s == 0.0, u_prev, np.ldexp(s, -2 * E))
    return E, u.astype(F32)


def model_unit_scheme(X_bits, codes, scales, zeros):
    """The kernel's arithmetic: T in units of u, B = 4^E (128 + q)."""
    M, N = X_bits.shape[0], codes.shape[0]
    T = np.zeros((M, N), F32)
    E, u = _split(scales[:, 0], np.ones(N, F32))
    G = scales.shape[1]
    with np.errstate(over="ignore", invalid="ignore"):
        for g, (x, q, _, z) in enumerate(_groups(X_bits, codes, scales, zeros)):
            B = np.ldexp(128.0 + q, 2 * E[:, None])          # exact BF16 operands
            T = (T + (x @ B.T).astype(F32)).astype(F32)      # matrix-core sums, fp32
            xs = x.sum(axis=1).astype(F32)                   # activation sums
            zb = np.ldexp(z + 128.0, 2 * E).astype(F32)
            if g + 1 < G:
                E, u_next = _split(scales[:, g + 1], u)
                r = (u / u_next).astype(F32)
                u = u_next
            else:
                r = u
            T = ((T.astype(np.float64) - zb[None, :] * xs[:, None].astype(np.float64)).astype(F32) * r).astype(F32)
    return T


def model_ratio_scheme(X_bits, codes, scales, zeros):
    """The earlier arithmetic: T in units of s_g, moved by s_g / s_{g+1}."""
    M, N = X_bits.shape[0], codes.shape[0]
    T = np.zeros((M, N), F32)
    G = scales.shape[1]
    s_all = O.bf16_to_f32(scales)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        for g, (x, q, _, z) in enumerate(_groups(X_bits, codes, scales, zeros)):
            T = (T + (x @ (128.0 + q).T).astype(F32)).astype(F32)
            xs = x.sum(axis=1).astype(F32)
            zb = (z + 128.0).astype(F32)
            s = s_all[:, g]
            r = (s * (F32(1) / s_all[:, g + 1])).astype(F32) if g + 1 < G else s
            T = ((T.astype(np.float64) - zb[None, :] * xs[:, None].astype(np.float64)).astype(F32) * r).astype(F32)
    return T


def _reference(X_bits, codes, scales, zeros):
    y_ref = O.matmul_ref(X_bits, codes, scales, zeros)
    mag = np.abs(O.bf16_to_f32(X_bits).astype(np.float64)) @ np.abs(O.dequantize(codes, scales, zeros)).T
    return y_ref, mag


def _as_bf16(T):
    return gen.from_bits(O.f32_to_bf16_rne(T))


def test_unit_scheme_on_extreme_groups_and_ratio_scheme_overflows():
    N, K, M = 96, 1536, 8
    W = gen.bits(gen.extreme_weights(N, K, "rescale_model", "w"))
    X = gen.bits(gen.activations(M, K, "rescale_model", "x"))
    codes, scales, zeros = O.quantize_pack(W)
    y_ref, mag = _reference(X, codes, scales, zeros)
    assert np.all(np.isfinite(y_ref))
    T = model_unit_scheme(X, codes, scales, zeros)
    assert np.all(np.isfinite(T))
    assert_output_close(_as_bf16(T), y_ref, mag, label="unit scheme, extreme groups")
    old = model_ratio_scheme(X, codes, scales, zeros)
    assert not np.all(np.isfinite(old)), "these inputs no longer stress the per-group rescale"


def test_unit_scheme_on_the_smallest_normal_scale_after_ordinary_groups():
    # two ordinary groups, then the +-2^-125 group (scale 2^-125): the case
    # where the ratio scheme multiplies by ~2^120
    hand = gen.hand_groups()
    rng = np.random.default_rng(7)
    rows = [np.concatenate([rng.standard_normal(256), hand["pm_2^-125"]]) for _ in range(16)]
    W = O.f32_to_bf16_rne(np.array(rows, np.float32))
    X = gen.bits(gen.activations(8, 384, "rescale_model", "tiny_last"))
    codes, scales, zeros = O.quantize_pack(W)
    assert np.all(scales[:, 2] == 0x0100)
    y_ref, mag = _reference(X, codes, scales, zeros)
    T = model_unit_scheme(X, codes, scales, zeros)
    assert_output_close(_as_bf16(T), y_ref, mag, label="tiny last group")
    assert not np.all(np.isfinite(model_ratio_scheme(X, codes, scales, zeros)))


@pytest.mark.parametrize("what", ["zero", "negative", "subnormal", "mixed"])
def test_unit_scheme_on_scales_outside_the_packer(what):
    # packed matrices the packer never writes but the matmul contract accepts
    # (e.g. read in place from another tool's container): zero, negative and
    # subnormal scales among ordinary ones
    N, K, M = 64, 1024, 8
    W = gen.bits(gen.weights(N, K, "rescale_model", "meta", shift=True))
    X = gen.bits(gen.activations(M, K, "rescale_model", "meta"))
    codes, scales, zeros = O.quantize_pack(W)
    scales = scales.copy()
    rng = np.random.default_rng(11)
    pick = rng.random(scales.shape) < 0.3
    if what == "zero":
        scales[pick] = 0x0000
    elif what == "negative":
        scales[pick] |= 0x8000
    elif what == "subnormal":
        scales[pick] = rng.integers(1, 0x80, size=int(pick.sum())).astype(np.uint16)
    else:
        choice = rng.integers(0, 3, size=int(pick.sum()))
        vals = scales[pick]
        vals = np.where(choice == 0, 0, np.where(choice == 1, vals | 0x8000, 0x0001)).astype(np.uint16)
        scales[pick] = vals
        scales[0, :] = 0      # a row of zero scales only
    y_ref, mag = _reference(X, codes, scales, zeros)
    T = model_unit_scheme(X, codes, scales, zeros)
    assert np.all(np.isfinite(T))
    assert_output_close(_as_bf16(T), y_ref, mag, label=f"{what} scales")
