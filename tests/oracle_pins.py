"""Pins that tie the CPU oracle to facts fixed outside itself.

Each check raises AssertionError on failure.  They are collected by
test_oracle_pins.py and reused by test_oracle_mutations.py, which plants
plausible mistakes in the oracle and asserts that some check catches each.

Sources of truth used here (never the oracle's own formulas retyped):
* closed forms derived by hand for constructed groups (derivations inline),
* the figures the pages print (tests/golden/storage_cost.json),
* library routines for special cases: torch's float32->bfloat16 conversion
  (round to nearest even), Python's decimal ROUND_HALF_UP (half away from
  zero), fractions.Fraction for exact rational arithmetic,
* brute force over all 16 codes on tiny inputs,
* invariants the pages state (all 16 codes used; output unchanged when the
  weights already lie on the grid).
"""

from __future__ import annotations

import decimal
import json
import os
from fractions import Fraction

import numpy as np
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits_of(values) -> np.ndarray:
    """Exact float -> BF16 bits for values known to be BF16-representable."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in BF16"
    return (u >> 16).astype(np.uint16)


def _frac_of_f32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


# ---------------------------------------------------------------------------
# Conversions and rounding
# ---------------------------------------------------------------------------

def check_bf16_rne_matches_torch(seed=1):
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties around the rounding boundary
    base = rng.integers(0, 2**16, size=20000, dtype=np.uint64).astype(np.uint32) << 16
    ties = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001])
    u = np.concatenate([u, ties]).astype(np.uint32)
    f = u.view(np.float32)
    finite = np.isfinite(f)
    f = f[finite]
    ours = O.f32_to_bf16_rne(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref), "f32->bf16 RNE disagrees with torch"
    # widening is exact
    back = O.bf16_to_f32(ref)
    ref_back = torch.from_numpy(ref.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back.view(np.uint32), ref_back.view(np.uint32))


def check_bf16_rtz_hand():
    # 0x3F80FFFF = 1 + (2^16-1) * 2^-23: truncation keeps 0x3F80, RNE gives 0x3F81
    x = np.array([0x3F80FFFF, 0xBF80FFFF, 0x3DCCCCCD, 0x3F800000, 0x00000001],
                 dtype=np.uint32).view(np.float32)
    assert list(O.f32_to_bf16_rtz(x)) == [0x3F80, 0xBF80, 0x3DCC, 0x3F80, 0x0000]
    assert list(O.f32_to_bf16_rne(x)) == [0x3F81, 0xBF81, 0x3DCD, 0x3F80, 0x0000]


def check_round_half_away(seed=2):
    hand = {2.5: 3, -2.5: -3, 0.5: 1, -0.5: -1, 1.5: 2, -1.5: -2, 6.5: 7,
            0.49999997: 0, -0.49999997: 0, 0.0: 0, 7.0: 7, -8.0: -8}
    for v, r in hand.items():
        assert O.round_half_away(np.float32(v)) == r, (v, r)
    rng = np.random.default_rng(seed)
    vals = np.concatenate([
        rng.normal(0, 20, size=3000).astype(np.float32),
        (rng.integers(-40, 40, size=1000) + 0.5).astype(np.float32),
    ])
    ours = O.round_half_away(vals)
    for v, r in zip(vals, ours):
        d = decimal.Decimal(float(v)).quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_UP)
        assert int(d) == int(r), (float(v), int(d), r)


# ---------------------------------------------------------------------------
# Hand-built groups with closed-form scale, zero point and codes
# ---------------------------------------------------------------------------

def _quantize_group(values):
    W = _bf16_bits_of(values).reshape(1, 128)
    q, s_bits, z = O.quantize(W)
    return q[0], int(s_bits[0, 0]), int(z[0, 0])


def check_hand_groups():
    j = np.arange(128) % 16

    # G1: w = (j - 8) * 2^-7.  min = -8*2^-7, max = 7*2^-7, D = 15*2^-7,
    # t = 2^-7 exactly -> s = 2^-7 (bits 0x3C00); z = -min/s = 8; q = j.
    q, s, z = _quantize_group((j - 8) * 2.0 ** -7)
    assert (s, z) == (0x3C00, 8)
    assert np.array_equal(q, j)
    words = O.pack_codes(q.reshape(1, 128))
    assert list(words[0, :2]) == [0x76543210, 0xFEDCBA98]
    assert np.array_equal(words[0], np.tile(np.array([0x76543210, 0xFEDCBA98], np.uint32), 8))

    # G2: all positive, w = 1 + j/16.  D = 15/16, s = 1/16 (0x3D80),
    # z = -16 (negative zero point), q = j.
    q, s, z = _quantize_group(1.0 + j / 16.0)
    assert (s, z) == (0x3D80, -16)
    assert np.array_equal(q, j)

    # G3: exact ties.  Start from G1 (s = 2^-7, z = 8) and put +-2.5 s and
    # 0.5 s at some positions: half away from zero gives 3 / -3 / 1, so the
    # codes are 11 / 5 / 9 (ties-to-even would give 10 / 6 / 8).
    v = (j - 8) * 2.0 ** -7
    v[16], v[17], v[18] = 2.5 * 2.0 ** -7, -2.5 * 2.0 ** -7, 0.5 * 2.0 ** -7
    q, s, z = _quantize_group(v)
    assert (s, z) == (0x3C00, 8)
    assert (q[16], q[17], q[18]) == (11, 5, 9)

    # G4: zero-point tie.  min = -6.5 s, max = 8.5 s with s = 2^-7:
    # D = 15 s -> s exact; -min/s = 6.5 -> z = 7; q(min) = -7 + 7 = 0,
    # q(max) = 9 + 7 = 16 -> clipped to 15.
    v = np.full(128, 0.0)
    v[0], v[1] = -6.5 * 2.0 ** -7, 8.5 * 2.0 ** -7
    q, s, z = _quantize_group(v)
    assert (s, z) == (0x3C00, 7)
    assert (q[0], q[1], q[2]) == (0, 15, 7)

    # G5: BF16 scale rounds toward zero.  min = -0.5, max = 1.0: D = 1.5,
    # t = fl32(0.1) = 0x3DCCCCCD, s = 0x3DCC (RNE would give 0x3DCD).
    v = np.zeros(128)
    v[0], v[1] = -0.5, 1.0
    q, s, z = _quantize_group(v)
    assert s == 0x3DCC
    s_f = np.float32(np.array([0x3DCC0000], np.uint32).view(np.float32)[0])
    # z = round(0.5 / 0.099609375 = 5.0196) = 5; q(max) = round(10.039) + 5 = 15
    assert z == 5 and q[0] == 0 and q[1] == 15
    assert s_f == np.float32(0.099609375)

    # G6: constant groups reconstruct exactly: c = 0.375 -> degenerate,
    # s = 0.375 (0x3EC0), z = -1, q = 0, w_hat = (0 - (-1)) * 0.375.
    q, s, z = _quantize_group(np.full(128, 0.375))
    assert (s, z) == (0x3EC0, -1) and np.all(q == 0)
    q, s, z = _quantize_group(np.full(128, -0.375))
    assert (s, z) == (0x3EC0, 1) and np.all(q == 0)

    # G7: all zero -> s = 1.0 (0x3F80), z = 0, q = 0.
    q, s, z = _quantize_group(np.zeros(128))
    assert (s, z) == (0x3F80, 0) and np.all(q == 0)

    # G8: subnormal constant 2^-130 -> degenerate, the fallback scale is
    # itself subnormal, so s = 1.0, z = 0, q = 0 (w_hat = 0).
    q, s, z = _quantize_group(np.full(128, 2.0 ** -130))
    assert (s, z) == (0x3F80, 0) and np.all(q == 0)

    # G9: +-2^-125: D/15 is subnormal -> degenerate; s = 2^-125 (0x0100),
    # z = 1, codes 0 and 2, reconstructing -2^-125 and +2^-125 exactly.
    v = np.where(np.arange(128) % 2 == 0, -(2.0 ** -125), 2.0 ** -125)
    q, s, z = _quantize_group(v)
    assert (s, z) == (0x0100, 1)
    assert np.all(q[0::2] == 0) and np.all(q[1::2] == 2)


def check_dequant_closed_form():
    # codes j, z = 8, s = 2^-7 -> w_hat = (j - 8) * 2^-7; plus a second group
    # with z = -16, s = 1/16 -> w_hat = 1 + j/16.  K = 256, two groups.
    j = np.arange(128) % 16
    q = np.concatenate([j, j]).reshape(1, 256).astype(np.uint8)
    codes = O.pack_codes(q)
    scales = np.array([[0x3C00, 0x3D80]], dtype=np.uint16)
    zeros = np.array([[8, -16]], dtype=np.int32)
    w = O.dequantize(codes, scales, zeros)[0]
    assert np.array_equal(w[:128], (j - 8) * 2.0 ** -7)
    assert np.array_equal(w[128:], 1.0 + j / 16.0)


def check_grouped_hand():
    """Groups of 32 and 64 (the smaller group sizes "Quantization I",
    "Concept", names), worked by hand on one row of 128 weights: quarter i
    holds (j - 8) * 2^-(7+i), j = k mod 16.
    * group 32: every group is its own grid, s = 2^-(7+i) (BF16 bits 0x3C00,
      0x3B80, 0x3B00, 0x3A80), z = 8, q = j;
    * group 64: group 0 spans quarters 0 and 1, so s = 2^-7, z = 8; quarter
      1's values are half a step apart and round half away from zero:
      q = 8 + round_half_away((j - 8) / 2); group 1 likewise with s = 2^-9;
    * group 128: one grid for the row, s = 2^-7, z = 8."""
    k = np.arange(128)
    j = k % 16
    w = (j - 8) * 2.0 ** -(7 + k // 32)
    Wb = _bf16_bits_of(w).reshape(1, 128)
    half = np.array([8 + int(np.sign(v) * np.floor(abs(v) + 0.5)) for v in (j[:32] - 8) / 2.0])
    q, s, z = O.quantize(Wb, group=32)
    assert list(s[0]) == [0x3C00, 0x3B80, 0x3B00, 0x3A80] and list(z[0]) == [8] * 4
    assert np.array_equal(q[0], j)
    q, s, z = O.quantize(Wb, group=64)
    assert list(s[0]) == [0x3C00, 0x3B00] and list(z[0]) == [8, 8]
    assert np.array_equal(q[0], np.concatenate([j[:32], half, j[:32], half]))
    assert list(half[:4]) == [4, 4, 5, 5] and list(half[-4:]) == [10, 11, 11, 12]
    q, s, z = O.quantize(Wb, group=128)
    assert list(s[0]) == [0x3C00] and list(z[0]) == [8]
    # dequantisation reads the group size from the shapes: group 32 here
    codes, scales, zeros = O.quantize_pack(Wb, group=32)
    assert np.array_equal(O.dequantize(codes, scales, zeros)[0], w)


def check_int8_on_grid_and_layout(seed=50, N=24, K=384):
    """W8A16: weights exactly on a grid (c - z0) * s0 with codes 0 and 255 in
    every group come back unchanged (s0 a power of two, so D / 255 = s0
    exactly); the bytes of the packed words are the codes in order; the
    dequantised weights equal the inputs and the output equals the
    unquantised matmul exactly (coarse inputs, exact fp64 sums)."""
    rng = np.random.default_rng(seed)
    G = K // 128
    c = rng.integers(0, 256, size=(N, G, 128))
    c[:, :, 5] = 0
    c[:, :, 77] = 255
    z0 = rng.integers(0, 256, size=(N, G))
    s0 = 2.0 ** rng.integers(-14, -8, size=(N, G))
    w = (c - z0[..., None]) * s0[..., None]
    W_bits = _bf16_bits_of(w.reshape(N, K).astype(np.float32))
    q, s_bits, z = O.quantize_int8(W_bits)
    assert np.array_equal(q.reshape(N, G, 128), c) and np.array_equal(z, z0)
    assert np.array_equal(O.bf16_to_f32(s_bits).astype(np.float64), s0)
    words = O.pack_codes_int8(q)
    assert words.shape == (N, K // 4)
    assert np.array_equal(words.astype("<u4").view(np.uint8).reshape(N, K), q)
    assert np.array_equal(O.unpack_codes_int8(words), q)
    assert np.array_equal(O.dequantize_int8(words, s_bits, z), w.reshape(N, K))
    x = (rng.integers(-63, 64, size=(3, K)) / 4.0).astype(np.float32)
    y = O.matmul_ref_int8(_bf16_bits_of(x), words, s_bits, z)
    assert np.array_equal(y, x.astype(np.float64) @ w.reshape(N, K).T)


def check_int8_brute_force(seed=51, N=3, K=128):
    """W8A16 codes are the nearest of the 256 grid points (ties away from
    zero), against the stored BF16 scale, on generated weights."""
    rng = np.random.default_rng(seed)
    w = (rng.normal(0, 0.02, size=(N, K)) + rng.uniform(-0.01, 0.01, size=(N, 1))).astype(np.float32)
    W_bits = O.f32_to_bf16_rne(w)
    q, s_bits, z = O.quantize_int8(W_bits)
    wf = O.bf16_to_f32(W_bits)
    mn, mx = wf.min(axis=1), wf.max(axis=1)
    for n in range(N):
        s = _frac_of_f32(O.bf16_to_f32(s_bits[n, 0]))
        # the step: s <= D / 255 < s (1 + 2^-7)
        D = _frac_of_f32(mx[n]) - _frac_of_f32(mn[n])
        assert s <= D / 255 < s * (1 + Fraction(1, 128))
        zz = int(z[n, 0])
        for k in range(K):
            wk = _frac_of_f32(wf[n, k])
            best = min(range(256), key=lambda cc: (abs(wk - (cc - zz) * s), -abs(cc - zz)))
            if best != q[n, k]:
                r = wk / s
                frac = r - (r.numerator // r.denominator)
                assert abs(frac - Fraction(1, 2)) < abs(r) * Fraction(1, 2 ** 22), (n, k, best, q[n, k])
        assert q[n].min() == 0 and q[n].max() >= 254


# ---------------------------------------------------------------------------
# Packing layout
# ---------------------------------------------------------------------------

def check_pack_layout(seed=3):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(5, 64), dtype=np.uint8)
    words = O.pack_codes(q)
    assert words.dtype == np.uint32 and words.shape == (5, 8)
    # byte stream: byte b holds k = 2b in the low nibble and k = 2b + 1 in the
    # high nibble (two codes per byte, consecutive along K)
    byts = words.astype("<u4").view(np.uint8).reshape(5, 32)
    expect = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(byts, expect)
    assert np.array_equal(O.unpack_codes(words), q)


# ---------------------------------------------------------------------------
# Invariants on generated groups (the pages: all 16 INT4 values used)
# ---------------------------------------------------------------------------

def check_min_max_codes(W_bits, group=128):
    q, s_bits, z = O.quantize(W_bits, group=group)
    N, K = W_bits.shape
    w = O.bf16_to_f32(W_bits).reshape(N, K // group, group)
    qg = q.reshape(N, K // group, group)
    imin = w.argmin(axis=-1)
    imax = w.argmax(axis=-1)
    qmin = np.take_along_axis(qg, imin[..., None], -1)[..., 0]
    qmax = np.take_along_axis(qg, imax[..., None], -1)[..., 0]
    assert np.all(qmin == 0), "the group minimum must map to code 0"
    mn, mx = w.min(-1), w.max(-1)
    straddles = (mn <= 0) & (mx >= 0) & (mx > mn)
    assert np.all(qmax[straddles] == 15), "the group maximum must map to code 15"
    # scale brackets the exact step: s <= D/15 < s * (1 + 2^-7)
    s = O.bf16_to_f32(s_bits).astype(np.float64)
    D = (mx.astype(np.float64) - mn.astype(np.float64))
    nz = D > 0
    assert np.all(s[nz] <= D[nz] / 15 * (1 + 2.0 ** -23))
    assert np.all(D[nz] / 15 < s[nz] * (1 + 2.0 ** -7) * (1 + 2.0 ** -22))
    return straddles.mean()


def check_all_codes_on_grid(seed=4, N=64, K=512, group=128):
    """Weights that lie exactly on a grid (q0 - z0) * s0 come back unchanged:
    pack returns (q0, s0, z0) and every group uses all 16 codes."""
    rng = np.random.default_rng(seed)
    G = K // group
    q0 = rng.integers(0, 16, size=(N, G, group))
    q0[:, :, 0] = 0
    q0[:, :, 1] = 15
    for n in range(N):                      # all 16 codes in every group
        for g in range(G):
            q0[n, g, 2:18] = rng.permutation(16)
    z0 = rng.integers(0, 16, size=(N, G))
    mant = 1.0 + rng.integers(0, 8, size=(N, G)) / 8.0          # <= 4 significant bits
    s0 = mant * 2.0 ** rng.integers(-12, -2, size=(N, G))
    w = (q0 - z0[..., None]) * s0[..., None]
    W_bits = _bf16_bits_of(w.reshape(N, K).astype(np.float32))
    q, s_bits, z = O.quantize(W_bits, group=group)
    assert np.array_equal(q.reshape(N, G, group), q0)
    assert np.array_equal(z, z0)
    assert np.array_equal(O.bf16_to_f32(s_bits).astype(np.float64), s0)
    for n in range(N):
        for g in range(G):
            assert len(np.unique(q.reshape(N, G, group)[n, g])) == 16
    return W_bits, (q, s_bits, z)


def check_on_grid_matmul_exact(seed=5):
    """On-grid weights: the reference output equals the unquantised matmul,
    exactly (inputs on coarse grids so every fp64 sum is exact)."""
    W_bits, _ = check_all_codes_on_grid(seed, N=48, K=384)
    rng = np.random.default_rng(seed + 100)
    x = (rng.integers(-255, 256, size=(6, 384)) / 8.0).astype(np.float32)
    X_bits = _bf16_bits_of(x)
    codes, scales, zeros = O.quantize_pack(W_bits)
    y = O.matmul_ref(X_bits, codes, scales, zeros)
    w = O.bf16_to_f32(W_bits).astype(np.float64)
    exact = x.astype(np.float64) @ w.T
    assert y.shape == (6, 48)
    assert np.array_equal(y, exact)
    rows = np.array([47, 3, 10])
    assert np.array_equal(O.matmul_ref(X_bits, codes, scales, zeros, rows=rows), exact[:, rows])


# ---------------------------------------------------------------------------
# Brute force on tiny inputs (exact rationals)
# ---------------------------------------------------------------------------

def check_brute_force(seed=6, M=4, K=128, N=8, group=128):
    rng = np.random.default_rng(seed)
    w = (rng.normal(0, 0.02, size=(N, K)) + rng.uniform(-0.01, 0.01, size=(N, 1))).astype(np.float32)
    W_bits = O.f32_to_bf16_rne(w)
    x = rng.normal(0, 1, size=(M, K)).astype(np.float32)
    X_bits = O.f32_to_bf16_rne(x)
    q, s_bits, z = O.quantize(W_bits, group=group)
    wf = O.bf16_to_f32(W_bits)
    near_ties = 0
    for n in range(N):
        for g in range(K // group):
            s = _frac_of_f32(O.bf16_to_f32(s_bits[n, g]))
            zz = int(z[n, g])
            for k in range(g * group, (g + 1) * group):
                wk = _frac_of_f32(wf[n, k])
                # argmin over the 16 codes of |w - (c - z) s|, ties away from zero
                best = min(range(16), key=lambda c: (abs(wk - (c - zz) * s), -abs(c - zz)))
                if best != q[n, k]:
                    r = wk / s
                    frac = r - (r.numerator // r.denominator)
                    assert abs(frac - Fraction(1, 2)) < abs(r) * Fraction(1, 2 ** 22), \
                        (n, k, best, q[n, k])
                    near_ties += 1
    # output: exact rational sum vs the fp64 reference
    codes, scales, zeros = O.pack_codes(q), s_bits, z
    y = O.matmul_ref(X_bits, codes, scales, zeros)
    xf = O.bf16_to_f32(X_bits)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                g = k // group
                s = _frac_of_f32(O.bf16_to_f32(s_bits[n, g]))
                term = _frac_of_f32(xf[m, k]) * (int(q[n, k]) - int(z[n, g])) * s
                acc += term
                mag += abs(term)
            assert abs(Fraction(float(y[m, n])) - acc) <= mag * Fraction(1, 2 ** 45), (m, n)
    return near_ties


# ---------------------------------------------------------------------------
# AWQ pieces
# ---------------------------------------------------------------------------

def check_awq_prescale_power_of_two(seed=7):
    """Scaling every input channel by 2 doubles each group's scale and leaves
    codes and zero points unchanged (the quantiser input is W * s)."""
    rng = np.random.default_rng(seed)
    W_bits = O.f32_to_bf16_rne(rng.normal(0, 0.02, size=(16, 256)).astype(np.float32))
    q1, s1, z1 = O.quantize(W_bits)
    q2, s2, z2 = O.quantize(W_bits, awq_s=np.full(256, 2.0, np.float32))
    assert np.array_equal(q1, q2) and np.array_equal(z1, z2)
    assert np.array_equal(O.bf16_to_f32(s2), 2 * O.bf16_to_f32(s1))
    # a per-channel scale that only touches channel 5 changes only groups 0
    s = np.ones(256, np.float32)
    s[5] = 4.0
    q3, s3, z3 = O.quantize(W_bits, awq_s=s)
    assert np.array_equal(s3[:, 1], s1[:, 1]) and np.array_equal(q3[:, 128:], q1[:, 128:])
    w = O.bf16_to_f32(W_bits).astype(np.float64)
    w[:, 5] *= 4.0
    wg = w[:, :128]
    D = wg.max(1) - wg.min(1)
    s3f = O.bf16_to_f32(s3[:, 0]).astype(np.float64)
    assert np.all(s3f <= D / 15 * (1 + 2.0 ** -23)) and np.all(D / 15 < s3f * (1 + 2.0 ** -6))


def check_awq_fold_hand():
    g = _bf16_bits_of(np.array([1.0, 1.0, -0.75, 3.0], np.float32))
    s = np.array([2.0, 3.0, 0.5, 1.0], np.float32)
    # 1/2 = 0.5 (0x3F00); fl32(1/3) = 0x3EAAAAAB -> RNE 0x3EAB; -1.5 = 0xBFC0; 3 = 0x4040
    assert list(O.awq_fold(s, g)) == [0x3F00, 0x3EAB, 0xBFC0, 0x4040]
    # the producer output after folding: X' = X * gamma' (bf16 RNE)
    X = _bf16_bits_of(np.array([[2.0, 3.0, 1.0, -1.0]], np.float32))
    assert list(O.apply_channel_scale(X, O.awq_fold(s, g))[0]) == [0x3F80, 0x3F80, 0xBFC0, 0xC040]


def check_awq_importance_and_scale(seed=8):
    rng = np.random.default_rng(seed)
    x = O.f32_to_bf16_rne(rng.normal(0, 1, size=(7, 5)).astype(np.float32))
    imp = O.awq_importance(x)
    xf = O.bf16_to_f32(x)
    for k in range(5):
        exact = sum(abs(_frac_of_f32(xf[t, k])) for t in range(7)) / 7
        assert abs(Fraction(float(imp[k])) - exact) <= exact * Fraction(1, 2 ** 50)
    # alpha = 1/2 is the square root (correctly rounded in float64, then fp32)
    v = np.abs(rng.normal(0, 3, size=1000)) + 1e-3
    assert np.array_equal(O.awq_scale(v, 0.5), np.sqrt(v).astype(np.float32))
    assert np.array_equal(O.awq_scale(v, 1.0), v.astype(np.float32))
    assert np.all(O.awq_scale(v, 0.0) == 1.0)


def check_awq_equivalence_unquantised(seed=9):
    """(X/s) (W diag(s))^T = X W^T: the fold leaves the output unchanged
    before any quantisation; with the BF16 rounding of X' the mismatch is at
    BF16 resolution."""
    rng = np.random.default_rng(seed)
    K, N, M = 256, 32, 4
    W_bits = O.f32_to_bf16_rne(rng.normal(0, 0.02, size=(N, K)).astype(np.float32))
    X_bits = O.f32_to_bf16_rne(rng.normal(0, 1, size=(M, K)).astype(np.float32))
    imp = O.awq_importance(X_bits)
    s = O.awq_scale(imp, 0.5)
    w = O.bf16_to_f32(W_bits).astype(np.float64)
    x = O.bf16_to_f32(X_bits).astype(np.float64)
    s64 = s.astype(np.float64)
    y0 = x @ w.T
    y1 = (x / s64) @ (w * s64).T
    assert np.max(np.abs(y1 - y0)) <= 1e-12 * np.max(np.abs(y0))
    one = _bf16_bits_of(np.ones(K, np.float32))
    xp = O.bf16_to_f32(O.apply_channel_scale(X_bits, O.awq_fold(s, one))).astype(np.float64)
    w_s = (O.bf16_to_f32(W_bits) * s).astype(np.float32).astype(np.float64)
    y2 = xp @ w_s.T
    assert np.linalg.norm(y2 - y0) / np.linalg.norm(y0) < 2.0 ** -7


# ---------------------------------------------------------------------------
# Storage cost (figures printed on the pages)
# ---------------------------------------------------------------------------

def check_storage_cost():
    with open(os.path.join(GOLDEN, "storage_cost.json")) as f:
        gold = json.load(f)
    N, K = 4096, 4096
    q = np.zeros((N, K), np.uint8)
    codes = O.pack_codes(q)
    s_bits = np.zeros((N, K // 128), np.uint16)
    z = np.zeros((N, K // 128), np.int32)
    nbytes = codes.nbytes + s_bits.nbytes + z.nbytes
    assert nbytes == O.storage_bytes(N, K)
    bits = 8 * nbytes / (N * K)
    assert bits == gold["bits_per_weight"]["value"]
    assert abs(16 / bits - gold["compression_vs_bf16"]["value"]) <= gold["compression_vs_bf16"]["rounding"]
    g = gold["quantised_layers_27b_gb"]
    gb = g["params"] * bits / 8 / 1e9
    assert g["low"] <= gb <= g["high"], gb
    assert 2 * gold["bf16_27b_gb"]["params"] / 1e9 == gold["bf16_27b_gb"]["value"]
    assert 0.5 * gold["int4_floor_27b_gb"]["params"] / 1e9 == gold["int4_floor_27b_gb"]["value"]
    assert 2 * gold["bf16_70b_gb"]["params"] / 1e9 == gold["bf16_70b_gb"]["value"]


def check_output_gate():
    """The tolerance gate itself: BF16 rounding of an exact output passes,
    a 1% perturbation fails."""
    rng = np.random.default_rng(10)
    y = rng.normal(0, 3, size=(8, 512))
    yb = O.bf16_to_f32(O.f32_to_bf16_rne(y.astype(np.float32))).astype(np.float64)
    assert O.output_ok(yb, y)
    assert not O.output_ok(y * 1.01, y)
    assert not O.output_ok(y + np.where(np.arange(512) == 7, 0.5, 0.0), y)


# ---------------------------------------------------------------------------
# Dense BF16 comparisons
# ---------------------------------------------------------------------------

def check_dequant_bf16_hand():
    """Offline BF16 expansion on constructed groups.
    Group 1: s = 2**-3, z = 3: (q - 3)/8 for q = 0..15 is a BF16 value, so
    the expansion is exact.
    Group 2: s = 1, z = -250: v = q + 250 runs over 250..265.  BF16 holds
    every integer below 256 and the even ones in [256, 512) (8 significant
    bits); an odd v >= 257 is a tie between its neighbours and goes to the
    one with an even last mantissa bit: 257 -> 256, 259 -> 260, 261 -> 260,
    263 -> 264, 265 -> 264 (mantissa m = (v - 256)/2)."""
    words = np.array([[0x76543210, 0xFEDCBA98] * 8, [0x76543210, 0xFEDCBA98] * 8], dtype=np.uint32)
    scales = np.array([[0x3E00], [0x3F80]], dtype=np.uint16)      # 2**-3, 1.0
    zeros = np.array([[3], [-250]], dtype=np.int32)
    got = O.dequantize_bf16(words, scales, zeros)
    q = np.arange(16)
    exp1 = _bf16_bits_of((q - 3) / 8.0)
    v2 = [250, 251, 252, 253, 254, 255, 256, 256, 258, 260, 260, 260, 262, 264, 264, 264]
    exp2 = _bf16_bits_of(v2)
    for rep in range(8):
        assert np.array_equal(got[0, 16 * rep:16 * rep + 16], exp1), got[0, :16]
        assert np.array_equal(got[1, 16 * rep:16 * rep + 16], exp2), got[1, :16]


def check_dequant_bf16_vs_torch(seed=12, N=16, K=512):
    """Where the float32 product is exact (|q - z| < 2**16 times an 8-bit
    scale), the expansion is the exact dequantised weight rounded once to
    BF16: compare with torch's float32 -> bfloat16 conversion (round to
    nearest even) of the float64 dequantisation."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes = O.pack_codes(q)
    scales = O.f32_to_bf16_rtz(rng.uniform(1e-3, 3.0, size=(N, K // 128)).astype(np.float32))
    zeros = rng.integers(-400, 400, size=(N, K // 128)).astype(np.int32)
    exact = O.dequantize(codes, scales, zeros).astype(np.float32)
    ref = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.dequantize_bf16(codes, scales, zeros), ref)


def check_dense_brute_force(seed=13, M=3, N=5, K=40):
    """Dense product against an exact rational sum of the BF16 inputs."""
    rng = np.random.default_rng(seed)
    X_bits = O.f32_to_bf16_rne(rng.normal(0, 1, size=(M, K)).astype(np.float32))
    W_bits = O.f32_to_bf16_rne(rng.normal(0, 0.05, size=(N, K)).astype(np.float32))
    y = O.dense_matmul_ref(X_bits, W_bits)
    assert y.shape == (M, N)
    xf, wf = O.bf16_to_f32(X_bits), O.bf16_to_f32(W_bits)
    for m in range(M):
        for n in range(N):
            acc = sum(_frac_of_f32(xf[m, k]) * _frac_of_f32(wf[n, k]) for k in range(K))
            mag = sum(abs(_frac_of_f32(xf[m, k]) * _frac_of_f32(wf[n, k])) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - acc) <= mag * Fraction(1, 2 ** 45), (m, n)
    rows = np.array([4, 1])
    assert np.array_equal(O.dense_matmul_ref(X_bits, W_bits, rows), y[:, rows])


def check_dense_matches_fused_on_grid(seed=14, M=4, N=6, K=256):
    """With power-of-two scales and small |q - z| the BF16 expansion is
    exact, so the dense product of the expanded weights equals the fused
    reference term for term."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes = O.pack_codes(q)
    scales = _bf16_bits_of(2.0 ** rng.integers(-8, 2, size=(N, K // 128)))
    zeros = rng.integers(-20, 20, size=(N, K // 128)).astype(np.int32)
    X_bits = O.f32_to_bf16_rne(rng.normal(0, 1, size=(M, K)).astype(np.float32))
    W_bits = O.dequantize_bf16(codes, scales, zeros)
    assert np.array_equal(O.dense_matmul_ref(X_bits, W_bits), O.matmul_ref(X_bits, codes, scales, zeros))


# ---------------------------------------------------------------------------
# Format variants: symmetric INT4 and the I64 code container
# ---------------------------------------------------------------------------

def check_symmetric_hand():
    """Constructed groups.
    G1: k * 2^-4 for k = -7..7 (and zeros): A = 7 * 2^-4, t = 2^-4 exactly,
    s = 2^-4 (bits 0x3D80), code = k + 8.
    G2: the same values times -3: A = 21 * 2^-4, t = 3 * 2^-4 = 0.1875 is a
    BF16 value (bits 0x3E40), codes = -k + 8.
    G3: all zero: t = 0 -> fallback bf16_rtz(0) = 0 -> s = 1.0 (0x3F80),
    every code 8.
    G4: one value 2^-126 (the smallest normal), the rest 0: t = 2^-126/7 is
    subnormal -> fallback s = 2^-126 (0x0080); the value becomes code 9
    (ratio 1), the zeros code 8."""
    k = np.concatenate([np.arange(-7, 8), np.zeros(113)]).astype(np.float64)
    groups = np.stack([k * 2.0 ** -4, -3 * k * 2.0 ** -4, np.zeros(128),
                       np.where(np.arange(128) == 5, 2.0 ** -126, 0.0)])
    W_bits = _bf16_bits_of(groups.reshape(1, 4 * 128))
    q, s_bits, z = O.quantize_symmetric(W_bits)
    assert list(s_bits[0]) == [0x3D80, 0x3E40, 0x3F80, 0x0080], [hex(v) for v in s_bits[0]]
    assert np.all(z == 8)
    q = q.reshape(4, 128).astype(np.int64)
    assert np.array_equal(q[0], (k + 8).astype(np.int64))
    assert np.array_equal(q[1], (-k + 8).astype(np.int64))
    assert np.all(q[2] == 8)
    assert q[3, 5] == 9 and np.all(np.delete(q[3], 5) == 8)


def check_symmetric_invariants(seed=15, N=48, K=1024):
    """Generated groups (with per-group shifts, so many groups are skewed):
    zero point 8; codes 1..15 (the code -8 is never needed); the largest
    magnitude maps to code 1 or 15; every weight is within half a scale step
    of its dequantised value (no clipping: |w|/s < 7.5)."""
    rng = np.random.default_rng(seed)
    w = (rng.normal(0, 0.02, size=(N, K)) + np.repeat(rng.uniform(-0.03, 0.03, size=(N, K // 128)), 128, 1))
    W_bits = O.f32_to_bf16_rne(w.astype(np.float32))
    q, s_bits, z = O.quantize_symmetric(W_bits)
    assert np.all(z == 8)
    assert q.min() >= 1 and q.max() <= 15
    wf = O.bf16_to_f32(W_bits).astype(np.float64).reshape(N, K // 128, 128)
    s = O.bf16_to_f32(s_bits).astype(np.float64)
    qg = q.reshape(N, K // 128, 128).astype(np.float64)
    err = np.abs(wf - (qg - 8) * s[..., None])
    assert np.all(err <= s[..., None] * (0.5 + 2.0 ** -20)), err.max()
    top = np.abs(wf).argmax(axis=-1)
    qtop = np.take_along_axis(qg, top[..., None], -1)[..., 0]
    assert np.all((qtop == 1) | (qtop == 15))
    # the scale reaches the largest magnitude: A/7 * (1 - 2^-7) < s <= A/7
    A = np.abs(wf).max(axis=-1)
    assert np.all(s <= A / 7) and np.all(s > A / 7 * (1 - 2.0 ** -7))


def check_symmetric_brute_force(seed=16, N=3, K=128):
    """Each code is the nearest of the 16 grid points (c - 8) s to w, ties
    away from zero, with exact rational arithmetic."""
    rng = np.random.default_rng(seed)
    W_bits = O.f32_to_bf16_rne(rng.normal(0, 0.05, size=(N, K)).astype(np.float32))
    q, s_bits, z = O.quantize_symmetric(W_bits)
    wf = O.bf16_to_f32(W_bits)
    for n in range(N):
        sc = _frac_of_f32(O.bf16_to_f32(s_bits[n, 0]))
        for k in range(K):
            wk = _frac_of_f32(wf[n, k])
            best = min(range(16), key=lambda c: (abs(wk - (c - 8) * sc), -abs(c - 8)))
            assert best == q[n, k], (n, k, best, q[n, k])


def check_i64_container(seed=17):
    """The I64 container holds sixteen codes per word, two per byte, low
    nibble first, consecutive along K: its byte stream is that of the
    two-codes-per-byte description, and so equals the 32-bit packing's."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(4, 256), dtype=np.uint8)
    w64 = O.pack_codes_i64(q)
    assert w64.dtype == np.int64 and w64.shape == (4, 16)
    byts = w64.astype("<i8").view(np.uint8).reshape(4, 128)
    expect = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(byts, expect)
    assert np.array_equal(w64.astype("<i8").view("<u4").reshape(4, 32), O.pack_codes(q).astype("<u4"))


# ---------------------------------------------------------------------------
# AWQ exponent search
# ---------------------------------------------------------------------------

def _salient_case(seed, N=64, K=512, T=64, w_salient=1.0):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.02, size=(N, K))
    sal = rng.choice(K, 5, replace=False)
    w[:, sal] *= w_salient
    x = rng.normal(0, 1, size=(T, K))
    x[:, sal] *= 20.0
    return O.f32_to_bf16_rne(w.astype(np.float32)), O.f32_to_bf16_rne(x.astype(np.float32))


def check_awq_search_alpha_zero_is_plain(seed=19):
    """alpha = 0 gives s = 1 exactly, so its error is that of the plain
    quantiser with the activations untouched."""
    Wb, Xb = _salient_case(seed)
    errs, _ = O.awq_search(Wb, Xb, [0.0, 0.5])
    codes, scales, zeros = O.quantize_pack(Wb)
    y = O.matmul_ref(Xb, codes, scales, zeros)
    yd = O.bf16_to_f32(Xb).astype(np.float64) @ O.bf16_to_f32(Wb).astype(np.float64).T
    assert errs[0] == np.linalg.norm(y - yd) / np.linalg.norm(yd)


def check_awq_search_protects_salient(seed=18):
    """The property AWQ rests on (Axe Corsa model card, "Stage 1"; cyankiwi
    docs, "The Baseline: AWQ": a few input channels with large activations
    carry the error): with five channels of 20x activations and ordinary
    weights, scaling those channels up cuts the output error by more than a
    fifth, and too large an exponent makes it worse again (the other
    channels lose resolution), so the best exponent is inside (0, 1)."""
    Wb, Xb = _salient_case(seed)
    alphas = np.linspace(0, 1, 11)
    errs, best = O.awq_search(Wb, Xb, alphas)
    assert errs[best] == errs.min()
    assert errs[best] < 0.8 * errs[0], errs
    assert 0 < best < len(alphas) - 1, errs
    assert errs[-1] > errs[best] * 1.5, errs


# ---------------------------------------------------------------------------
# Chain of dependent linears (decoder-stack weight stream, its glue)
# ---------------------------------------------------------------------------

def _bf16_value(bits) -> Fraction:
    return _frac_of_f32(O.bf16_to_f32(np.uint16(bits)))


def check_f64_to_bf16_single_rounding(seed=31):
    """float64 -> BF16 with one rounding to the nearest BF16 value, ties to
    even, against exact rationals: random magnitudes, exact midpoints of
    neighbouring BF16 values, and values one float64 ulp either side of them
    (where a detour through float32 would round twice)."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal(400) * np.exp2(rng.integers(-40, 40, 400))
    b = O.f32_to_bf16_rtz(base.astype(np.float32)).astype(np.int64)
    lo = O.bf16_to_f32(b.astype(np.uint16)).astype(np.float64)
    hi = O.bf16_to_f32((b + 1).astype(np.uint16)).astype(np.float64)
    mid = (lo + hi) / 2                                  # exact in float64
    xs = np.concatenate([base, mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)])
    got = O.f64_to_bf16_rne(xs)
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        t = int(O.f32_to_bf16_rtz(np.float32(x)))
        cands = [c for c in range(t - 2, t + 3) if 0 <= c < 0x10000 and (c & 0x7F80) != 0x7F80
                 and (c >> 15) == (t >> 15)]
        best = min(cands, key=lambda c: (abs(fx - _bf16_value(c)), c & 1))
        assert int(g) == best, (x, hex(int(g)), hex(best))
    # a value whose float32 rounding lands on a midpoint (float32 would round twice)
    x = -0.011505127308113048
    assert int(O.f64_to_bf16_rne(np.array([x]))[0]) == 0xBC3D


def check_silu_identities():
    """silu(g) - silu(-g) = g for every g (sigma(g) + sigma(-g) = 1),
    silu(0) = 0, silu(g) -> g for large g and -> 0 for very negative g."""
    g = np.linspace(-30, 30, 601)
    d = O.silu_ref(g) - O.silu_ref(-g)
    assert np.allclose(d, g, rtol=1e-14, atol=1e-14)
    assert O.silu_ref(np.array([0.0]))[0] == 0.0
    assert abs(O.silu_ref(np.array([50.0]))[0] - 50.0) < 1e-12
    v = O.silu_ref(np.array([-50.0]))[0]
    assert v < 0 and abs(v) < 1e-19
    # sigma(1) = e / (1 + e): silu(1) = 0.7310585786300049 (to double precision)
    assert abs(O.silu_ref(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15


def check_chain_input_hand():
    """The glue of a chain linear on a hand example: four query heads of two
    inputs, two key/value heads (group 2), previous output [q | k | v]."""
    q = [1, 2, 3, 4, 5, 6, 7, 8]
    k = [9, 10, 11, 12]
    v = [13, 14, 15, 16]
    y = _bf16_bits_of(np.array([q + k + v], np.float32))
    x = O.chain_input("attn1", y, 8, params=(12, 2, 2))
    assert list(O.bf16_to_f32(x)[0]) == [13, 14, 13, 14, 15, 16, 15, 16]
    # the previous output as is, and a producer weight
    x = O.chain_input("prev", y, 4)
    assert list(O.bf16_to_f32(x)[0]) == [1, 2, 3, 4]
    gam = _bf16_bits_of(np.array([0.5, 2.0, -1.0, 0.25], np.float32))
    x = O.chain_input("prev", y, 4, gamma_bits=gam)
    assert list(O.bf16_to_f32(x)[0]) == [0.5, 4.0, -3.0, 1.0]
    # swiglu: [gate | up], silu(0) * u = 0; and the odd part: x(g) - x(-g) = g u
    gate = np.array([0.0, 1.5, -2.0, 3.0], np.float32)
    up = np.array([7.0, 1.0, 1.0, -1.0], np.float32)
    xp = O.bf16_to_f32(O.chain_input("swiglu", _bf16_bits_of(np.concatenate([gate, up])[None]), 4))
    xm = O.bf16_to_f32(O.chain_input("swiglu", _bf16_bits_of(np.concatenate([-gate, up])[None]), 4))
    assert xp[0, 0] == 0.0
    d = (xp - xm).astype(np.float64)[0]
    assert np.all(np.abs(d - gate * up) <= 2 * 2.0 ** -8 * (np.abs(xp) + np.abs(xm))[0] + 1e-30)
    # the chain's own input, truncated to K
    x0 = _bf16_bits_of(np.array([[1, 2, 3, 4, 5, 6]], np.float32))
    assert list(O.bf16_to_f32(O.chain_input("x0", None, 4, x0_bits=x0))[0]) == [1, 2, 3, 4]


def check_chain_two_linears_exact(seed=33):
    """A chain of two on-grid linears whose intermediate output is exactly a
    BF16 value: the second output equals the dense product of the two weight
    matrices (fp64, exact) -- the chain feeds the stored output of the first
    linear, unchanged, into the second."""
    rng = np.random.default_rng(seed)
    M, K1, N1 = 3, 256, 128
    # first linear: one weight 15 * 2^-4 per row at a random input, the rest 0
    w1 = np.zeros((N1, K1), np.float64)
    pos = rng.integers(0, K1, size=N1)
    w1[np.arange(N1), pos] = 15 * 2.0 ** -4
    x0 = rng.integers(-17, 18, size=(M, K1)).astype(np.float64)
    # second linear: on-grid weights with every code in every group
    W2_bits, _ = check_all_codes_on_grid(seed + 1, N=24, K=N1)
    c1 = O.quantize_pack(_bf16_bits_of(w1.astype(np.float32)))
    c2 = O.quantize_pack(W2_bits)
    lin = [dict(codes=c1[0], scales=c1[1], zeros=c1[2], kind="x0"),
           dict(codes=c2[0], scales=c2[1], zeros=c2[2], kind="prev")]
    out = O.chain_ref(_bf16_bits_of(x0.astype(np.float32)), lin)
    y1 = x0 @ w1.T
    w2 = O.bf16_to_f32(W2_bits).astype(np.float64)
    assert np.array_equal(out[0][1], y1)
    assert np.array_equal(O.bf16_to_f32(out[0][2]).astype(np.float64), y1)   # exactly BF16
    assert np.array_equal(out[1][1], y1 @ w2.T)
