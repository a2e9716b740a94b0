"""Group scales at the edges of the format, through every matmul entry point,
against the CPU oracle.

Two kinds of input:
* weights whose groups of 128 mix ordinary draws with the quantiser's special
  cases (constant, all-zero, subnormal constant, +-2^-125 whose scale is the
  smallest normal BF16 value, values far from zero with a large negative
  zero point), packed by the library (bit-exact against the oracle's packer)
  and by the oracle;
* packed matrices from the oracle's packer with some scales replaced by zero,
  negative or subnormal values -- inputs the packer never writes but the
  matmul contract accepts (for example codes and metadata read in place from
  another tool's container).
Every output is compared with the oracle's fp64 product of the same packed
matrix (Axe Corsa model card, "The Two-Stage Pipeline": w_hat = (q - z_g) s_g
for every group).
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, assert_pack_equal, sample_rows, zero_weight_group_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def to_dev_packed(codes, scales, zeros):
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).to(DEV)
    s = gen.from_bits(scales, device=DEV)
    z = torch.from_numpy(np.ascontiguousarray(zeros, dtype=np.int32)).to(DEV)
    return w4.PackedLinear(c, s, z)


def to_dev_packed_int8(codes, scales, zeros):
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).to(DEV)
    s = gen.from_bits(scales, device=DEV)
    z = torch.from_numpy(np.ascontiguousarray(zeros, dtype=np.int32)).to(DEV)
    return w4.PackedLinearInt8(c, s, z)


def ref_packed(X_bits, codes, scales, zeros, int8=False):
    x = np.abs(O.bf16_to_f32(X_bits).astype(np.float64))
    if int8:
        return (O.matmul_ref_int8(X_bits, codes, scales, zeros),
                x @ np.abs(O.dequantize_int8(codes, scales, zeros)).T)
    return O.matmul_ref(X_bits, codes, scales, zeros), x @ np.abs(O.dequantize(codes, scales, zeros)).T


def check(y, X_bits, packed_np, label, rows=None, mrows=None, int8=False):
    torch.cuda.synchronize()
    codes, scales, zeros = packed_np
    if mrows is not None:
        X_bits = X_bits[mrows]
        y = y[torch.as_tensor(mrows, device=DEV)]
    if rows is not None:
        y = y[:, torch.as_tensor(rows, device=DEV)]
        codes, scales, zeros = codes[rows], scales[rows], zeros[rows]
    y_ref, mag = ref_packed(X_bits, codes, scales, zeros, int8)
    assert np.all(np.isfinite(y.float().cpu().numpy())), f"{label}: non-finite output"
    assert_output_close(y, y_ref, mag, label=label,
                        gates_only_cols=zero_weight_group_rows(codes, scales, zeros, int8))


def modified_scales(scales, what, seed):
    """Replace about 30% of the scales by zero, negative or subnormal values
    (what = 'mixed' takes all three and zeroes one whole row)."""
    s = scales.copy()
    rng = np.random.default_rng(seed)
    pick = rng.random(s.shape) < 0.3
    if what == "zero":
        s[pick] = 0
    elif what == "negative":
        s[pick] |= 0x8000
    elif what == "subnormal":
        s[pick] = rng.integers(1, 0x80, size=int(pick.sum())).astype(np.uint16)
    else:
        choice = rng.integers(0, 3, size=int(pick.sum()))
        v = s[pick]
        s[pick] = np.where(choice == 0, 0, np.where(choice == 1, v | 0x8000, 0x0001)).astype(np.uint16)
        s[0, :] = 0
    return s


# (M, N, K): the three tile kernels of the group-128 GEMM -- 64 x 128 tiles,
# 128 x 128 tiles (48 large tiles), 256 x 256 tiles (4 x 49 large tiles) --
# and 256 x 256 tiles with K split over 8 runs through the binding's
# workspace (2 x 12 large tiles, K = 8192)
GEMM_SHAPES = [(300, 520, 1536), (500, 6100, 512), (1000, 12300, 384), (300, 3000, 8192)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_extreme_groups(M, N, K):
    W = gen.extreme_weights(N, K, "extreme", f"gemm{N}", device=DEV)
    X = gen.activations(M, K, "extreme", f"gemm{N}", device=DEV)
    p = w4.w4a16_pack(W)
    y = w4.w4a16_gemm(X, p)
    Wb = gen.bits(W)
    big = N > 1000
    rows = sample_rows(N, 96, seed=N) if big else None
    mrows = sample_rows(M, 48, seed=M) if big else None
    assert_pack_equal(p, Wb, rows=rows)
    check(y, gen.bits(X), O.quantize_pack(Wb), f"gemm extreme {M}x{N}x{K}", rows, mrows)


@pytest.mark.parametrize("M", [1, 5, 16, 32])
def test_gemv_extreme_groups(M):
    N, K = 700, 2048
    W = gen.extreme_weights(N, K, "extreme", "gemv", device=DEV)
    X = gen.activations(M, K, "extreme", "gemv", device=DEV)
    p = w4.w4a16_pack(W)
    y = w4.w4a16_gemv(X, p)
    check(y, gen.bits(X), O.quantize_pack(gen.bits(W)), f"gemv extreme M={M}")


@pytest.mark.parametrize("group", [32, 64])
@pytest.mark.parametrize("M", [1, 5, 16, 300])
def test_grouped_extreme_groups(group, M):
    N, K = 520, 1024
    W = gen.extreme_weights(N, K, "extreme", f"grouped{group}", device=DEV)
    X = gen.activations(M, K, "extreme", f"grouped{group}", device=DEV)
    p = w4.w4a16_pack(W, group=group)
    y = w4.w4a16_linear(X, p)      # gemv_grouped up to M = 32, gemm_grouped above
    Wb = gen.bits(W)
    assert_pack_equal(p, Wb, group=group)
    check(y, gen.bits(X), O.quantize_pack(Wb, None, group), f"group {group} extreme M={M}")


@pytest.mark.parametrize("M", [1, 4, 300])
def test_int8_extreme_groups(M):
    N, K = 520, 1024
    W = gen.extreme_weights(N, K, "extreme", "int8", device=DEV)
    X = gen.activations(M, K, "extreme", "int8", device=DEV)
    p = w4.w4a16_pack_int8(W)
    y = w4.w4a16_gemv_int8(X, p) if M <= 4 else w4.w4a16_gemm_int8(X, p)
    check(y, gen.bits(X), O.quantize_pack_int8(gen.bits(W)), f"int8 extreme M={M}", int8=True)


@pytest.mark.parametrize("what", ["zero", "negative", "subnormal", "mixed"])
def test_scales_outside_the_packer_group128(what):
    N, K = 700, 2048
    Wb = gen.bits(gen.weights(N, K, "extreme", "meta", shift=True))
    codes, scales, zeros = O.quantize_pack(Wb)
    scales = modified_scales(scales, what, seed=len(what))
    p = to_dev_packed(codes, scales, zeros)
    for M in (1, 5, 16, 32, 300):
        X = gen.activations(M, K, "extreme", "meta", device=DEV)
        y = w4.w4a16_linear(X, p)
        check(y, gen.bits(X), (codes, scales, zeros), f"{what} scales M={M}")
    # the 256 x 256 tile kernel
    M, N, K = 1000, 12300, 384
    Wb = gen.bits(gen.weights(N, K, "extreme", "meta_big"))
    codes, scales, zeros = O.quantize_pack(Wb)
    scales = modified_scales(scales, what, seed=7 + len(what))
    p = to_dev_packed(codes, scales, zeros)
    X = gen.activations(M, K, "extreme", "meta_big", device=DEV)
    y = w4.w4a16_gemm(X, p)
    check(y, gen.bits(X), (codes, scales, zeros), f"{what} scales, large tiles",
          rows=sample_rows(N, 96, seed=3), mrows=sample_rows(M, 48, seed=4))
    # the same tiles with K split over 8 runs (binding's workspace)
    M, N, K = 300, 3000, 8192
    Wb = gen.bits(gen.weights(N, K, "extreme", "meta_split"))
    codes, scales, zeros = O.quantize_pack(Wb)
    scales = modified_scales(scales, what, seed=11 + len(what))
    p = to_dev_packed(codes, scales, zeros)
    X = gen.activations(M, K, "extreme", "meta_split", device=DEV)
    y = w4.w4a16_gemm(X, p)
    check(y, gen.bits(X), (codes, scales, zeros), f"{what} scales, split K",
          rows=sample_rows(N, 96, seed=13), mrows=sample_rows(M, 48, seed=14))


@pytest.mark.parametrize("group", [32, 64])
def test_scales_outside_the_packer_grouped(group):
    N, K = 520, 1024
    Wb = gen.bits(gen.weights(N, K, "extreme", f"meta{group}", shift=True))
    codes, scales, zeros = O.quantize_pack(Wb, None, group)
    scales = modified_scales(scales, "mixed", seed=group)
    p = to_dev_packed(codes, scales, zeros)
    for M in (1, 5, 16, 300):
        X = gen.activations(M, K, "extreme", f"meta{group}", device=DEV)
        y = w4.w4a16_linear(X, p)
        check(y, gen.bits(X), (codes, scales, zeros), f"group {group} mixed scales M={M}")


def test_scales_outside_the_packer_int8():
    N, K = 520, 1024
    Wb = gen.bits(gen.weights(N, K, "extreme", "meta8", shift=True))
    codes, scales, zeros = O.quantize_pack_int8(Wb)
    scales = modified_scales(scales, "mixed", seed=8)
    p = to_dev_packed_int8(codes, scales, zeros)
    for M in (1, 3, 4, 300):
        X = gen.activations(M, K, "extreme", "meta8", device=DEV)
        y = w4.w4a16_gemv_int8(X, p) if M <= 4 else w4.w4a16_gemm_int8(X, p)
        check(y, gen.bits(X), (codes, scales, zeros), f"int8 mixed scales M={M}", int8=True)
