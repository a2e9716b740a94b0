"""Helpers that compare the HIP library's outputs with the CPU oracle.

The oracle only ever sees the generator's inputs (W, X, per-channel vectors)
as BF16/FP32 bits; it never receives anything the library computed.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
from synth import gen

BF16_HALF_ULP_REL = 2.0 ** -8      # |bf16_rne(y) - y| <= 2^-8 |y|
ACC_REL = 1e-4                     # float32 accumulation, relative to sum |x w_hat|


def u32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def i32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().astype(np.int32)


def assert_pack_equal(p, W_bits, rows=None, awq_s=None, group=128):
    """Packed output of the library equals the oracle's bit for bit (on the
    given rows, or all rows)."""
    if rows is None:
        rows = np.arange(W_bits.shape[0])
    codes, scales, zeros = O.quantize_pack(W_bits[rows], awq_s, group)
    g_codes = u32(p.codes)[rows]
    g_scales = gen.bits(p.scales)[rows]
    g_zeros = i32(p.zeros)[rows]
    for name, a, b in (("codes", g_codes, codes), ("scales", g_scales, scales), ("zeros", g_zeros, zeros)):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            r, c = bad[0]
            raise AssertionError(f"{name} differ at {len(bad)} places; first row {rows[r]} col {c}: "
                                 f"gpu {a[r, c]:#x} oracle {b[r, c]:#x}")


def reference(X_bits, W_bits, rows=None, awq_s=None, group=128):
    """Oracle output Y_ref [M][len(rows)] and sum_k |x w_hat| for the bound."""
    if rows is None:
        rows = np.arange(W_bits.shape[0])
    codes, scales, zeros = O.quantize_pack(W_bits[rows], awq_s, group)
    y_ref = O.matmul_ref(X_bits, codes, scales, zeros)
    w_hat = O.dequantize(codes, scales, zeros)
    x = O.bf16_to_f32(X_bits).astype(np.float64)
    mag = np.abs(x) @ np.abs(w_hat).T
    return y_ref, mag


def assert_output_close(y_gpu: torch.Tensor, y_ref, mag, *, gate_min_elems=2048, label="",
                        strict=True, gates_only_cols=None):
    """Per element: within half a BF16 ulp of the fp64 oracle plus a float32
    accumulation allowance; and the output gates (relative L2 <= 2e-3 and
    |err| <= 1e-2 (|ref| + 1)), the L2 gate only where the output is large
    enough for the statistic to be meaningful.  Output columns flagged in
    gates_only_cols (see zero_weight_group_rows) are held to the gates only."""
    y = O.bf16_to_f32(gen.bits(y_gpu)).astype(np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    err = np.abs(y - y_ref)
    bound = BF16_HALF_ULP_REL * np.abs(y_ref) * (1 + 1e-3) + ACC_REL * mag + 1e-30
    if gates_only_cols is not None:
        bound = np.where(np.asarray(gates_only_cols, bool)[None, :], np.inf, bound)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert not strict or np.all(err <= bound), (
        f"{label}: element {worst} gpu {y[worst]!r} ref {y_ref[worst]!r} bound {bound[worst]!r}")
    rel, elem = O.output_errors(y, y_ref)
    assert elem <= O.ELEM_TOL, f"{label}: per-element gate {elem}"
    if y.size >= gate_min_elems:
        assert rel <= O.REL_L2_TOL, f"{label}: relative L2 {rel}"
    return rel, elem


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """First, last and `count` random distinct rows (sorted)."""
    rng = np.random.default_rng(seed)
    pick = rng.choice(N, size=min(count, N), replace=False)
    return np.unique(np.concatenate([[0, N - 1], pick]))


def zero_weight_group_rows(codes, scales, zeros, int8=False):
    """Weight rows [N] holding a group whose weights all dequantise to zero
    (every code equals the group's zero point; the packer's all-zero and
    subnormal groups, scale 1.0).  The kernels form each group as
    s (sum x (128 + q) - (128 + z) sum x) in float32, whose rounding is
    relative to |s| (128 + |z|) |sum x|; for such a group none of that is
    covered by the accumulation allowance relative to sum |x w_hat|, so these
    rows are held to the output gates only."""
    q = O.unpack_codes_int8(codes) if int8 else O.unpack_codes(codes)
    N, G = scales.shape
    qg = q.reshape(N, G, -1).astype(np.int64)
    return np.any(np.all(qg == np.asarray(zeros, np.int64)[:, :, None], axis=2), axis=1)
