"""Quantisation groups of 32 and 64 inputs on the GPU against the CPU oracle:
the packer (bit-exact) and the decode and prefill matmuls on its output,
plus the same matmuls on packed inputs the oracle produced."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, assert_pack_equal, reference, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"
GROUPS = [32, 64]


def to_dev_packed(codes, scales, zeros):
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).to(DEV)
    s = gen.from_bits(scales, device=DEV)
    z = torch.from_numpy(np.ascontiguousarray(zeros, dtype=np.int32)).to(DEV)
    return w4.PackedLinear(c, s, z)


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (16, 4096), (257, 1024)])
def test_pack_bit_exact(group, N, K):
    W = gen.weights(N, K, "groups", f"{N}x{K}", shift=True, device=DEV)
    p = w4.w4a16_pack(W, group=group)
    torch.cuda.synchronize()
    assert p.group == group and tuple(p.scales.shape) == (N, K // group)
    assert_pack_equal(p, gen.bits(W), group=group)


@pytest.mark.parametrize("group", GROUPS)
def test_pack_awq_llama_shape_sampled(group):
    L = [l for l in gen.LLAMA8B if l.name == "gate_up"][0]
    W = gen.weights(L.N, L.K, "groups", L.name, shift=True, device=DEV)
    s = gen.channel_vector(L.K, "groups", L.name, "awq").to(DEV)
    p = w4.w4a16_pack(W, awq_s=s, group=group)
    torch.cuda.synchronize()
    rows = sample_rows(L.N, 64, seed=group)
    codes, scales, zeros = O.quantize_pack(gen.bits(W[torch.as_tensor(rows, device=DEV)]),
                                           s.cpu().numpy(), group)
    assert np.array_equal(p.codes.cpu().numpy().view(np.uint32)[rows], codes)
    assert np.array_equal(gen.bits(p.scales)[rows], scales)
    assert np.array_equal(p.zeros.cpu().numpy()[rows], zeros)


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 16, 32])
def test_gemv_ragged(group, M):
    # 100 rows: a ragged tail for every row blocking; three 128-input blocks
    N, K = 100, 384
    W = gen.weights(N, K, "groups", "gemv", shift=True, device=DEV)
    X = gen.activations(M, K, "groups", "gemv", device=DEV)
    p = w4.w4a16_pack(W, group=group)
    y = w4.w4a16_gemv(X, p)
    torch.cuda.synchronize()
    y_ref, mag = reference(gen.bits(X), gen.bits(W), group=group)
    assert_output_close(y, y_ref, mag, label=f"group {group} M={M}")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_gemv_oracle_packed_long_rows(group, M):
    """Packed inputs from the oracle, K = 14336 (the long-row kernels)."""
    N, K = 300, 14336
    W = gen.weights(N, K, "groups", "long", shift=True, device=DEV)
    Wb = gen.bits(W)
    codes, scales, zeros = O.quantize_pack(Wb, None, group)
    p = to_dev_packed(codes, scales, zeros)
    X = gen.activations(M, K, "groups", "long", device=DEV)
    y = w4.w4a16_gemv(X, p)
    torch.cuda.synchronize()
    rows = sample_rows(N, 48, seed=M)
    y_ref = O.matmul_ref(gen.bits(X), codes, scales, zeros, rows=rows)
    w_hat = O.dequantize(codes[rows], scales[rows], zeros[rows])
    mag = np.abs(O.bf16_to_f32(gen.bits(X)).astype(np.float64)) @ np.abs(w_hat).T
    assert_output_close(y[:, torch.as_tensor(rows, device=DEV)], y_ref, mag,
                        label=f"group {group} M={M} long")


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (256, 1000, 2048), (300, 130, 640), (129, 2000, 4096)])
def test_gemm(group, M, N, K):
    W = gen.weights(N, K, "groups", f"gemm{M}", shift=True, device=DEV)
    X = gen.activations(M, K, "groups", f"gemm{M}", device=DEV)
    p = w4.w4a16_pack(W, group=group)
    y = w4.w4a16_gemm(X, p)
    torch.cuda.synchronize()
    rows = sample_rows(N, 96, seed=N)
    y_ref, mag = reference(gen.bits(X), gen.bits(W), rows=rows, group=group)
    assert_output_close(y[:, torch.as_tensor(rows, device=DEV)], y_ref, mag,
                        label=f"group {group} gemm {M}x{N}x{K}")


@pytest.mark.parametrize("group", GROUPS)
def test_gemm_canaries_and_llama_prefill_sampled(group):
    # strided output with canaries around it
    M, N, K = 1000, 1300, 512
    W = gen.weights(N, K, "groups", "canary", shift=True, device=DEV)
    X = gen.activations(M, K, "groups", "canary", device=DEV)
    p = w4.w4a16_pack(W, group=group)
    canary = torch.full((M + 2, N + 16), -77.0, dtype=torch.bfloat16, device=DEV)
    out = canary[1:M + 1, 8:N + 8]
    w4.w4a16_gemm(X, p, out=out)
    torch.cuda.synchronize()
    inner = torch.zeros_like(canary, dtype=torch.bool)
    inner[1:M + 1, 8:N + 8] = True
    assert torch.all(canary[~inner] == -77.0), "write outside Y"
    rows, mrows = sample_rows(N, 64, seed=5), sample_rows(M, 40, seed=6)
    midx, ridx = torch.as_tensor(mrows, device=DEV), torch.as_tensor(rows, device=DEV)
    y_ref, mag = reference(gen.bits(X[midx]), gen.bits(W), rows=rows, group=group)
    assert_output_close(out[midx][:, ridx], y_ref, mag, label=f"group {group} canary")
    # the 8B-shaped down projection at M = 4096, sampled
    L = [l for l in gen.LLAMA8B if l.name == "down"][0]
    W = gen.weights(L.N, L.K, "groups", L.name, device=DEV)
    X = gen.activations(4096, L.K, "groups", L.name, device=DEV)
    p = w4.w4a16_pack(W, group=group)
    y = w4.w4a16_gemm(X, p)
    torch.cuda.synchronize()
    rows, mrows = sample_rows(L.N, 24, seed=7), sample_rows(4096, 16, seed=8)
    midx, ridx = torch.as_tensor(mrows, device=DEV), torch.as_tensor(rows, device=DEV)
    y_ref, mag = reference(gen.bits(X[midx]), gen.bits(W), rows=rows, group=group)
    assert_output_close(y[midx][:, ridx], y_ref, mag, label=f"group {group} down M=4096")


def test_group_128_is_the_default_path():
    """The grouped entry points with group 128 give the same bits as the
    plain ones."""
    N, K, M = 500, 1024, 300
    W = gen.weights(N, K, "groups", "g128", shift=True, device=DEV)
    X = gen.activations(M, K, "groups", "g128", device=DEV)
    p = w4.w4a16_pack(W)
    q = w4.empty_packed(N, K, DEV)
    st = w4.lib.w4a16_pack_grouped(w4._ptr(W), N, K, K, w4._ptr(None), 128, w4._ptr(q.codes),
                                   w4._ptr(q.scales), w4._ptr(q.zeros), w4._stream(W))
    assert st == 0
    for fn, gfn, m in ((w4.lib.w4a16_gemv, w4.lib.w4a16_gemv_grouped, 8),
                       (w4.lib.w4a16_gemm, w4.lib.w4a16_gemm_grouped, M)):
        a = torch.empty(m, N, dtype=torch.bfloat16, device=DEV)
        b = torch.empty_like(a)
        assert fn(w4._ptr(X), m, K, w4._ptr(p.codes), w4._ptr(p.scales), w4._ptr(p.zeros), N, K,
                  w4._ptr(a), N, w4._stream(X)) == 0
        assert gfn(w4._ptr(X), m, K, w4._ptr(p.codes), w4._ptr(p.scales), w4._ptr(p.zeros), N, K,
                   128, w4._ptr(b), N, w4._stream(X)) == 0
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    torch.cuda.synchronize()
    assert torch.equal(p.codes, q.codes) and torch.equal(p.zeros, q.zeros)
    assert torch.equal(p.scales.view(torch.int16), q.scales.view(torch.int16))


@pytest.mark.parametrize("group", GROUPS)
def test_linear_dispatch_boundary_and_awq(group):
    """w4a16_linear at the decode / prefill boundary (M = 32, 33) on AWQ
    pre-scaled weights packed with the smaller group."""
    N, K = 640, 1024
    W = gen.weights(N, K, "groups", "lin", shift=True, device=DEV)
    s = gen.channel_vector(K, "groups", "lin", "awq").to(DEV)
    p = w4.w4a16_pack(W, awq_s=s, group=group)
    for M in (32, 33):
        X = gen.activations(M, K, "groups", f"lin{M}", device=DEV)
        y = w4.w4a16_linear(X, p)
        torch.cuda.synchronize()
        y_ref, mag = reference(gen.bits(X), gen.bits(W), awq_s=s.cpu().numpy(), group=group)
        assert_output_close(y, y_ref, mag, label=f"group {group} linear M={M}")
