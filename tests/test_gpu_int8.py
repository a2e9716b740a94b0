"""W8A16 variant on the GPU against the CPU oracle: the 8-bit packer
(bit-exact) and the decode product, on the library's packing and on packed
inputs the oracle produced."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def u32(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def assert_int8_pack_equal(p, W_bits, rows=None, awq_s=None):
    if rows is None:
        rows = np.arange(W_bits.shape[0])
    codes, scales, zeros = O.quantize_pack_int8(W_bits[rows], awq_s)
    for name, a, b in (("codes", u32(p.codes)[rows], codes), ("scales", gen.bits(p.scales)[rows], scales),
                       ("zeros", p.zeros.cpu().numpy()[rows], zeros)):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            r, c = bad[0]
            raise AssertionError(f"{name} differ at {len(bad)} places; first row {rows[r]} col {c}: "
                                 f"gpu {a[r, c]:#x} oracle {b[r, c]:#x}")


def int8_reference(X_bits, codes, scales, zeros, rows=None):
    if rows is not None:
        codes, scales, zeros = codes[rows], scales[rows], zeros[rows]
    y_ref = O.matmul_ref_int8(X_bits, codes, scales, zeros)
    mag = np.abs(O.bf16_to_f32(X_bits).astype(np.float64)) @ np.abs(O.dequantize_int8(codes, scales, zeros)).T
    return y_ref, mag


@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (16, 4096), (257, 1024)])
def test_pack_bit_exact(N, K):
    W = gen.weights(N, K, "int8", f"{N}x{K}", shift=True, device=DEV)
    p = w4.w4a16_pack_int8(W)
    torch.cuda.synchronize()
    assert_int8_pack_equal(p, gen.bits(W))


def test_pack_awq_llama_shape_sampled():
    L = [l for l in gen.LLAMA8B if l.name == "gate_up"][0]
    W = gen.weights(L.N, L.K, "int8", L.name, shift=True, device=DEV)
    s = gen.channel_vector(L.K, "int8", L.name, "awq").to(DEV)
    p = w4.w4a16_pack_int8(W, awq_s=s)
    torch.cuda.synchronize()
    rows = sample_rows(L.N, 64, seed=8)
    codes, scales, zeros = O.quantize_pack_int8(gen.bits(W[torch.as_tensor(rows, device=DEV)]),
                                                s.cpu().numpy())
    assert np.array_equal(u32(p.codes)[rows], codes)
    assert np.array_equal(gen.bits(p.scales)[rows], scales)
    assert np.array_equal(p.zeros.cpu().numpy()[rows], zeros)


@pytest.mark.parametrize("N,K", [(100, 384), (1000, 2048), (8, 32768)])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_gemv_library_packed(M, N, K):
    W = gen.weights(N, K, "int8", f"g{N}x{K}", shift=True, device=DEV)
    X = gen.activations(M, K, "int8", f"g{N}x{K}", device=DEV)
    p = w4.w4a16_pack_int8(W)
    y = w4.w4a16_gemv_int8(X, p)
    torch.cuda.synchronize()
    codes, scales, zeros = O.quantize_pack_int8(gen.bits(W))
    y_ref, mag = int8_reference(gen.bits(X), codes, scales, zeros)
    assert_output_close(y, y_ref, mag, label=f"int8 M={M} {N}x{K}")


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_oracle_packed_llama_layers_sampled(M):
    """Random codes (all 256 values), scales and zero points from a seeded
    generator, the 8B-shaped layers, sampled rows."""
    rng = np.random.default_rng(60 + M)
    for L in gen.LLAMA8B:
        codes = rng.integers(0, 2 ** 32, size=(L.N, L.K // 4), dtype=np.uint64).astype(np.uint32)
        scales = O.f32_to_bf16_rtz(rng.uniform(1e-5, 1e-3, size=(L.N, L.K // 128)).astype(np.float32))
        zeros = rng.integers(0, 256, size=(L.N, L.K // 128)).astype(np.int32)
        p = w4.PackedLinearInt8(torch.from_numpy(codes.view(np.int32)).to(DEV), gen.from_bits(scales, DEV),
                                torch.from_numpy(zeros).to(DEV))
        X = gen.activations(M, L.K, "int8", L.name, device=DEV)
        # strided output with canary columns
        buf = torch.full((M, L.N + 8), -5.0, dtype=torch.bfloat16, device=DEV)
        y = buf[:, :L.N]
        w4.w4a16_gemv_int8(X, p, out=y)
        torch.cuda.synchronize()
        assert torch.all(buf[:, L.N:] == -5.0), "write outside Y"
        rows = sample_rows(L.N, 48, seed=L.N)
        y_ref, mag = int8_reference(gen.bits(X), codes, scales, zeros, rows)
        assert_output_close(y[:, torch.as_tensor(rows, device=DEV)], y_ref, mag,
                            label=f"int8 {L.name} M={M}")


@pytest.mark.parametrize("N,K", [(1, 128), (5, 256), (37, 32768)])
def test_gemv_edge_shapes(N, K):
    W = gen.weights(N, K, "int8", f"edge{N}x{K}", shift=True, device=DEV)
    p = w4.w4a16_pack_int8(W)
    torch.cuda.synchronize()
    assert_int8_pack_equal(p, gen.bits(W))
    codes, scales, zeros = O.quantize_pack_int8(gen.bits(W))
    for M in (1, 3):
        X = gen.activations(M, K, "int8", f"edge{N}x{K}", device=DEV)
        y = w4.w4a16_gemv_int8(X, p)
        torch.cuda.synchronize()
        y_ref, mag = int8_reference(gen.bits(X), codes, scales, zeros)
        assert_output_close(y, y_ref, mag, label=f"int8 edge M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (256, 1000, 2048), (300, 130, 640), (129, 2000, 4096)])
def test_gemm(M, N, K):
    W = gen.weights(N, K, "int8", f"gemm{M}", shift=True, device=DEV)
    X = gen.activations(M, K, "int8", f"gemm{M}", device=DEV)
    p = w4.w4a16_pack_int8(W)
    y = w4.w4a16_gemm_int8(X, p)
    torch.cuda.synchronize()
    codes, scales, zeros = O.quantize_pack_int8(gen.bits(W))
    rows = sample_rows(N, 96, seed=N)
    y_ref, mag = int8_reference(gen.bits(X), codes, scales, zeros, rows)
    assert_output_close(y[:, torch.as_tensor(rows, device=DEV)], y_ref, mag, label=f"int8 gemm {M}x{N}x{K}")


def test_gemm_oracle_packed_canaries_and_llama_prefill_sampled():
    # random 8-bit codes from a seeded generator, strided output with canaries
    M, N, K = 1000, 1300, 512
    rng = np.random.default_rng(70)
    codes = rng.integers(0, 2 ** 32, size=(N, K // 4), dtype=np.uint64).astype(np.uint32)
    scales = O.f32_to_bf16_rtz(rng.uniform(1e-5, 1e-3, size=(N, K // 128)).astype(np.float32))
    zeros = rng.integers(0, 256, size=(N, K // 128)).astype(np.int32)
    p = w4.PackedLinearInt8(torch.from_numpy(codes.view(np.int32)).to(DEV), gen.from_bits(scales, DEV),
                            torch.from_numpy(zeros).to(DEV))
    X = gen.activations(M, K, "int8", "canary", device=DEV)
    canary = torch.full((M + 2, N + 16), -77.0, dtype=torch.bfloat16, device=DEV)
    out = canary[1:M + 1, 8:N + 8]
    w4.w4a16_gemm_int8(X, p, out=out)
    torch.cuda.synchronize()
    inner = torch.zeros_like(canary, dtype=torch.bool)
    inner[1:M + 1, 8:N + 8] = True
    assert torch.all(canary[~inner] == -77.0), "write outside Y"
    rows, mrows = sample_rows(N, 64, seed=71), sample_rows(M, 40, seed=72)
    midx, ridx = torch.as_tensor(mrows, device=DEV), torch.as_tensor(rows, device=DEV)
    y_ref, mag = int8_reference(gen.bits(X[midx]), codes, scales, zeros, rows)
    assert_output_close(out[midx][:, ridx], y_ref, mag, label="int8 gemm canary")
    # the 8B-shaped gate_up projection at M = 4096, sampled
    L = [l for l in gen.LLAMA8B if l.name == "gate_up"][0]
    W = gen.weights(L.N, L.K, "int8", L.name, device=DEV)
    X = gen.activations(4096, L.K, "int8", L.name, device=DEV)
    p = w4.w4a16_pack_int8(W)
    y = w4.w4a16_gemm_int8(X, p)
    torch.cuda.synchronize()
    rows, mrows = sample_rows(L.N, 24, seed=73), sample_rows(4096, 16, seed=74)
    midx, ridx = torch.as_tensor(mrows, device=DEV), torch.as_tensor(rows, device=DEV)
    codes, scales, zeros = O.quantize_pack_int8(gen.bits(W[ridx]))
    y_ref, mag = int8_reference(gen.bits(X[midx]), codes, scales, zeros)
    assert_output_close(y[midx][:, ridx], y_ref, mag, label="int8 gate_up M=4096")
