"""Dense BF16 comparisons on the GPU against the CPU oracle: the offline BF16
expansion of packed weights (bit-exact) and the dense decode / prefill
products.  Packed inputs come from the oracle's packer or from a seeded
generator, never from the library."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def to_dev_packed(codes, scales, zeros):
    c = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32)).to(DEV)
    s = gen.from_bits(scales, device=DEV)
    z = torch.from_numpy(np.ascontiguousarray(zeros, dtype=np.int32)).to(DEV)
    return w4.PackedLinear(c, s, z)


def random_packed(N, K, seed):
    """Seeded packed inputs: any codes, positive normal BF16 scales, zero
    points around the code range (the generator draws them; no arithmetic
    of the method)."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    scales = O.f32_to_bf16_rtz(rng.uniform(1e-4, 0.05, size=(N, K // 128)).astype(np.float32))
    zeros = rng.integers(-40, 56, size=(N, K // 128)).astype(np.int32)
    return codes, scales, zeros


def dense_reference(X_bits, W_bits, rows=None):
    y_ref = O.dense_matmul_ref(X_bits, W_bits, rows)
    W = W_bits if rows is None else W_bits[rows]
    mag = np.abs(O.bf16_to_f32(X_bits).astype(np.float64)) @ np.abs(O.bf16_to_f32(W).astype(np.float64)).T
    return y_ref, mag


@pytest.mark.parametrize("N,K", [(37, 128), (300, 640), (64, 4096), (1000, 384)])
def test_dequantize_bit_exact_oracle_packed(N, K):
    W = gen.weights(N, K, "dense", f"deq_{N}x{K}", shift=True, device=DEV)
    codes, scales, zeros = O.quantize_pack(gen.bits(W))
    p = to_dev_packed(codes, scales, zeros)
    # strided output with canary columns
    buf = torch.full((N, K + 8), -3.0, dtype=torch.bfloat16, device=DEV)
    out = buf[:, :K]
    w4.w4a16_dequantize_bf16(p, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(gen.bits(out), O.dequantize_bf16(codes, scales, zeros))
    assert torch.all(buf[:, K:] == -3.0), "write outside W"


def test_dequantize_bit_exact_llama_shape_sampled():
    N, K = 28672, 4096
    codes, scales, zeros = random_packed(N, K, seed=21)
    p = to_dev_packed(codes, scales, zeros)
    out = w4.w4a16_dequantize_bf16(p)
    torch.cuda.synchronize()
    rows = sample_rows(N, 64, seed=22)
    got = gen.bits(out[torch.as_tensor(rows, device=DEV)])
    assert np.array_equal(got, O.dequantize_bf16(codes[rows], scales[rows], zeros[rows]))
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N,K", [(37, 128), (1000, 384), (256, 4096), (100, 14336)])
def test_dense_gemv_small(N, K):
    W = gen.weights(N, K, "dense", f"gemv_{N}x{K}", device=DEV)
    Wb = gen.bits(W)
    for M in range(1, w4.DENSE_GEMV_MAX_M + 1):
        X = gen.activations(M, K, "dense", f"gemv_{N}x{K}", device=DEV)
        y = w4.w4a16_dense_gemv(X, W)
        torch.cuda.synchronize()
        y_ref, mag = dense_reference(gen.bits(X), Wb)
        assert_output_close(y, y_ref, mag, label=f"dense gemv M={M} {N}x{K}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_dense_gemv_llama8b_sampled(M):
    for layer in gen.LLAMA8B:
        W = gen.weights(layer.N, layer.K, "dense", layer.name, device=DEV)
        X = gen.activations(M, layer.K, "dense", layer.name, device=DEV)
        y = w4.w4a16_dense_gemv(X, W)
        torch.cuda.synchronize()
        rows = sample_rows(layer.N, 48, seed=layer.N + M)
        Wb = gen.bits(W[torch.as_tensor(rows, device=DEV)])
        y_ref, mag = dense_reference(gen.bits(X), Wb)
        assert_output_close(y[:, torch.as_tensor(rows, device=DEV)], y_ref, mag,
                            label=f"dense gemv {layer.name} M={M}")
        del W
        torch.cuda.empty_cache()


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (129, 130, 256), (300, 2000, 4096), (7, 100, 384)])
def test_dense_gemm_small(M, N, K):
    W = gen.weights(N, K, "dense", f"gemm_{M}x{N}x{K}", device=DEV)
    X = gen.activations(M, K, "dense", f"gemm_{M}x{N}x{K}", device=DEV)
    y = w4.w4a16_dense_gemm(X, W)
    torch.cuda.synchronize()
    rows = sample_rows(N, 96, seed=N + K)
    y_ref, mag = dense_reference(gen.bits(X), gen.bits(W), rows)
    assert_output_close(y[:, torch.as_tensor(rows, device=DEV)], y_ref, mag, label=f"dense gemm {M}x{N}x{K}")


def test_dense_gemm_ragged_canaries():
    M, N, K = 1000, 8300, 384
    W = gen.weights(N, K, "dense", "gemm_canary", device=DEV)
    X = gen.activations(M, K, "dense", "gemm_canary", device=DEV)
    canary = torch.full((M + 3, N + 24), -77.0, dtype=torch.bfloat16, device=DEV)
    out = canary[1:M + 1, 8:N + 8]
    w4.w4a16_dense_gemm(X, W, out=out)
    torch.cuda.synchronize()
    inner = torch.zeros_like(canary, dtype=torch.bool)
    inner[1:M + 1, 8:N + 8] = True
    assert torch.all(canary[~inner] == -77.0), "write outside Y"
    rows = sample_rows(N, 64, seed=31)
    mrows = sample_rows(M, 48, seed=32)
    midx = torch.as_tensor(mrows, device=DEV)
    ridx = torch.as_tensor(rows, device=DEV)
    y_ref, mag = dense_reference(gen.bits(X[midx]), gen.bits(W), rows)
    assert_output_close(out[midx][:, ridx], y_ref, mag, label="dense gemm ragged")


def test_dense_gemm_llama8b_prefill_sampled():
    M = 4096
    for layer in gen.LLAMA8B:
        W = gen.weights(layer.N, layer.K, "dense", layer.name, device=DEV)
        X = gen.activations(M, layer.K, "dense", layer.name, device=DEV)
        y = w4.w4a16_dense_gemm(X, W)
        torch.cuda.synchronize()
        rows = sample_rows(layer.N, 32, seed=layer.N)
        mrows = sample_rows(M, 24, seed=layer.K)
        midx = torch.as_tensor(mrows, device=DEV)
        ridx = torch.as_tensor(rows, device=DEV)
        y_ref, mag = dense_reference(gen.bits(X[midx]), gen.bits(W), rows)
        assert_output_close(y[midx][:, ridx], y_ref, mag, label=f"dense gemm {layer.name}")
        del W, X, y
        torch.cuda.empty_cache()


def test_dense_of_expansion_matches_fused_on_grid():
    """Weights already on the BF16 grid of the expansion (power-of-two
    scales, small |q - z|): the dense product of the expanded weights and
    the fused product agree to float32 summation order."""
    N, K, M = 512, 1024, 64
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    scales = O.f32_to_bf16_rtz((2.0 ** rng.integers(-9, -4, size=(N, K // 128))).astype(np.float32))
    zeros = rng.integers(-8, 24, size=(N, K // 128)).astype(np.int32)
    p = to_dev_packed(codes, scales, zeros)
    Wd = w4.w4a16_dequantize_bf16(p)
    X = gen.activations(M, K, "dense", "grid", device=DEV)
    a = w4.w4a16_dense_gemm(X, Wd).float()
    b = w4.w4a16_gemm(X, p).float()
    torch.cuda.synchronize()
    assert torch.all((a - b).abs() <= 2.0 ** -7 * b.abs() + 1e-3)
