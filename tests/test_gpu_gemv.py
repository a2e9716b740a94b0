"""w4a16_gemv (decode, M <= 32) on the GPU vs the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, reference, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def run(fn, X, p):
    y = fn(X, p)
    torch.cuda.synchronize()
    return y


def check_case(fn, M, N, K, cfg, layer, shift=False, rows=None, label=""):
    W = gen.weights(N, K, cfg, layer, shift=shift, device=DEV)
    X = gen.activations(M, K, cfg, layer, device=DEV)
    p = w4.w4a16_pack(W)
    y = run(fn, X, p)
    if rows is None:
        y_ref, mag = reference(gen.bits(X), gen.bits(W))
        return assert_output_close(y, y_ref, mag, label=label)
    ridx = torch.as_tensor(rows, device=DEV)
    y_ref, mag = reference(gen.bits(X), gen.bits(W[ridx]))
    return assert_output_close(y[:, ridx], y_ref, mag, label=label)


@pytest.mark.parametrize("M", list(range(1, 33)))
def test_every_m_ragged_small(M):
    # 100 rows = six full 16-row tiles and a ragged tail; three groups
    check_case(w4.w4a16_gemv, M, 100, 384, "gemv", "small", shift=True, label=f"M={M}")


@pytest.mark.parametrize("N,K", [(1, 128), (17, 128), (16, 256), (40, 2048), (3, 14336)])
def test_edge_shapes(N, K):
    for M in (1, 5, 16, 17, 32):
        check_case(w4.w4a16_gemv, M, N, K, "gemv", f"edge{N}x{K}", label=f"M={M} N={N} K={K}")


def test_single_linear_4096_full():
    rel, _ = check_case(w4.w4a16_gemv, 1, 4096, 4096, 1, "linear", label="4096x4096")
    assert rel < 2e-3


@pytest.mark.parametrize("M", [1, 4, 8, 16, 32])
def test_llama8b_layers_sampled(M):
    for layer in gen.LLAMA8B:
        rows = sample_rows(layer.N, 256, seed=layer.N + M)
        check_case(w4.w4a16_gemv, M, layer.N, layer.K, "llama8b_decode", layer.name, rows=rows,
                   label=f"{layer.name} M={M}")


@pytest.mark.parametrize("M", [1, 8, 32])
def test_llama70b_layers_sampled(M):
    for layer in gen.LLAMA70B:
        rows = sample_rows(layer.N, 96, seed=layer.N + M)
        check_case(w4.w4a16_gemv, M, layer.N, layer.K, "llama70b_decode", layer.name, shift=True,
                   rows=rows, label=f"{layer.name} M={M}")
        torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 3, 8])
def test_stack40_layers_sampled(M):
    # one layer of the 40-layer stack (K = 5120, 27648: slices not a power of two)
    for layer in gen.STACK40_LAYER:
        rows = sample_rows(layer.N, 96, seed=layer.N + 7 * M)
        check_case(w4.w4a16_gemv, M, layer.N, layer.K, "stack40_decode", layer.name, rows=rows,
                   label=f"{layer.name} M={M}")
        torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [3, 4, 5, 8])
@pytest.mark.parametrize("N,K", [(37, 640), (256, 8320), (64, 16384), (29, 16512), (2048, 20480),
                                 (40, 33024)])
def test_matrix_core_small_m_shapes(M, N, K):
    # ragged row counts, partial 512-input slices, two slices per wave, just
    # past the two-slice limit (long-row kernel, or the dot kernel for few
    # rows), and rows longer than the dot kernel takes
    check_case(w4.w4a16_gemv, M, N, K, "gemv", f"quad{N}x{K}", shift=True, label=f"M={M} N={N} K={K}")


@pytest.mark.parametrize("N,K", [(28669, 4096), (16379, 4096), (10233, 2048)])
def test_matrix_core_small_m_long_blocks_ragged(N, K):
    # row counts whose even fill of the CUs takes 14, 16 and 10 four-row
    # batches per block, each with a partial last block (its rows clamp)
    tail = np.arange(N - 64, N)
    for M in (3, 6, 8):
        rows = np.unique(np.concatenate([sample_rows(N, 96, seed=N + M), tail]))
        check_case(w4.w4a16_gemv, M, N, K, "gemv", f"quadnb{N}x{K}", shift=True, rows=rows,
                   label=f"M={M} N={N} K={K}")


def test_on_grid_weights_match_unquantised_matmul():
    import oracle_pins as P
    W_bits, _ = P.check_all_codes_on_grid(seed=31, N=80, K=512)
    W = gen.from_bits(W_bits, DEV)
    for M in (1, 13, 32):
        X = gen.activations(M, 512, "gemv", "grid", device=DEV)
        y = run(w4.w4a16_gemv, X, w4.w4a16_pack(W))
        exact = O.bf16_to_f32(gen.bits(X)).astype(np.float64) @ O.bf16_to_f32(W_bits).astype(np.float64).T
        mag = np.abs(O.bf16_to_f32(gen.bits(X)).astype(np.float64)) @ np.abs(
            O.bf16_to_f32(W_bits).astype(np.float64)).T
        assert_output_close(y, exact, mag, label=f"on-grid M={M}")


def test_strides_canaries_and_determinism():
    M, N, K = 9, 200, 1024
    W = gen.weights(N, K, "gemv", "stride", device=DEV)
    p = w4.w4a16_pack(W)
    Xbig = gen.activations(M, K + 64, "gemv", "stride", device=DEV)
    X = Xbig[:, 16:K + 16]                      # ldx = K + 64, 16-byte aligned start
    canary = torch.full((M + 2, N + 40), 1234.0, dtype=torch.bfloat16, device=DEV)
    out = canary[1:M + 1, 8:N + 8]             # ldy = N + 40
    w4.w4a16_gemv(X, p, out=out)
    torch.cuda.synchronize()
    inner = torch.zeros_like(canary, dtype=torch.bool)
    inner[1:M + 1, 8:N + 8] = True
    assert torch.all(canary[~inner] == 1234.0), "write outside Y"
    y_ref, mag = reference(gen.bits(X.contiguous()), gen.bits(W))
    assert_output_close(out, y_ref, mag, label="strided")
    y2 = torch.empty_like(out)
    w4.w4a16_gemv(X, p, out=y2)
    torch.cuda.synchronize()
    assert torch.equal(out, y2)


def test_zero_points_outside_code_range():
    # all-positive and all-negative groups give zero points far outside 0..15
    N, K = 64, 512
    W = gen.weights(N, K, "gemv", "far", device=DEV).float()
    W = torch.where(torch.arange(N, device=DEV)[:, None] % 2 == 0, W.abs() + 0.5, -W.abs() - 2.0)
    W = W.to(torch.bfloat16)
    p = w4.w4a16_pack(W)
    z = p.zeros.cpu().numpy()
    assert z.min() < -50 and z.max() > 50
    X = gen.activations(7, K, "gemv", "far", device=DEV)
    y = run(w4.w4a16_gemv, X, p)
    y_ref, mag = reference(gen.bits(X), gen.bits(W))
    assert_output_close(y, y_ref, mag, label="far zero points")
