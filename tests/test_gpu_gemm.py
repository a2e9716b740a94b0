"""w4a16_gemm (prefill, matrix cores) on the GPU vs the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, reference, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def plain_gemm(X, p, out=None):
    """w4a16_gemm without a workspace: the tile kernels alone, never a split K."""
    return w4._matmul(w4.lib.w4a16_gemm, "w4a16_gemm", X, p, out)


def check_case(M, N, K, cfg, layer, shift=False, rows=None, mrows=None, label="", split=False):
    W = gen.weights(N, K, cfg, layer, shift=shift, device=DEV)
    X = gen.activations(M, K, cfg, layer, device=DEV)
    p = w4.w4a16_pack(W)
    y = w4.w4a16_gemm(X, p) if split else plain_gemm(X, p)
    torch.cuda.synchronize()
    if mrows is not None:
        midx = torch.as_tensor(mrows, device=DEV)
        X, y = X[midx], y[midx]
    if rows is None:
        y_ref, mag = reference(gen.bits(X), gen.bits(W))
        return assert_output_close(y, y_ref, mag, label=label)
    ridx = torch.as_tensor(rows, device=DEV)
    y_ref, mag = reference(gen.bits(X), gen.bits(W[ridx]))
    return assert_output_close(y[:, ridx], y_ref, mag, label=label)


@pytest.mark.parametrize("M,N,K", [
    (1, 16, 128), (7, 100, 384), (128, 128, 128), (129, 130, 256), (200, 333, 640),
    (256, 512, 1024), (33, 1000, 512), (512, 64, 2048)])
def test_small_full(M, N, K):
    check_case(M, N, K, "gemm", f"{M}x{N}x{K}", shift=True, label=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M", [512, 2048, 4096])
def test_llama8b_prefill_sampled(M):
    for layer in gen.LLAMA8B:
        rows = sample_rows(layer.N, 48, seed=layer.N + M)
        mrows = sample_rows(M, 32, seed=M + 7)
        # the binding's w4a16_gemm, with its cached workspace (K split where
        # the large tiles do not fill the CUs), and the tile kernels alone
        for split in (True, False):
            check_case(M, layer.N, layer.K, "llama8b_prefill", layer.name, rows=rows, mrows=mrows,
                       label=f"{layer.name} M={M} split={split}", split=split)
        torch.cuda.empty_cache()


def test_matches_gemv_for_small_m():
    N, K = 300, 2048
    W = gen.weights(N, K, "gemm", "vs_gemv", device=DEV)
    p = w4.w4a16_pack(W)
    for M in (1, 16, 32):
        X = gen.activations(M, K, "gemm", "vs_gemv", device=DEV)
        a = w4.w4a16_gemm(X, p)
        b = w4.w4a16_gemv(X, p)
        torch.cuda.synchronize()
        # same arithmetic up to float32 summation order: within one BF16 ulp
        fa = a.float(); fb = b.float()
        assert torch.all((fa - fb).abs() <= 2.0 ** -7 * fb.abs() + 1e-3)


def test_canaries_and_determinism():
    M, N, K = 150, 260, 512
    W = gen.weights(N, K, "gemm", "canary", device=DEV)
    p = w4.w4a16_pack(W)
    X = gen.activations(M, K, "gemm", "canary", device=DEV)
    canary = torch.full((M + 3, N + 24), -77.0, dtype=torch.bfloat16, device=DEV)
    out = canary[2:M + 2, 16:N + 16]
    plain_gemm(X, p, out=out)
    torch.cuda.synchronize()
    inner = torch.zeros_like(canary, dtype=torch.bool)
    inner[2:M + 2, 16:N + 16] = True
    assert torch.all(canary[~inner] == -77.0), "write outside Y"
    y2 = plain_gemm(X, p)
    torch.cuda.synchronize()
    assert torch.equal(out, y2)
    y_ref, mag = reference(gen.bits(X), gen.bits(W))
    assert_output_close(out, y_ref, mag, label="canary")


def test_large_tiles_ragged_with_canaries():
    # enough 256 x 256 tiles for the large-tile kernel (4 x 49 = 196, at least
    # three per four of the 256 CUs), ragged in M and N, written into a
    # strided view
    M, N, K = 1000, 12300, 384
    W = gen.weights(N, K, "gemm", "big_ragged", shift=True, device=DEV)
    p = w4.w4a16_pack(W)
    X = gen.activations(M, K, "gemm", "big_ragged", device=DEV)
    canary = torch.full((M + 3, N + 24), -77.0, dtype=torch.bfloat16, device=DEV)
    out = canary[1:M + 1, 8:N + 8]
    plain_gemm(X, p, out=out)
    torch.cuda.synchronize()
    inner = torch.zeros_like(canary, dtype=torch.bool)
    inner[1:M + 1, 8:N + 8] = True
    assert torch.all(canary[~inner] == -77.0), "write outside Y"
    rows = sample_rows(N, 96, seed=5)
    mrows = sample_rows(M, 48, seed=6)
    ridx = torch.as_tensor(rows, device=DEV)
    midx = torch.as_tensor(mrows, device=DEV)
    y_ref, mag = reference(gen.bits(X[midx]), gen.bits(W[ridx]))
    assert_output_close(out[midx][:, ridx], y_ref, mag, label="large tiles, ragged")


def test_tiny_tiles_long_rows():
    # few large tiles (2 x 8), and 64 x 128 tiles fill the CUs better than
    # 128 x 128 (80 against 48 blocks): the 64 x 128 kernel, ragged M, 32 groups
    check_case(300, 2000, 4096, "gemm", "small_long", shift=True, rows=sample_rows(2000, 64, seed=9),
               label="64x128 tiles, K=4096")


def test_small_tiles_ragged():
    # 48 large tiles; 128 x 128 (4 x 48 = 192 blocks) and 64 x 128 (384) fill
    # the same share of the CU rounds, so the 128 x 128 kernel; ragged M and N
    check_case(500, 6100, 512, "gemm", "small_ragged", shift=True, rows=sample_rows(6100, 64, seed=10),
               mrows=sample_rows(500, 48, seed=11), label="128x128 tiles, ragged")


def test_tile_choice_boundary():
    # just below and at the large-tile threshold (191 and 192 large tiles of
    # 256 x 256 on 256 CUs): both kernels, ragged M, against the oracle
    for M, N in ((200, 256 * 191 - 50), (200, 256 * 192 - 50)):
        check_case(M, N, 256, "gemm", f"boundary_{N}", shift=True, rows=sample_rows(N, 48, seed=N),
                   mrows=sample_rows(M, 32, seed=M), label=f"tile boundary {M}x{N}")
        torch.cuda.empty_cache()
