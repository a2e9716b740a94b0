"""The decode kernels that can split K through a caller's workspace, against
the CPU oracle: for 9 <= M <= 32 the walk over row tiles (rows of at most 32
groups), the walk that splits K over blocks (longer rows), and the ring
kernel that takes longer rows without a workspace (and rows too long for the
small-M kernels); for 3 <= M <= 8 the four-row matrix-core kernel with and
without its K split.  Outputs are the oracle's fp64 product of the
packed matrix (Axe Corsa model card, "The Two-Stage Pipeline"), sampled
rows on the large shapes."""
import ctypes

import numpy as np
import pytest
import torch

from synth import gen
from parity import assert_output_close, reference, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def ws_bytes(M, N, K):
    n = ctypes.c_int64(0)
    w4._check("w4a16_gemv_workspace_bytes", w4.lib.w4a16_gemv_workspace_bytes(M, N, K, ctypes.byref(n)))
    return n.value


def plain(X, p):
    """w4a16_gemv: no workspace, never splits K."""
    y = w4._matmul(w4.lib.w4a16_gemv, "w4a16_gemv", X, p, None)
    torch.cuda.synchronize()
    return y


def split(X, p, ws):
    y = w4.w4a16_gemv(X, p, workspace=ws)
    torch.cuda.synchronize()
    return y


def check(y, X, W, rows, label):
    if rows is None:
        y_ref, mag = reference(gen.bits(X), gen.bits(W))
        return assert_output_close(y, y_ref, mag, label=label)
    ridx = torch.as_tensor(rows, device=DEV)
    y_ref, mag = reference(gen.bits(X), gen.bits(W[ridx]))
    return assert_output_close(y[:, ridx], y_ref, mag, label=label)


# (N, K): short rows (one block's 32 groups), rows of 36, 64 and 112 groups
# (two, two and four runs), ragged row counts
SHAPES = [(300, 4096), (40, 4608), (700, 8192), (3000, 14336), (5, 14336)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_split_and_unsplit_against_the_oracle(N, K):
    W = gen.weights(N, K, "gemv", f"paths{N}x{K}", shift=True, device=DEV)
    p = w4.w4a16_pack(W)
    rows = sample_rows(N, 160, seed=N + K) if N > 500 else None
    for M in (9, 16, 17, 32):
        X = gen.activations(M, K, "gemv", f"paths{N}x{K}", device=DEV)
        need = ws_bytes(M, N, K)
        assert (need > 0) == (K > 4096), (M, N, K, need)
        y0 = plain(X, p)
        check(y0, X, W, rows, f"unsplit M={M} N={N} K={K}")
        if need:
            ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
            y1 = split(X, p, ws)
            check(y1, X, W, rows, f"split M={M} N={N} K={K}")
            y2 = split(X, p, ws)
            assert torch.equal(y1, y2), "split-K result not deterministic"
            # each launch leaves the counters (first 64 KiB) at zero
            assert int(ws[:65536].count_nonzero()) == 0


# (N, K) for 3 <= M <= 8: two runs of one slice per wave (K = 14336, 9216,
# 16384), four runs (28672), four runs of 13.5 slices (27648; at N = 2555 ten
# batches per block, the last range ragged)
QUAD_SPLIT_SHAPES = [(300, 14336), (40, 28672), (700, 27648), (2555, 27648), (37, 9216), (5, 16384)]


@pytest.mark.parametrize("N,K", QUAD_SPLIT_SHAPES)
def test_small_m_split_and_unsplit_against_the_oracle(N, K):
    W = gen.weights(N, K, "gemv", f"qsplit{N}x{K}", shift=True, device=DEV)
    p = w4.w4a16_pack(W)
    rows = sample_rows(N, 160, seed=N + K) if N > 500 else None
    for M in (3, 4, 5, 8):
        X = gen.activations(M, K, "gemv", f"qsplit{N}x{K}", device=DEV)
        need = ws_bytes(M, N, K)
        assert need > 0, (M, N, K, need)
        y0 = plain(X, p)
        check(y0, X, W, rows, f"unsplit M={M} N={N} K={K}")
        if need:
            ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
            y1 = split(X, p, ws)
            check(y1, X, W, rows, f"split M={M} N={N} K={K}")
            y2 = split(X, p, ws)
            assert torch.equal(y1, y2), "split-K result not deterministic"
            assert int(ws[:65536].count_nonzero()) == 0


def test_one_workspace_serves_a_sequence_of_shapes():
    shapes = [(700, 8192, 32), (300, 14336, 5), (300, 4096, 16), (3000, 14336, 9), (40, 28672, 8),
              (40, 4608, 17), (37, 9216, 3), (700, 8192, 9)]
    need = max(ws_bytes(M, N, K) for N, K, M in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (N, K, M) in enumerate(shapes):
        W = gen.weights(N, K, "gemv", f"seq{i}", device=DEV)
        X = gen.activations(M, K, "gemv", f"seq{i}", device=DEV)
        y = split(X, w4.w4a16_pack(W), ws)
        check(y, X, W, sample_rows(N, 128, seed=i) if N > 500 else None, f"sequence {i}: M={M} N={N} K={K}")
    assert int(ws[:65536].count_nonzero()) == 0


def test_too_small_a_workspace_runs_the_unsplit_kernel():
    M, N, K = 16, 500, 8192
    W = gen.weights(N, K, "gemv", "small_ws", device=DEV)
    X = gen.activations(M, K, "gemv", "small_ws", device=DEV)
    p = w4.w4a16_pack(W)
    need = ws_bytes(M, N, K)
    assert need > 0
    ws = torch.zeros(need - 64, dtype=torch.uint8, device=DEV)
    assert torch.equal(split(X, p, ws), plain(X, p))


@pytest.mark.parametrize("M", [1, 2])
def test_rows_too_long_for_the_small_m_kernels(M):
    # K > 32768: past the dot kernel's slices, so the ring kernel runs
    N, K = 37, 33024
    W = gen.weights(N, K, "gemv", "longrow", shift=True, device=DEV)
    X = gen.activations(M, K, "gemv", "longrow", device=DEV)
    check(plain(X, w4.w4a16_pack(W)), X, W, None, f"long rows M={M}")


@pytest.mark.parametrize("M,N,K", [(8, 300, 14336), (5, 40, 28672), (4, 2555, 27648), (16, 700, 8192),
                                   (32, 3000, 14336)])
def test_split_k_in_a_replayed_graph(M, N, K):
    # the split paths' counters reset themselves inside each launch (no fill
    # is recorded in the graph): every replay, with other work on the stream
    # between replays, gives the eager result bit for bit
    W = gen.weights(N, K, "gemv", f"graph{N}x{K}", device=DEV)
    X = gen.activations(M, K, "gemv", f"graph{N}x{K}", device=DEV)
    p = w4.w4a16_pack(W)
    need = ws_bytes(M, N, K)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    y_eager = split(X, p, ws)
    y = torch.empty_like(y_eager)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        w4.w4a16_gemv(X, p, y, workspace=ws)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            w4.w4a16_gemv(X, p, y, workspace=ws)
    for i in range(4):
        y.fill_(0)
        y_other = plain(gen.activations(M, K, "gemv", f"graph{i}", device=DEV), p)   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i} differs from the eager result"
        assert int(ws[:65536].count_nonzero()) == 0
        del y_other
