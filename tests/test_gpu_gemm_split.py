"""w4a16_gemm_ws (prefill with K split over blocks through a caller's
workspace) on the GPU against the CPU oracle: the split runs' float32
partial tiles are added in a fixed order and rounded once, so the result is
the same product as the unsplit kernel up to float32 summation order (Axe
Corsa model card, "The Two-Stage Pipeline": w_hat = (q - z) s for every
group, summed over all of K).  Sampled rows on the large shapes."""
import ctypes

import pytest
import torch

from synth import gen
from parity import assert_output_close, reference, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def ws_bytes(M, N, K):
    n = ctypes.c_int64(0)
    w4._check("w4a16_gemm_workspace_bytes", w4.lib.w4a16_gemm_workspace_bytes(M, N, K, ctypes.byref(n)))
    return n.value


def plain(X, p, out=None):
    """w4a16_gemm without a workspace: never splits K."""
    y = w4._matmul(w4.lib.w4a16_gemm, "w4a16_gemm", X, p, out)
    torch.cuda.synchronize()
    return y


def split(X, p, ws, out=None):
    y = w4.w4a16_gemm(X, p, out, workspace=ws)
    torch.cuda.synchronize()
    return y


def check(y, X, W, rows, mrows, label):
    if mrows is not None:
        midx = torch.as_tensor(mrows, device=DEV)
        X, y = X[midx], y[midx]
    ridx = torch.as_tensor(rows, device=DEV)
    y_ref, mag = reference(gen.bits(X), gen.bits(W[ridx]))
    return assert_output_close(y[:, ridx], y_ref, mag, label=label)


# (M, N, K): every tile split -- 256 x 256 tiles over 8 runs (2 x 12 tiles,
# K = 8192; N % 4 == 0 and not), over 4 runs (4 x 16 tiles, K = 14336, the
# down projection's shape), 128 x 128 tiles over 2 runs (the o projection's
# shape at M = 512) -- and one round of whole 256 x 256 tiles with the tiles
# past it split over 2 runs (4 x 80 tiles: 64 split; 4 x 79: 60 split, and a
# tile count that is not a multiple of the eight XCDs keeps the plain order)
SPLIT_SHAPES = [(300, 3000, 8192), (300, 3001, 8192), (1000, 4096, 14336), (512, 4096, 4096),
                (1000, 20400, 2048), (1000, 20200, 2048)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_split_against_the_oracle(M, N, K):
    W = gen.weights(N, K, "gemm", f"split{M}x{N}x{K}", shift=True, device=DEV)
    X = gen.activations(M, K, "gemm", f"split{M}x{N}x{K}", device=DEV)
    p = w4.w4a16_pack(W)
    need = ws_bytes(M, N, K)
    assert need > 0, (M, N, K)
    rows = sample_rows(N, 128, seed=N + K)
    mrows = sample_rows(M, 48, seed=M + K)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    # a strided output with canaries around it
    canary = torch.full((M + 2, N + 16), -77.0, dtype=torch.bfloat16, device=DEV)
    out = canary[1:M + 1, 8:N + 8]
    split(X, p, ws, out=out)
    inner = torch.zeros_like(canary, dtype=torch.bool)
    inner[1:M + 1, 8:N + 8] = True
    assert torch.all(canary[~inner] == -77.0), "write outside Y"
    check(out, X, W, rows, mrows, f"split {M}x{N}x{K}")
    ws.fill_(0xFF)   # any workspace contents: the runs overwrite their partials
    y2 = split(X, p, ws)
    assert torch.equal(out, y2), "split-K result not deterministic"
    y0 = plain(X, p)
    check(y0, X, W, rows, mrows, f"unsplit {M}x{N}x{K}")
    # the same product up to float32 summation order: within one BF16 ulp
    f0, f2 = y0.float(), y2.float()
    assert torch.all((f2 - f0).abs() <= 2.0 ** -7 * f0.abs() + 1e-3 * f0.abs().max())


def test_too_small_a_workspace_runs_the_unsplit_kernel():
    M, N, K = 300, 3000, 8192
    W = gen.weights(N, K, "gemm", "small_ws", device=DEV)
    X = gen.activations(M, K, "gemm", "small_ws", device=DEV)
    p = w4.w4a16_pack(W)
    need = ws_bytes(M, N, K)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    assert torch.equal(split(X, p, ws), plain(X, p))


def test_split_plans():
    tile = 256 * 256 * 4
    # whole rounds of large tiles: not split (the 8B-shaped gate_up at
    # M = 4096, 1792 tiles; o and down at M = 4096, 256 tiles)
    assert ws_bytes(4096, 28672, 4096) == 0
    assert ws_bytes(4096, 4096, 14336) == 0
    # a round and a half (qkv at M = 4096, 384 tiles; gate_up at M = 2048,
    # 896): the last 128 tiles over 2 runs
    assert ws_bytes(4096, 6144, 4096) == 2 * 128 * tile
    assert ws_bytes(2048, 28672, 4096) == 2 * 128 * tile
    # a remainder too large for half a round (gate_up at M = 1024, 448 tiles)
    assert ws_bytes(1024, 28672, 4096) == 0
    # too few large tiles: all split (down at M = 512: 32 tiles over 8 runs)
    assert ws_bytes(512, 4096, 14336) == 8 * 32 * tile
    # too few inputs per run
    assert ws_bytes(512, 4096, 1024) == 0


def test_split_in_a_replayed_graph():
    # no counters and no fills: every replay, with other work on the stream
    # between replays, gives the eager result bit for bit
    M, N, K = 1000, 4096, 14336
    W = gen.weights(N, K, "gemm", "split_graph", device=DEV)
    X = gen.activations(M, K, "gemm", "split_graph", device=DEV)
    p = w4.w4a16_pack(W)
    ws = torch.empty(ws_bytes(M, N, K), dtype=torch.uint8, device=DEV)
    y_eager = split(X, p, ws)
    y = torch.empty_like(y_eager)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        w4.w4a16_gemm(X, p, y, workspace=ws)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            w4.w4a16_gemm(X, p, y, workspace=ws)
    for i in range(3):
        y.fill_(0)
        y_other = plain(gen.activations(M, K, "gemm", f"split_graph{i}", device=DEV), p)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i} differs from the eager result"
        del y_other
