"""Thin Python binding of the W4A16 HIP library (libw4a16.so).

The functions below carry the names of the C entry points in
include/w4a16.h and only marshal arguments: they check dtypes, devices and
shapes of torch tensors, allocate outputs with torch, pass raw device
pointers and the current HIP stream to the library, and turn a non-zero
status into an exception.  Every arithmetic step runs in the library's
kernels; there is no fallback path.  If the library is missing the import
of this package fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw4a16.so")

GROUP = 128
GEMV_MAX_M = 32
DENSE_GEMV_MAX_M = 8

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m int4_weight_only_gemv_amd.build)")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "w4a16_abi_version": ([], ctypes.c_int),
    "w4a16_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "w4a16_pack": ([_p, _i64, _i64, _i64, _p, _p, _p, _p, _p], ctypes.c_int),
    "w4a16_gemv": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_gemv_workspace_bytes": ([_i64, _i64, _i64, _p], ctypes.c_int),
    "w4a16_gemv_ws": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_gemm": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_gemm_workspace_bytes": ([_i64, _i64, _i64, _p], ctypes.c_int),
    "w4a16_gemm_ws": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_awq_importance": ([_p, _i64, _i64, _i64, _p, _p], ctypes.c_int),
    "w4a16_awq_scale": ([_p, _i64, ctypes.c_float, _p, _p], ctypes.c_int),
    "w4a16_awq_fold": ([_p, _i64, _p, _p, _p], ctypes.c_int),
    "w4a16_scale_channels": ([_p, _i64, _i64, _i64, _p, _p, _i64, _p], ctypes.c_int),
    "w4a16_pack_symmetric": ([_p, _i64, _i64, _i64, _p, _p, _p, _p, _p], ctypes.c_int),
    "w4a16_dequantize_bf16": ([_p, _p, _p, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_dense_gemv": ([_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_dense_gemm": ([_p, _i64, _i64, _p, _i64, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_pack_grouped": ([_p, _i64, _i64, _i64, _p, _i64, _p, _p, _p, _p], ctypes.c_int),
    "w4a16_pack_int8": ([_p, _i64, _i64, _i64, _p, _p, _p, _p, _p], ctypes.c_int),
    "w4a16_gemv_int8": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_gemm_int8": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_gemv_grouped": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_gemm_grouped": ([_p, _i64, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _i64, _p], ctypes.c_int),
    "w4a16_awq_search_error": ([_p, _i64, _p, _i64, _i64, _i64, _p, _p], ctypes.c_int),
    "w4a16_hbm_read_probe": ([_p, _i64, _p, _p], ctypes.c_int),
    "w4a16_chain_workspace_bytes": ([ctypes.c_int, _p], ctypes.c_int),
    "w4a16_chain_prepare": ([_p, ctypes.c_int, _i64, _p, _i64, _p, _p], ctypes.c_int),
    "w4a16_chain_run": ([_p, _p, _i64, _p], ctypes.c_int),
    "w4a16_chain_status": ([_p, _p, _p], ctypes.c_int),
    "w4a16_chain_run_noalloc": ([_p, ctypes.c_int, _i64, _p, _i64, _p, _p], ctypes.c_int),
}
for _name, (_args, _ret) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _ret

EXPORTS = tuple(_SIGS)


class W4A16Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {lib.w4a16_strerror(status).decode()}")


def _check(fn: str, status: int):
    if status != 0:
        raise W4A16Error(fn, status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, dtype, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous along its last dim")


def abi_version() -> int:
    return lib.w4a16_abi_version()


class PackedLinear:
    """A packed weight matrix: codes [N][K/8] int32 (uint32 bits),
    scales [N][K/group] bfloat16, zeros [N][K/group] int32; the group size
    (32, 64 or 128) follows from the shapes."""

    __slots__ = ("codes", "scales", "zeros", "N", "K", "group")

    def __init__(self, codes, scales, zeros):
        self.codes, self.scales, self.zeros = codes, scales, zeros
        self.N = codes.shape[0]
        self.K = codes.shape[1] * 8
        self.group = self.K // scales.shape[1] if scales.shape[1] else GROUP

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.zeros))


def empty_packed(N: int, K: int, device, group: int = GROUP) -> PackedLinear:
    codes = torch.empty(N, K // 8, dtype=torch.int32, device=device)
    scales = torch.empty(N, K // group, dtype=torch.bfloat16, device=device)
    zeros = torch.empty(N, K // group, dtype=torch.int32, device=device)
    return PackedLinear(codes, scales, zeros)


def _pack(fn, name, W, awq_s, out, group=None):
    _need(W, torch.bfloat16, "W", 2)
    N, K = W.shape
    if awq_s is not None:
        _need(awq_s, torch.float32, "awq_s", 1)
        if awq_s.shape[0] != K or not awq_s.is_contiguous():
            raise ValueError("awq_s must be a contiguous float32 [K]")
    p = out if out is not None else empty_packed(N, K, W.device, group or GROUP)
    if group is None:
        _check(name, fn(_ptr(W), N, K, W.stride(0), _ptr(awq_s), _ptr(p.codes), _ptr(p.scales),
                        _ptr(p.zeros), _stream(W)))
    else:
        if p.group != group:
            raise ValueError("out has the wrong group size")
        _check(name, fn(_ptr(W), N, K, W.stride(0), _ptr(awq_s), group, _ptr(p.codes),
                        _ptr(p.scales), _ptr(p.zeros), _stream(W)))
    return p


def w4a16_pack(W: torch.Tensor, awq_s: torch.Tensor | None = None,
               out: PackedLinear | None = None, group: int = GROUP) -> PackedLinear:
    """Quantise + pack a BF16 weight [N][K] (see w4a16_pack in w4a16.h);
    group 32 or 64 goes through w4a16_pack_grouped."""
    if group == GROUP:
        return _pack(lib.w4a16_pack, "w4a16_pack", W, awq_s, out)
    return _pack(lib.w4a16_pack_grouped, "w4a16_pack_grouped", W, awq_s, out, group)


def w4a16_pack_symmetric(W: torch.Tensor, awq_s: torch.Tensor | None = None,
                         out: PackedLinear | None = None) -> PackedLinear:
    """Symmetric INT4 variant (zero point 8; see w4a16_pack_symmetric)."""
    return _pack(lib.w4a16_pack_symmetric, "w4a16_pack_symmetric", W, awq_s, out)


class PackedLinearInt8:
    """W8A16 packed matrix: codes [N][K/4] int32 (four 8-bit codes per word),
    scales [N][K/128] bfloat16, zeros [N][K/128] int32."""

    __slots__ = ("codes", "scales", "zeros", "N", "K")

    def __init__(self, codes, scales, zeros):
        self.codes, self.scales, self.zeros = codes, scales, zeros
        self.N = codes.shape[0]
        self.K = codes.shape[1] * 4

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.zeros))


def w4a16_pack_int8(W: torch.Tensor, awq_s: torch.Tensor | None = None) -> PackedLinearInt8:
    """W8A16 quantise + pack (see w4a16_pack_int8 in w4a16.h)."""
    _need(W, torch.bfloat16, "W", 2)
    N, K = W.shape
    if awq_s is not None:
        _need(awq_s, torch.float32, "awq_s", 1)
        if awq_s.shape[0] != K or not awq_s.is_contiguous():
            raise ValueError("awq_s must be a contiguous float32 [K]")
    p = PackedLinearInt8(torch.empty(N, K // 4, dtype=torch.int32, device=W.device),
                         torch.empty(N, K // GROUP, dtype=torch.bfloat16, device=W.device),
                         torch.empty(N, K // GROUP, dtype=torch.int32, device=W.device))
    _check("w4a16_pack_int8", lib.w4a16_pack_int8(_ptr(W), N, K, W.stride(0), _ptr(awq_s), _ptr(p.codes),
                                                  _ptr(p.scales), _ptr(p.zeros), _stream(W)))
    return p


def w4a16_gemv_int8(X: torch.Tensor, p: PackedLinearInt8, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X . w_hat^T for 8-bit codes, 1 <= M <= 4 (decode)."""
    return _matmul(lib.w4a16_gemv_int8, "w4a16_gemv_int8", X, p, out)


def w4a16_gemm_int8(X: torch.Tensor, p: PackedLinearInt8, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X . w_hat^T for 8-bit codes on the matrix cores, any M (prefill)."""
    return _matmul(lib.w4a16_gemm_int8, "w4a16_gemm_int8", X, p, out)


def packed_from_i64(codes_i64: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor) -> PackedLinear:
    """A packed matrix whose codes sit in an I64 container [N][K/16] (sixteen
    codes per word, two per byte, low nibble first): the same bytes as the
    32-bit layout, taken as a view (no copy)."""
    _need(codes_i64, torch.int64, "codes_i64", 2)
    if not codes_i64.is_contiguous():
        raise ValueError("codes_i64 must be contiguous")
    return PackedLinear(codes_i64.view(torch.int32), scales, zeros)


def codes_as_i64(p: PackedLinear) -> torch.Tensor:
    """The codes of `p` viewed as the I64 container [N][K/16] (no copy)."""
    return p.codes.view(torch.int64)


def _matmul(fn, name, X: torch.Tensor, p: PackedLinear, out: torch.Tensor | None):
    _need(X, torch.bfloat16, "X", 2)
    M, K = X.shape
    if K != p.K:
        raise ValueError(f"X has K={K}, weights have K={p.K}")
    if out is None:
        out = torch.empty(M, p.N, dtype=torch.bfloat16, device=X.device)
    else:
        _need(out, torch.bfloat16, "out", 2)
        if tuple(out.shape) != (M, p.N):
            raise ValueError("out has the wrong shape")
    if getattr(p, "group", GROUP) == GROUP:
        st = fn(_ptr(X), M, X.stride(0), _ptr(p.codes), _ptr(p.scales), _ptr(p.zeros),
                p.N, p.K, _ptr(out), out.stride(0), _stream(X))
    else:
        fn, name = getattr(lib, name + "_grouped"), name + "_grouped"
        st = fn(_ptr(X), M, X.stride(0), _ptr(p.codes), _ptr(p.scales), _ptr(p.zeros),
                p.N, p.K, p.group, _ptr(out), out.stride(0), _stream(X))
    _check(name, st)
    return out


# Decode workspaces, one per (device, stream): zero-filled tensors that grow
# to the largest size asked for (each call leaves them reusable; see
# w4a16_gemv_ws in include/w4a16.h).  No workspace is created or grown while
# the stream is being captured into a graph: such a call runs unsplit.
_workspaces: dict = {}


def gemv_workspace(X: torch.Tensor, N: int, K: int) -> torch.Tensor | None:
    """The cached decode workspace of X's device and current stream, grown to
    what w4a16_gemv_ws can use for this shape (None when it needs none or the
    stream is capturing and none is large enough yet)."""
    nbytes = ctypes.c_int64(0)
    _check("w4a16_gemv_workspace_bytes",
           lib.w4a16_gemv_workspace_bytes(X.shape[0], N, K, ctypes.byref(nbytes)))
    if nbytes.value == 0:
        return None
    stream = torch.cuda.current_stream(X.device)
    key = (X.device.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes.value:
        if torch.cuda.is_current_stream_capturing():
            return ws if ws is not None and ws.numel() >= nbytes.value else None
        ws = torch.zeros(nbytes.value, dtype=torch.uint8, device=X.device)
        _workspaces[key] = ws
    return ws


def w4a16_gemv(X: torch.Tensor, p: PackedLinear, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X . w_hat^T for 1 <= M <= 32 (decode); groups other than 128 go
    through w4a16_gemv_grouped.  With groups of 128 the call goes through
    w4a16_gemv_ws with `workspace` (a zero-filled uint8 tensor) or, if None,
    the cached workspace of the device and stream."""
    if getattr(p, "group", GROUP) != GROUP:
        return _matmul(lib.w4a16_gemv, "w4a16_gemv", X, p, out)
    _need(X, torch.bfloat16, "X", 2)
    M, K = X.shape
    if K != p.K:
        raise ValueError(f"X has K={K}, weights have K={p.K}")
    if out is None:
        out = torch.empty(M, p.N, dtype=torch.bfloat16, device=X.device)
    else:
        _need(out, torch.bfloat16, "out", 2)
        if tuple(out.shape) != (M, p.N):
            raise ValueError("out has the wrong shape")
    if workspace is None and 3 <= M <= GEMV_MAX_M:   # M <= 2 never splits K
        workspace = gemv_workspace(X, p.N, p.K)
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check("w4a16_gemv_ws", lib.w4a16_gemv_ws(_ptr(X), M, X.stride(0), _ptr(p.codes), _ptr(p.scales),
                                              _ptr(p.zeros), p.N, p.K, _ptr(out), out.stride(0), ws_ptr,
                                              ws_bytes, _stream(X)))
    return out


# Prefill workspaces, one per (device, stream), separate from the decode
# ones (whose counters must stay zero): scratch for the float32 partial
# outputs of a split K, grown to the largest size asked for; none is created
# or grown while the stream is being captured.
_gemm_workspaces: dict = {}


def gemm_workspace(X: torch.Tensor, N: int, K: int) -> torch.Tensor | None:
    """The cached prefill workspace of X's device and current stream, grown
    to what w4a16_gemm_ws can use for this shape (None when it needs none or
    the stream is capturing and none is large enough yet)."""
    nbytes = ctypes.c_int64(0)
    _check("w4a16_gemm_workspace_bytes",
           lib.w4a16_gemm_workspace_bytes(X.shape[0], N, K, ctypes.byref(nbytes)))
    if nbytes.value == 0:
        return None
    stream = torch.cuda.current_stream(X.device)
    key = (X.device.index, stream.cuda_stream)
    ws = _gemm_workspaces.get(key)
    if ws is None or ws.numel() < nbytes.value:
        if torch.cuda.is_current_stream_capturing():
            return ws if ws is not None and ws.numel() >= nbytes.value else None
        ws = torch.empty(nbytes.value, dtype=torch.uint8, device=X.device)
        _gemm_workspaces[key] = ws
    return ws


def w4a16_gemm(X: torch.Tensor, p: PackedLinear, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X . w_hat^T on the matrix cores, any M (prefill); groups other than
    128 go through w4a16_gemm_grouped.  With groups of 128 the call goes
    through w4a16_gemm_ws with `workspace` (a uint8 tensor) or, if None, the
    cached prefill workspace of the device and stream."""
    if getattr(p, "group", GROUP) != GROUP:
        return _matmul(lib.w4a16_gemm, "w4a16_gemm", X, p, out)
    _need(X, torch.bfloat16, "X", 2)
    M, K = X.shape
    if K != p.K:
        raise ValueError(f"X has K={K}, weights have K={p.K}")
    if out is None:
        out = torch.empty(M, p.N, dtype=torch.bfloat16, device=X.device)
    else:
        _need(out, torch.bfloat16, "out", 2)
        if tuple(out.shape) != (M, p.N):
            raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = gemm_workspace(X, p.N, p.K)
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check("w4a16_gemm_ws", lib.w4a16_gemm_ws(_ptr(X), M, X.stride(0), _ptr(p.codes), _ptr(p.scales),
                                              _ptr(p.zeros), p.N, p.K, _ptr(out), out.stride(0), ws_ptr,
                                              ws_bytes, _stream(X)))
    return out


def w4a16_linear(X: torch.Tensor, p: PackedLinear, out: torch.Tensor | None = None) -> torch.Tensor:
    """Pick the decode kernel for M <= 32 and the matrix-core kernel above."""
    if X.shape[0] <= GEMV_MAX_M:
        return w4a16_gemv(X, p, out)
    return w4a16_gemm(X, p, out)


def w4a16_awq_importance(Xcal: torch.Tensor) -> torch.Tensor:
    _need(Xcal, torch.bfloat16, "Xcal", 2)
    T, K = Xcal.shape
    out = torch.empty(K, dtype=torch.float32, device=Xcal.device)
    _check("w4a16_awq_importance",
           lib.w4a16_awq_importance(_ptr(Xcal), T, K, Xcal.stride(0), _ptr(out), _stream(Xcal)))
    return out


def w4a16_awq_scale(importance: torch.Tensor, alpha: float) -> torch.Tensor:
    _need(importance, torch.float32, "importance", 1)
    out = torch.empty_like(importance)
    _check("w4a16_awq_scale", lib.w4a16_awq_scale(_ptr(importance), importance.shape[0],
                                                  float(alpha), _ptr(out), _stream(importance)))
    return out


def w4a16_awq_fold(s: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor | None = None):
    """In place: gamma /= s (and beta), BF16 round to nearest even."""
    _need(s, torch.float32, "s", 1)
    _need(gamma, torch.bfloat16, "gamma", 1)
    if beta is not None:
        _need(beta, torch.bfloat16, "beta", 1)
    K = s.shape[0]
    if gamma.shape[0] != K or (beta is not None and beta.shape[0] != K):
        raise ValueError("gamma/beta must have K entries")
    _check("w4a16_awq_fold", lib.w4a16_awq_fold(_ptr(s), K, _ptr(gamma), _ptr(beta), _stream(s)))
    return gamma, beta


def w4a16_scale_channels(X: torch.Tensor, gamma: torch.Tensor,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    _need(X, torch.bfloat16, "X", 2)
    _need(gamma, torch.bfloat16, "gamma", 1)
    M, K = X.shape
    if out is None:
        out = torch.empty(M, K, dtype=torch.bfloat16, device=X.device)
    _check("w4a16_scale_channels",
           lib.w4a16_scale_channels(_ptr(X), M, K, X.stride(0), _ptr(gamma), _ptr(out),
                                    out.stride(0), _stream(X)))
    return out


def w4a16_awq_search_error(Y: torch.Tensor, Yref: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Relative L2 distance of two BF16 outputs [M][N] (the search
    objective), as a float64 tensor of one element on the device."""
    _need(Y, torch.bfloat16, "Y", 2)
    _need(Yref, torch.bfloat16, "Yref", 2)
    if Y.shape != Yref.shape:
        raise ValueError("Y and Yref must have the same shape")
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=Y.device)
    M, N = Y.shape
    _check("w4a16_awq_search_error",
           lib.w4a16_awq_search_error(_ptr(Y), Y.stride(0), _ptr(Yref), Yref.stride(0), M, N,
                                      _ptr(out), _stream(Y)))
    return out


def w4a16_awq_search(W: torch.Tensor, Xcal: torch.Tensor, alphas, X: torch.Tensor | None = None):
    """AWQ's grid search over the exponent alpha of s = importance^alpha,
    run on this library's kernels: importance from Xcal, then per alpha the
    scale, the packed W diag(s), the activations X diag(s)^-1 through the
    folded producer weight bf16(1/s), the fused product, and its relative
    L2 error against the dense BF16 product of X and W (X defaults to Xcal),
    all library calls.  Returns (index of the best alpha, list of errors)."""
    _need(W, torch.bfloat16, "W", 2)
    X = Xcal if X is None else X
    K = W.shape[1]
    imp = w4a16_awq_importance(Xcal)
    y_dense = w4a16_dense_gemm(X, W)
    err = torch.empty(len(alphas), dtype=torch.float64, device=W.device)
    for i, a in enumerate(alphas):
        s = w4a16_awq_scale(imp, float(a))
        p = w4a16_pack(W, awq_s=s)
        gamma = torch.ones(K, dtype=torch.bfloat16, device=W.device)
        w4a16_awq_fold(s, gamma)
        Xs = w4a16_scale_channels(X, gamma)
        w4a16_awq_search_error(w4a16_gemm(Xs, p), y_dense, out=err[i:i + 1])
    errs = err.tolist()
    best = min(range(len(errs)), key=lambda i: errs[i])
    return best, errs


# ---------------------------------------------------------------------------
# Decode of a chain of dependent linears in one persistent launch
# ---------------------------------------------------------------------------

CHAIN_INPUTS = {"x0": 0, "prev": 1, "swiglu": 2, "attn1": 3}
CHAIN_TIMEOUT = 1


class ChainLinearC(ctypes.Structure):
    """w4a16_chain_linear of w4a16.h."""
    _fields_ = [("codes", _p), ("scales", _p), ("zeros", _p), ("gamma", _p), ("Y", _p),
                ("N", _i64), ("K", _i64), ("ldy", _i64),
                ("input", ctypes.c_int32), ("v_offset", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("group", ctypes.c_int32)]


class ChainPlanC(ctypes.Structure):
    """w4a16_chain_plan of w4a16.h."""
    _fields_ = [("workspace", _p), ("n_linears", ctypes.c_int32), ("M", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("max_k", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("k0", ctypes.c_int32), ("spin_limit", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("lds_bytes", _i64)]


class ChainPlan:
    """A prepared chain: the plan, its workspace and the tensors it refers to
    (kept alive here).  outputs[l] is linear l's BF16 output [M][N_l]."""

    def __init__(self, plan, workspace, linears, outputs):
        self.plan, self.workspace, self.linears, self.outputs = plan, workspace, linears, outputs


def w4a16_chain_prepare(linears, M: int, outputs=None) -> ChainPlan:
    """Prepare a chain of linears for w4a16_chain_run.  linears: a list of
    dicts with "p" (a PackedLinear of groups of 128), "input" (one of
    CHAIN_INPUTS; the first must be "x0"), optional "params" (v_offset,
    head_dim, group) for "attn1" and optional "gamma" (BF16 [K]).  Outputs
    are allocated here unless given ([M][N_l] BF16 tensors)."""
    if not linears:
        raise ValueError("empty chain")
    dev = linears[0]["p"].codes.device
    if outputs is None:   # rows padded to a multiple of 8 elements (16-byte aligned)
        outputs = [torch.empty(M, (L["p"].N + 7) // 8 * 8, dtype=torch.bfloat16, device=dev)[:, :L["p"].N]
                   for L in linears]
    arr = (ChainLinearC * len(linears))()
    for i, (L, y) in enumerate(zip(linears, outputs)):
        p = L["p"]
        if p.group != GROUP:
            raise ValueError("chains take groups of 128")
        _need(y, torch.bfloat16, "output", 2)
        g = L.get("gamma")
        if g is not None:
            _need(g, torch.bfloat16, "gamma", 1)
        v_off, hd, grp = L.get("params") or (0, 0, 0)
        arr[i] = ChainLinearC(_ptr(p.codes), _ptr(p.scales), _ptr(p.zeros), _ptr(g), _ptr(y),
                              p.N, p.K, y.stride(0), CHAIN_INPUTS[L["input"]], v_off, hd, grp)
    nbytes = ctypes.c_int64(0)
    _check("w4a16_chain_workspace_bytes", lib.w4a16_chain_workspace_bytes(len(linears), ctypes.byref(nbytes)))
    ws = torch.empty(nbytes.value + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    ws_view = ws[off:off + nbytes.value]
    plan = ChainPlanC()
    _check("w4a16_chain_prepare", lib.w4a16_chain_prepare(arr, len(linears), M, _ptr(ws_view), nbytes.value,
                                                          ctypes.byref(plan), _stream(ws)))
    return ChainPlan(plan, ws, list(linears), outputs)


def w4a16_chain_run(plan: ChainPlan, X0: torch.Tensor):
    """Run the chain on X0 [M][K_0] (one launch); returns the outputs."""
    _need(X0, torch.bfloat16, "X0", 2)
    if X0.shape[0] != plan.plan.M:
        raise ValueError(f"X0 has {X0.shape[0]} rows, the plan {plan.plan.M}")
    _check("w4a16_chain_run", lib.w4a16_chain_run(ctypes.byref(plan.plan), _ptr(X0), X0.stride(0), _stream(X0)))
    return plan.outputs


def w4a16_chain_status(plan: ChainPlan) -> int:
    """0, or CHAIN_TIMEOUT if a barrier wait gave up since the last call
    (synchronises the current stream)."""
    st = ctypes.c_int(0)
    _check("w4a16_chain_status", lib.w4a16_chain_status(ctypes.byref(plan.plan), ctypes.byref(st),
                                                        _stream(plan.workspace)))
    return st.value


def w4a16_chain_run_noalloc(linears, X0: torch.Tensor, outputs=None, wait_status: bool = True):
    """Prepare and run a chain in one call without a workspace (the
    library's fixed device array; for callers that cannot allocate; calls on
    one GPU must not overlap).  linears as for w4a16_chain_prepare; outputs
    are allocated here unless given.  With wait_status the call waits for the
    run and returns (outputs, status), status 0 or CHAIN_TIMEOUT; otherwise
    (outputs, None)."""
    _need(X0, torch.bfloat16, "X0", 2)
    M = X0.shape[0]
    dev = X0.device
    if outputs is None:
        outputs = [torch.empty(M, (L["p"].N + 7) // 8 * 8, dtype=torch.bfloat16, device=dev)[:, :L["p"].N]
                   for L in linears]
    arr = (ChainLinearC * len(linears))()
    for i, (L, y) in enumerate(zip(linears, outputs)):
        p = L["p"]
        if p.group != GROUP:
            raise ValueError("chains take groups of 128")
        _need(y, torch.bfloat16, "output", 2)
        g = L.get("gamma")
        v_off, hd, grp = L.get("params") or (0, 0, 0)
        arr[i] = ChainLinearC(_ptr(p.codes), _ptr(p.scales), _ptr(p.zeros), _ptr(g), _ptr(y),
                              p.N, p.K, y.stride(0), CHAIN_INPUTS[L["input"]], v_off, hd, grp)
    st = ctypes.c_int(-1)
    _check("w4a16_chain_run_noalloc",
           lib.w4a16_chain_run_noalloc(arr, len(linears), M, _ptr(X0), X0.stride(0),
                                       ctypes.byref(st) if wait_status else None, _stream(X0)))
    return outputs, (st.value if wait_status else None)


def w4a16_hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Stream-read every byte of `buf` (a contiguous device tensor whose size
    is a multiple of 16 bytes) and discard it: the measurement helper behind
    the measured HBM read ceiling.  Returns the sink word (device int32)."""
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check("w4a16_hbm_read_probe",
           lib.w4a16_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(buf)))
    return sink


# ---------------------------------------------------------------------------
# Dense BF16 comparisons (not the fused path; see w4a16.h)
# ---------------------------------------------------------------------------

def w4a16_dequantize_bf16(p: PackedLinear, out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense BF16 weights [N][K] of an offline expansion of `p`."""
    if out is None:
        out = torch.empty(p.N, p.K, dtype=torch.bfloat16, device=p.codes.device)
    else:
        _need(out, torch.bfloat16, "out", 2)
        if tuple(out.shape) != (p.N, p.K):
            raise ValueError("out has the wrong shape")
    _check("w4a16_dequantize_bf16",
           lib.w4a16_dequantize_bf16(_ptr(p.codes), _ptr(p.scales), _ptr(p.zeros), p.N, p.K,
                                     _ptr(out), out.stride(0), _stream(out)))
    return out


def _dense(fn, name, X: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None):
    _need(X, torch.bfloat16, "X", 2)
    _need(W, torch.bfloat16, "W", 2)
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError(f"X has K={K}, W has K={W.shape[1]}")
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    else:
        _need(out, torch.bfloat16, "out", 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    _check(name, fn(_ptr(X), M, X.stride(0), _ptr(W), W.stride(0), N, K, _ptr(out), out.stride(0),
                    _stream(X)))
    return out


def w4a16_dense_gemv(X: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense BF16 Y = X . W^T for 1 <= M <= 8 (decode comparison)."""
    return _dense(lib.w4a16_dense_gemv, "w4a16_dense_gemv", X, W, out)


def w4a16_dense_gemm(X: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense BF16 Y = X . W^T on the matrix cores, any M (prefill comparison)."""
    return _dense(lib.w4a16_dense_gemm, "w4a16_dense_gemm", X, W, out)
