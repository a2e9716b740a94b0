"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments before touching the GPU.  No call here
reaches a kernel launch (every argument set fails validation)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
lib = w4.lib

OK, INVALID, MISALIGNED, UNSUPPORTED, HIPERR = 0, 1, 2, 3, 4
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(w4a16_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    assert header_functions() == sorted([
        "w4a16_abi_version", "w4a16_strerror", "w4a16_pack", "w4a16_gemv", "w4a16_gemm",
        "w4a16_awq_importance", "w4a16_awq_scale", "w4a16_awq_fold", "w4a16_scale_channels",
        "w4a16_dequantize_bf16", "w4a16_dense_gemv", "w4a16_dense_gemm", "w4a16_pack_symmetric",
        "w4a16_pack_grouped", "w4a16_gemv_grouped", "w4a16_gemm_grouped",
        "w4a16_pack_int8", "w4a16_gemv_int8", "w4a16_gemm_int8", "w4a16_awq_search_error",
        "w4a16_hbm_read_probe", "w4a16_chain_workspace_bytes", "w4a16_chain_prepare",
        "w4a16_chain_run", "w4a16_chain_status", "w4a16_chain_run_noalloc",
        "w4a16_gemv_workspace_bytes", "w4a16_gemv_ws", "w4a16_gemm_workspace_bytes", "w4a16_gemm_ws"])


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", w4.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(w4a16_\w+)$", out, re.M))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(w4.EXPORTS) == set(header_functions())


def test_version_and_strerror():
    assert lib.w4a16_abi_version() == 10
    for st in range(5):
        assert lib.w4a16_strerror(st)
    assert b"unknown" in lib.w4a16_strerror(99)


def p(v):
    return ctypes.c_void_p(v)


def gemv(fn=None, X=FAKE, M=1, ldx=4096, codes=FAKE, scales=FAKE, zeros=FAKE, N=4096, K=4096,
         Y=FAKE, ldy=4096):
    fn = fn or lib.w4a16_gemv
    return fn(p(X), M, ldx, p(codes), p(scales), p(zeros), N, K, p(Y), ldy, p(0))


@pytest.mark.parametrize("fn", ["w4a16_gemv", "w4a16_gemm"])
def test_matmul_validation(fn):
    f = getattr(lib, fn)
    assert gemv(f, X=0) == INVALID
    assert gemv(f, codes=0) == INVALID
    assert gemv(f, scales=0) == INVALID
    assert gemv(f, zeros=0) == INVALID
    assert gemv(f, Y=0) == INVALID
    assert gemv(f, M=0) == INVALID
    assert gemv(f, N=0) == INVALID
    assert gemv(f, K=0) == INVALID
    assert gemv(f, K=4000, ldx=4000) == INVALID          # K % 128
    assert gemv(f, K=64, ldx=64) == INVALID              # K < 128
    assert gemv(f, ldx=4095) == INVALID                  # ldx < K
    assert gemv(f, ldy=100) == INVALID                   # ldy < N
    assert gemv(f, X=FAKE + 2) == MISALIGNED             # X not 16-byte aligned
    assert gemv(f, ldx=4100) == MISALIGNED               # ldx % 8
    assert gemv(f, codes=FAKE + 4) == MISALIGNED
    assert gemv(f, scales=FAKE + 1) == MISALIGNED
    assert gemv(f, zeros=FAKE + 2) == MISALIGNED
    assert gemv(f, Y=FAKE + 1) == MISALIGNED
    assert gemv(f, N=1 << 30, ldy=1 << 30) == UNSUPPORTED


def test_gemv_rejects_large_m():
    assert gemv(M=33) == INVALID
    assert gemv(M=1 << 20) == INVALID


def gemv_ws(ws=FAKE + (1 << 24), nbytes=1 << 20, X=FAKE, M=16, ldx=4096, codes=FAKE, scales=FAKE,
            zeros=FAKE, N=4096, K=4096, Y=FAKE, ldy=4096):
    return lib.w4a16_gemv_ws(p(X), M, ldx, p(codes), p(scales), p(zeros), N, K, p(Y), ldy, p(ws), nbytes,
                             p(0))


def test_gemv_ws_validation():
    # the matmul checks first, then the workspace's
    assert gemv_ws(X=0) == INVALID and gemv_ws(M=33) == INVALID and gemv_ws(X=FAKE + 2) == MISALIGNED
    assert gemv_ws(nbytes=-1) == INVALID
    assert gemv_ws(ws=0, nbytes=64) == INVALID                 # no pointer for a size
    assert gemv_ws(ws=FAKE + (1 << 24) + 32) == MISALIGNED      # 64-byte alignment
    # overlapping the activations, the output or the packed matrix
    assert gemv_ws(ws=FAKE, nbytes=64) == INVALID
    assert gemv_ws(X=1 << 28, ws=(1 << 28) + 64, nbytes=64) == INVALID
    assert gemv_ws(Y=1 << 28, ws=(1 << 28) + 4096, nbytes=64) == INVALID
    assert gemv_ws(codes=1 << 28, ws=(1 << 28) + 8 * 1024 * 1024 - 64, nbytes=64) == INVALID
    assert gemv_ws(scales=1 << 28, ws=(1 << 28) + 4096 * 32 * 2 - 64, nbytes=64) == INVALID
    assert gemv_ws(zeros=1 << 28, ws=(1 << 28) + 4096 * 32 * 4 - 64, nbytes=64) == INVALID
    n = ctypes.c_int64(7)
    assert lib.w4a16_gemv_workspace_bytes(16, 4096, 4096, None) == INVALID
    assert lib.w4a16_gemv_workspace_bytes(0, 4096, 4096, ctypes.byref(n)) == INVALID and n.value == 0
    assert lib.w4a16_gemv_workspace_bytes(33, 4096, 4096, ctypes.byref(n)) == INVALID
    assert lib.w4a16_gemv_workspace_bytes(16, 4096, 4000, ctypes.byref(n)) == INVALID
    assert lib.w4a16_gemv_workspace_bytes(16, 1 << 30, 4096, ctypes.byref(n)) == UNSUPPORTED


def gemm_ws(ws=FAKE + (1 << 24), nbytes=1 << 20, X=FAKE, M=512, ldx=4096, codes=FAKE, scales=FAKE,
            zeros=FAKE, N=4096, K=4096, Y=FAKE, ldy=4096):
    return lib.w4a16_gemm_ws(p(X), M, ldx, p(codes), p(scales), p(zeros), N, K, p(Y), ldy, p(ws), nbytes,
                             p(0))


def test_gemm_ws_validation():
    # the matmul and GEMM-limit checks first, then the workspace's
    assert gemm_ws(X=0) == INVALID and gemm_ws(K=4000) == INVALID and gemm_ws(X=FAKE + 2) == MISALIGNED
    assert gemm_ws(ldx=1 << 23, ws=FAKE + (1 << 40)) == UNSUPPORTED
    assert gemm_ws(nbytes=-1) == INVALID
    assert gemm_ws(ws=0, nbytes=64) == INVALID                  # no pointer for a size
    assert gemm_ws(ws=FAKE + (1 << 24) + 8) == MISALIGNED       # 16-byte alignment
    # overlapping the activations, the output or the packed matrix
    assert gemm_ws(ws=FAKE, nbytes=64) == INVALID
    assert gemm_ws(X=1 << 28, ws=(1 << 28) + 511 * 8192 + 64, nbytes=64) == INVALID
    assert gemm_ws(Y=1 << 28, ws=(1 << 28) + 4096, nbytes=64) == INVALID
    assert gemm_ws(codes=1 << 28, ws=(1 << 28) + 8 * 1024 * 1024 - 64, nbytes=64) == INVALID
    assert gemm_ws(scales=1 << 28, ws=(1 << 28) + 4096 * 32 * 2 - 64, nbytes=64) == INVALID
    assert gemm_ws(zeros=1 << 28, ws=(1 << 28) + 4096 * 32 * 4 - 64, nbytes=64) == INVALID
    n = ctypes.c_int64(7)
    assert lib.w4a16_gemm_workspace_bytes(512, 4096, 4096, None) == INVALID
    assert lib.w4a16_gemm_workspace_bytes(0, 4096, 4096, ctypes.byref(n)) == INVALID and n.value == 0
    assert lib.w4a16_gemm_workspace_bytes(512, 4096, 4000, ctypes.byref(n)) == INVALID
    assert lib.w4a16_gemm_workspace_bytes(512, 1 << 30, 4096, ctypes.byref(n)) == UNSUPPORTED


@pytest.mark.parametrize("fn", ["w4a16_pack", "w4a16_pack_symmetric"])
def test_pack_validation(fn):
    f = getattr(lib, fn)

    def call(W=FAKE, N=16, K=256, ldw=256, s=0, c=FAKE, sc=FAKE, z=FAKE):
        return f(p(W), N, K, ldw, p(s), p(c), p(sc), p(z), p(0))

    assert call(W=0) == INVALID
    assert call(c=0) == INVALID and call(sc=0) == INVALID and call(z=0) == INVALID
    assert call(N=0) == INVALID
    assert call(K=200, ldw=200) == INVALID
    assert call(ldw=255) == INVALID
    assert call(W=FAKE + 1) == MISALIGNED
    assert call(c=FAKE + 8) == MISALIGNED
    assert call(sc=FAKE + 1) == MISALIGNED
    assert call(z=FAKE + 2) == MISALIGNED
    assert call(s=FAKE + 2) == MISALIGNED
    assert call(N=1 << 30) == UNSUPPORTED


def test_awq_validation():
    assert lib.w4a16_awq_importance(p(0), 4, 8, 8, p(FAKE), p(0)) == INVALID
    assert lib.w4a16_awq_importance(p(FAKE), 0, 8, 8, p(FAKE), p(0)) == INVALID
    assert lib.w4a16_awq_importance(p(FAKE), 4, 8, 7, p(FAKE), p(0)) == INVALID
    assert lib.w4a16_awq_importance(p(FAKE + 1), 4, 8, 8, p(FAKE), p(0)) == MISALIGNED
    assert lib.w4a16_awq_scale(p(FAKE), 8, ctypes.c_float(1.5), p(FAKE), p(0)) == INVALID
    assert lib.w4a16_awq_scale(p(FAKE), 8, ctypes.c_float(-0.1), p(FAKE), p(0)) == INVALID
    assert lib.w4a16_awq_scale(p(FAKE), 8, ctypes.c_float(float("nan")), p(FAKE), p(0)) == INVALID
    assert lib.w4a16_awq_scale(p(FAKE + 2), 8, ctypes.c_float(0.5), p(FAKE), p(0)) == MISALIGNED
    assert lib.w4a16_awq_fold(p(0), 8, p(FAKE), p(0), p(0)) == INVALID
    assert lib.w4a16_awq_fold(p(FAKE), 0, p(FAKE), p(0), p(0)) == INVALID
    assert lib.w4a16_awq_fold(p(FAKE), 8, p(FAKE + 1), p(0), p(0)) == MISALIGNED
    assert lib.w4a16_scale_channels(p(FAKE), 2, 8, 7, p(FAKE), p(FAKE), 8, p(0)) == INVALID
    assert lib.w4a16_scale_channels(p(FAKE), 2, 8, 8, p(FAKE), p(FAKE), 7, p(0)) == INVALID
    assert lib.w4a16_scale_channels(p(FAKE), 2, 8, 8, p(FAKE + 1), p(FAKE), 8, p(0)) == MISALIGNED
    pr = lib.w4a16_hbm_read_probe
    assert pr(p(0), 1024, p(FAKE), p(0)) == INVALID
    assert pr(p(FAKE), 1000, p(FAKE), p(0)) == INVALID
    assert pr(p(FAKE + 8), 1024, p(FAKE), p(0)) == MISALIGNED
    e = lib.w4a16_awq_search_error
    assert e(p(0), 8, p(FAKE), 8, 2, 8, p(FAKE), p(0)) == INVALID
    assert e(p(FAKE), 8, p(FAKE), 8, 0, 8, p(FAKE), p(0)) == INVALID
    assert e(p(FAKE), 7, p(FAKE), 8, 2, 8, p(FAKE), p(0)) == INVALID
    assert e(p(FAKE), 8, p(FAKE), 8, 2, 8, p(FAKE + 4), p(0)) == MISALIGNED


def test_binding_rejects_cpu_tensors():
    import torch
    W = torch.zeros(16, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w4.w4a16_pack(W)
    with pytest.raises(TypeError):
        w4.w4a16_pack(W.float())


def dense(fn, X=FAKE, M=1, ldx=4096, W=FAKE, ldw=4096, N=4096, K=4096, Y=FAKE, ldy=4096):
    return fn(p(X), M, ldx, p(W), ldw, N, K, p(Y), ldy, p(0))


@pytest.mark.parametrize("fn", ["w4a16_dense_gemv", "w4a16_dense_gemm"])
def test_dense_validation(fn):
    f = getattr(lib, fn)
    assert dense(f, X=0) == INVALID
    assert dense(f, W=0) == INVALID
    assert dense(f, Y=0) == INVALID
    assert dense(f, M=0) == INVALID
    assert dense(f, N=0) == INVALID
    assert dense(f, K=4000, ldx=4000, ldw=4000) == INVALID   # K % 128
    assert dense(f, ldw=4000) == INVALID                     # ldw < K
    assert dense(f, ldx=4095) == INVALID
    assert dense(f, ldy=100) == INVALID
    assert dense(f, X=FAKE + 2) == MISALIGNED
    assert dense(f, W=FAKE + 8) == MISALIGNED
    assert dense(f, ldw=4100) == MISALIGNED
    assert dense(f, Y=FAKE + 1) == MISALIGNED
    assert dense(f, N=1 << 30, ldy=1 << 30) == UNSUPPORTED


def test_dense_gemv_m_limit():
    assert dense(lib.w4a16_dense_gemv, M=9) == INVALID


def test_dequantize_validation():
    f = lib.w4a16_dequantize_bf16

    def call(codes=FAKE, scales=FAKE, zeros=FAKE, N=16, K=256, W=FAKE, ldw=256):
        return f(p(codes), p(scales), p(zeros), N, K, p(W), ldw, p(0))
    assert call(codes=0) == INVALID
    assert call(W=0) == INVALID
    assert call(N=0) == INVALID
    assert call(K=200, ldw=200) == INVALID
    assert call(ldw=128) == INVALID
    assert call(codes=FAKE + 4) == MISALIGNED
    assert call(scales=FAKE + 1) == MISALIGNED
    assert call(zeros=FAKE + 2) == MISALIGNED
    assert call(W=FAKE + 2) == MISALIGNED
    assert call(ldw=260) == MISALIGNED
    assert call(N=1 << 30) == UNSUPPORTED


@pytest.mark.parametrize("fn", ["w4a16_gemv_grouped", "w4a16_gemm_grouped"])
def test_grouped_matmul_validation(fn):
    f = getattr(lib, fn)

    def call(group=64, X=FAKE, M=1, ldx=4096, codes=FAKE, scales=FAKE, zeros=FAKE, N=4096, K=4096,
             Y=FAKE, ldy=4096):
        return f(p(X), M, ldx, p(codes), p(scales), p(zeros), N, K, group, p(Y), ldy, p(0))
    for g in (0, 16, 96, 256, -64):
        assert call(group=g) == INVALID
    assert call(K=4000, ldx=4000) == INVALID              # K % 128 for every group
    assert call(X=0) == INVALID
    assert call(scales=FAKE + 8) == MISALIGNED            # 16-byte rule below 128
    assert call(zeros=FAKE + 4) == MISALIGNED
    assert call(group=128, scales=FAKE + 8, zeros=FAKE + 4, M=0) == INVALID
    assert call(N=1 << 30, ldy=1 << 30) == UNSUPPORTED


def test_grouped_pack_validation():
    f = lib.w4a16_pack_grouped

    def call(group=32, W=FAKE, N=16, K=256, ldw=256, c=FAKE, sc=FAKE, z=FAKE):
        return f(p(W), N, K, ldw, p(0), group, p(c), p(sc), p(z), p(0))
    for g in (0, 8, 48, 256):
        assert call(group=g) == INVALID
    assert call(K=96, ldw=96) == INVALID
    assert call(c=FAKE + 8) == MISALIGNED
    assert call(N=1 << 30) == UNSUPPORTED


def test_int8_validation():
    f = lib.w4a16_gemv_int8
    assert gemv(f, M=5) == INVALID                       # M <= 4
    assert gemv(f, M=0) == INVALID
    assert gemv(f, K=32896, ldx=32896) == UNSUPPORTED     # K <= 32768
    assert gemv(f, X=FAKE + 2) == MISALIGNED
    assert gemv(f, codes=FAKE + 4) == MISALIGNED
    g = lib.w4a16_gemm_int8
    assert gemv(g, M=0) == INVALID and gemv(g, K=200, ldx=200) == INVALID
    assert gemv(g, scales=FAKE + 1) == MISALIGNED
    pk = lib.w4a16_pack_int8
    assert pk(p(FAKE), 16, 200, 200, p(0), p(FAKE), p(FAKE), p(FAKE), p(0)) == INVALID
    assert pk(p(FAKE), 16, 256, 256, p(0), p(FAKE + 8), p(FAKE), p(FAKE), p(0)) == MISALIGNED
    assert pk(p(0), 16, 256, 256, p(0), p(FAKE), p(FAKE), p(FAKE), p(0)) == INVALID


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.parametrize("fn", ["w4a16_gemm", "w4a16_gemm_int8"])
def test_gemm_offset_limits(fn):
    f = getattr(lib, fn)
    big = 1 << 23                                   # W4A16_GEMM_MAX_LD
    assert gemv(f, ldx=big) == UNSUPPORTED
    assert gemv(f, K=1 << 25, ldx=(1 << 25) + 8) == UNSUPPORTED   # W4A16_GEMM_MAX_K (ldx checked too)
    # ceil(M/64) * ceil(N/128) tiles must stay below 2^31
    assert gemv(f, M=1 << 29, N=1 << 29, ldy=1 << 29) == UNSUPPORTED


def test_grouped_gemm_offset_limits():
    f = lib.w4a16_gemm_grouped

    def call(M=1, ldx=4096, K=4096, group=64):
        return f(p(FAKE), M, ldx, p(FAKE), p(FAKE), p(FAKE), 4096, K, group, p(FAKE), 4096, p(0))
    assert call(ldx=1 << 23) == UNSUPPORTED
    g = lib.w4a16_gemv_grouped

    def callv(M, ldx):
        return g(p(FAKE), M, ldx, p(FAKE), p(FAKE), p(FAKE), 4096, 4096, 64, p(FAKE), 4096, p(0))
    assert callv(16, 1 << 23) == UNSUPPORTED        # M > 8 runs the GEMM


def test_dense_gemm_offset_limits():
    f = lib.w4a16_dense_gemm
    assert dense(f, ldx=1 << 23) == UNSUPPORTED
    assert dense(f, ldw=1 << 23) == UNSUPPORTED


def test_limits_match_header():
    text = open(HEADER).read()
    assert "#define W4A16_GEMM_MAX_LD ((int64_t)1 << 23)" in text
    assert "#define W4A16_GEMM_MAX_K ((int64_t)1 << 25)" in text
    assert "#define W4A16_MAX_DIM ((int64_t)1 << 30)" in text


@pytest.mark.skipif(not _no_gpu(), reason="only where no GPU is visible: the call would launch")
def test_valid_call_without_a_device_is_unsupported():
    # arguments that pass every check reach the device check, which finds no
    # gfx950 device here and refuses before any launch
    assert gemv() == UNSUPPORTED
    assert gemv(lib.w4a16_gemm) == UNSUPPORTED
    assert gemv_ws() == UNSUPPORTED
    assert gemm_ws() == UNSUPPORTED
    n = ctypes.c_int64(7)
    assert lib.w4a16_gemm_workspace_bytes(512, 4096, 4096, ctypes.byref(n)) == UNSUPPORTED and n.value == 0
    assert lib.w4a16_gemv_workspace_bytes(16, 4096, 14336, ctypes.byref(n)) == UNSUPPORTED and n.value == 0
    assert lib.w4a16_pack(p(FAKE), 16, 256, 256, p(0), p(FAKE), p(FAKE), p(FAKE), p(0)) == UNSUPPORTED
    assert lib.w4a16_awq_fold(p(FAKE), 8, p(FAKE), p(0), p(0)) == UNSUPPORTED


def _chain(specs):
    """A host array of chain linears at fake, well-separated device addresses;
    specs: dicts overriding the defaults of each linear."""
    arr = (w4.ChainLinearC * len(specs))()
    for i, sp in enumerate(specs):
        base = FAKE * (16 + 64 * i)
        d = dict(codes=base, scales=base + (1 << 24), zeros=base + (2 << 24), gamma=0, Y=base + (3 << 24),
                 N=1024, K=1024, ldy=1024, input=0 if i == 0 else 1, v_offset=0, head_dim=0, group=0)
        d.update(sp)
        for k, v in d.items():
            setattr(arr[i], k, v)
    return arr


def chain_prepare(specs, M=1, ws=FAKE * 8192, nbytes=1 << 20):
    arr = _chain(specs)
    plan = w4.ChainPlanC()
    return lib.w4a16_chain_prepare(arr, len(specs), M, p(ws), nbytes, ctypes.byref(plan), p(0))


def test_chain_validation():
    two = [{}, {}]
    assert chain_prepare([]) == INVALID                          # no linears
    assert chain_prepare(two, M=0) == INVALID
    assert chain_prepare(two, M=3) == INVALID                    # W4A16_CHAIN_MAX_M
    assert chain_prepare(two, nbytes=64) == INVALID              # workspace too small
    assert chain_prepare(two, ws=FAKE * 8192 + 128) == MISALIGNED
    assert chain_prepare([{"input": 1}, {}]) == INVALID          # the first linear takes X0
    assert chain_prepare([{}, {"K": 1000}]) == INVALID           # K % 128
    assert chain_prepare([{}, {"K": 2048}]) == INVALID           # PREV wider than the previous output
    assert chain_prepare([{"N": 2048}, {"input": 2, "K": 1152}]) == INVALID   # SwiGLU needs 2K outputs
    assert chain_prepare([{}, {"input": 3, "K": 512, "head_dim": 0, "group": 1}]) == INVALID
    assert chain_prepare([{}, {"input": 3, "K": 512, "head_dim": 128, "group": 1,
                               "v_offset": 600}]) == INVALID     # value block past the previous output
    assert chain_prepare([{}, {"input": 4}]) == INVALID          # unknown input kind
    assert chain_prepare([{}, {"ldy": 1000}]) == INVALID         # ldy < N
    assert chain_prepare([{}, {"ldy": 1028, "N": 1028}]) == MISALIGNED   # ldy % 8
    assert chain_prepare([{}, {"Y": FAKE * 80 + 8}]) == MISALIGNED
    assert chain_prepare([{}, {"gamma": FAKE * 90 + 4}]) == MISALIGNED
    assert chain_prepare([{"K": 32896}, {}]) == UNSUPPORTED      # W4A16_CHAIN_MAX_K
    a = _chain(two)
    assert chain_prepare([{}, {"Y": a[1].codes}]) == INVALID     # output over its own matrix
    assert chain_prepare([{}, {"Y": a[0].Y}]) == INVALID         # output over its input
    # every check passes: no device here
    assert chain_prepare(two) == UNSUPPORTED


def test_chain_noalloc_validation():
    arr = _chain([{}, {}])
    st = ctypes.c_int(-1)
    assert lib.w4a16_chain_run_noalloc(arr, 2, 1, p(0), 1024, ctypes.byref(st), p(0)) == INVALID
    assert lib.w4a16_chain_run_noalloc(arr, 2, 1, p(FAKE + 8), 1024, ctypes.byref(st), p(0)) == MISALIGNED
    assert lib.w4a16_chain_run_noalloc(arr, 2, 1, p(FAKE), 1020, ctypes.byref(st), p(0)) == MISALIGNED
    big = _chain([{}] * 257)
    assert lib.w4a16_chain_run_noalloc(big, 257, 1, p(FAKE), 1024, ctypes.byref(st), p(0)) == UNSUPPORTED
    assert lib.w4a16_chain_run_noalloc(arr, 2, 1, p(FAKE), 1024, ctypes.byref(st), p(0)) == UNSUPPORTED
