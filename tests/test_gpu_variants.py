"""Format variants on the GPU against the CPU oracle: the symmetric INT4
packer (bit-exact) and the matmuls on its output, and the I64 code container
consumed in place."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, i32, sample_rows, u32

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def assert_symmetric_pack_equal(p, W_bits, rows=None, awq_s=None):
    if rows is None:
        rows = np.arange(W_bits.shape[0])
    codes, scales, zeros = O.quantize_pack_symmetric(W_bits[rows], awq_s)
    for name, a, b in (("codes", u32(p.codes)[rows], codes), ("scales", gen.bits(p.scales)[rows], scales),
                       ("zeros", i32(p.zeros)[rows], zeros)):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            r, c = bad[0]
            raise AssertionError(f"{name} differ at {len(bad)} places; first row {rows[r]} col {c}: "
                                 f"gpu {a[r, c]:#x} oracle {b[r, c]:#x}")


def symmetric_reference(X_bits, W_bits, rows):
    codes, scales, zeros = O.quantize_pack_symmetric(W_bits[rows])
    y_ref = O.matmul_ref(X_bits, codes, scales, zeros)
    w_hat = O.dequantize(codes, scales, zeros)
    mag = np.abs(O.bf16_to_f32(X_bits).astype(np.float64)) @ np.abs(w_hat).T
    return y_ref, mag


def test_symmetric_hand_groups():
    k = np.concatenate([np.arange(-7, 8), np.zeros(113)])
    rows = np.stack([k * 2.0 ** -4, -3 * k * 2.0 ** -4, np.zeros(128),
                     np.where(np.arange(128) == 5, 2.0 ** -126, 0.0), np.full(128, -0.375)])
    Wb = O.f32_to_bf16_rne(rows.astype(np.float32))
    p = w4.w4a16_pack_symmetric(gen.from_bits(Wb, DEV))
    torch.cuda.synchronize()
    assert_symmetric_pack_equal(p, Wb)
    assert list(gen.bits(p.scales)[:4, 0]) == [0x3D80, 0x3E40, 0x3F80, 0x0080]
    assert np.all(i32(p.zeros) == 8)


@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (16, 4096), (257, 1024)])
def test_symmetric_pack_shapes(N, K):
    W = gen.weights(N, K, "sym", f"{N}x{K}", shift=True, device=DEV)
    p = w4.w4a16_pack_symmetric(W)
    torch.cuda.synchronize()
    assert_symmetric_pack_equal(p, gen.bits(W))


def test_symmetric_pack_awq_and_llama_shape():
    L = [l for l in gen.LLAMA8B if l.name == "gate_up"][0]
    W = gen.weights(L.N, L.K, "sym", L.name, shift=True, device=DEV)
    s = gen.channel_vector(L.K, "sym", L.name, "awq").to(DEV)
    p = w4.w4a16_pack_symmetric(W, awq_s=s)
    torch.cuda.synchronize()
    rows = sample_rows(L.N, 64, seed=51)
    # the oracle sees the sampled rows of W only
    codes, scales, zeros = O.quantize_pack_symmetric(gen.bits(W[torch.as_tensor(rows, device=DEV)]),
                                                     s.cpu().numpy())
    assert np.array_equal(u32(p.codes)[rows], codes)
    assert np.array_equal(gen.bits(p.scales)[rows], scales)
    assert np.all(i32(p.zeros) == 8)


@pytest.mark.parametrize("M", [1, 4, 16, 300])
def test_matmul_on_symmetric_weights(M):
    N, K = 1000, 2048
    W = gen.weights(N, K, "sym", "mm", shift=True, device=DEV)
    X = gen.activations(M, K, "sym", "mm", device=DEV)
    p = w4.w4a16_pack_symmetric(W)
    y = w4.w4a16_linear(X, p)
    torch.cuda.synchronize()
    rows = sample_rows(N, 64, seed=M)
    y_ref, mag = symmetric_reference(gen.bits(X), gen.bits(W), rows)
    assert_output_close(y[:, torch.as_tensor(rows, device=DEV)], y_ref, mag, label=f"symmetric M={M}")


def test_i64_container_bytes_and_in_place_use():
    """Codes written by the oracle into an I64 container (sixteen per word)
    feed the kernels through a view; and the library's own packing viewed as
    I64 is that container, byte for byte."""
    N, K, M = 300, 1024, 8
    W = gen.weights(N, K, "i64", "c", shift=True, device=DEV)
    Wb = gen.bits(W)
    q, scales, zeros = O.quantize(Wb)
    c64 = torch.from_numpy(O.pack_codes_i64(q)).to(DEV)
    p = w4.packed_from_i64(c64, gen.from_bits(scales, DEV), torch.from_numpy(zeros).to(DEV))
    assert p.codes.data_ptr() == c64.data_ptr()          # a view, not a copy
    X = gen.activations(M, K, "i64", "c", device=DEV)
    y = w4.w4a16_gemv(X, p)
    torch.cuda.synchronize()
    codes = O.pack_codes(q)
    y_ref = O.matmul_ref(gen.bits(X), codes, scales, zeros)
    mag = np.abs(O.bf16_to_f32(gen.bits(X)).astype(np.float64)) @ np.abs(O.dequantize(codes, scales, zeros)).T
    assert_output_close(y, y_ref, mag, label="i64 container")
    own = w4.w4a16_pack(W)
    torch.cuda.synchronize()
    assert np.array_equal(w4.codes_as_i64(own).cpu().numpy(), O.pack_codes_i64(q))
