"""w4a16_pack on the GPU vs the CPU oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_pack_equal, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def _hand_rows():
    """The constructed groups of the oracle pins, one per row."""
    j = np.arange(128) % 16
    rows = []
    rows.append((j - 8) * 2.0 ** -7)
    rows.append(1.0 + j / 16.0)
    v = (j - 8) * 2.0 ** -7
    v[16], v[17], v[18] = 2.5 * 2.0 ** -7, -2.5 * 2.0 ** -7, 0.5 * 2.0 ** -7
    rows.append(v)
    v = np.zeros(128); v[0], v[1] = -6.5 * 2.0 ** -7, 8.5 * 2.0 ** -7
    rows.append(v)
    v = np.zeros(128); v[0], v[1] = -0.5, 1.0
    rows.append(v)
    rows.append(np.full(128, 0.375))
    rows.append(np.full(128, -0.375))
    rows.append(np.zeros(128))
    rows.append(np.full(128, 2.0 ** -130))
    rows.append(np.where(np.arange(128) % 2 == 0, -(2.0 ** -125), 2.0 ** -125))
    rows.append(np.full(128, -3.0e38))
    rows.append(np.linspace(100.0, 101.0, 128))
    f = np.array(rows, dtype=np.float32)
    return O.f32_to_bf16_rne(f)


def test_hand_groups():
    Wb = _hand_rows()
    # expected closed forms (derived in the oracle pins)
    W = gen.from_bits(Wb, DEV)
    p = w4.w4a16_pack(W)
    torch.cuda.synchronize()
    assert_pack_equal(p, Wb)
    s = gen.bits(p.scales)[:, 0]
    z = p.zeros.cpu().numpy()[:, 0]
    assert list(s[:10]) == [0x3C00, 0x3D80, 0x3C00, 0x3C00, 0x3DCC, 0x3EC0, 0x3EC0, 0x3F80, 0x3F80, 0x0100]
    assert list(z[:10]) == [8, -16, 8, 7, 5, -1, 1, 0, 0, 1]


@pytest.mark.parametrize("N,K", [(1, 128), (37, 384), (16, 4096), (257, 1024)])
def test_small_shapes(N, K):
    W = gen.weights(N, K, "pack", f"{N}x{K}", shift=True, device=DEV)
    p = w4.w4a16_pack(W)
    torch.cuda.synchronize()
    assert_pack_equal(p, gen.bits(W))


def test_strided_and_unaligned_source():
    N, K = 48, 512
    big = gen.weights(N, K + 24, "pack", "strided", device=DEV)
    for view in (big[:, :K], big[:, 8:K + 8], big[:, 1:K + 1], big[:, 3:K + 3]):
        p = w4.w4a16_pack(view)
        torch.cuda.synchronize()
        assert_pack_equal(p, gen.bits(view.contiguous()))


def test_awq_prescale():
    N, K = 96, 1024
    W = gen.weights(N, K, "pack", "awq", device=DEV)
    s = gen.channel_vector(K, "pack", "awq", "s", device=DEV)
    p = w4.w4a16_pack(W, awq_s=s)
    torch.cuda.synchronize()
    assert_pack_equal(p, gen.bits(W), awq_s=s.cpu().numpy())


def test_on_grid_roundtrip():
    import oracle_pins as P
    W_bits, (q0, s0, z0) = P.check_all_codes_on_grid(seed=21, N=64, K=512)
    p = w4.w4a16_pack(gen.from_bits(W_bits, DEV))
    torch.cuda.synchronize()
    assert np.array_equal(gen.bits(p.scales), s0)
    assert np.array_equal(p.zeros.cpu().numpy(), z0)
    assert np.array_equal(p.codes.cpu().numpy().view(np.uint32), O.pack_codes(q0))


def test_single_linear_4096_full():
    W = gen.weights(4096, 4096, 1, "linear", device=DEV)
    p = w4.w4a16_pack(W)
    torch.cuda.synchronize()
    assert_pack_equal(p, gen.bits(W))


@pytest.mark.parametrize("workload", ["llama8b_decode", "llama70b_decode"])
def test_model_layers_sampled(workload):
    spec = gen.WORKLOADS[workload]
    for layer in spec["layers"]:
        W = gen.weights(layer.N, layer.K, workload, layer.name, shift=spec["shift"], device=DEV)
        p = w4.w4a16_pack(W)
        torch.cuda.synchronize()
        rows = sample_rows(layer.N, 96, seed=layer.N)
        Wrows = gen.bits(W[torch.as_tensor(rows, device=DEV)])
        codes, scales, zeros = O.quantize_pack(Wrows)
        assert np.array_equal(p.codes[torch.as_tensor(rows, device=DEV)].cpu().numpy().view(np.uint32), codes)
        assert np.array_equal(gen.bits(p.scales[torch.as_tensor(rows, device=DEV)]), scales)
        assert np.array_equal(p.zeros[torch.as_tensor(rows, device=DEV)].cpu().numpy(), zeros)
        del W, p
        torch.cuda.empty_cache()


def test_deterministic():
    W = gen.weights(300, 2048, "pack", "det", device=DEV)
    a = w4.w4a16_pack(W)
    b = w4.w4a16_pack(W)
    torch.cuda.synchronize()
    for x, y in ((a.codes, b.codes), (a.scales, b.scales), (a.zeros, b.zeros)):
        assert torch.equal(x, y)


def test_resident_bytes_match_storage_cost():
    N, K = 2048, 4096
    W = gen.weights(N, K, "pack", "bytes", device=DEV)
    p = w4.w4a16_pack(W)
    assert p.nbytes() == O.storage_bytes(N, K)
    assert 8 * p.nbytes() / (N * K) == 4.375
