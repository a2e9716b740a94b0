"""AWQ helpers on the GPU vs the CPU oracle, and the AWQ-folded decode path
on one layer of the 40-layer stack's shapes."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import assert_output_close, assert_pack_equal, reference, sample_rows

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def test_importance_and_scale():
    T, K = 512, 5120
    Xc = gen.activations(T, K, "awq", "calib", role="Xcal", device=DEV)
    imp = w4.w4a16_awq_importance(Xc)
    s = w4.w4a16_awq_scale(imp, 0.5)
    torch.cuda.synchronize()
    imp_ref = O.awq_importance(gen.bits(Xc))
    # float64 sums in different orders, one rounding to float32: <= 1 ulp
    assert np.allclose(imp.cpu().numpy(), imp_ref, rtol=2 ** -23, atol=0)
    s_ref = O.awq_scale(imp_ref, 0.5)
    assert np.allclose(s.cpu().numpy(), s_ref, rtol=2 ** -22, atol=0)
    for alpha in (0.0, 0.25, 1.0):
        s2 = w4.w4a16_awq_scale(imp, alpha)
        torch.cuda.synchronize()
        assert np.allclose(s2.cpu().numpy(), O.awq_scale(imp.cpu().numpy(), alpha), rtol=2 ** -22)


def test_fold_and_scale_channels_bit_exact():
    K = 5120
    s = gen.channel_vector(K, "awq", "fold", "s", device=DEV)
    gamma = gen.activations(1, K, "awq", "fold", role="gamma", device=DEV)[0].contiguous()
    beta = gen.activations(1, K, "awq", "fold", role="beta", device=DEV)[0].contiguous()
    g0, b0 = gen.bits(gamma), gen.bits(beta)
    w4.w4a16_awq_fold(s, gamma, beta)
    torch.cuda.synchronize()
    s_np = s.cpu().numpy()
    assert np.array_equal(gen.bits(gamma), O.awq_fold(s_np, g0))
    assert np.array_equal(gen.bits(beta), O.awq_fold(s_np, b0))
    X = gen.activations(8, K, "awq", "fold", device=DEV)
    xp = w4.w4a16_scale_channels(X, gamma)
    torch.cuda.synchronize()
    assert np.array_equal(gen.bits(xp), O.apply_channel_scale(gen.bits(X), gen.bits(gamma)))


@pytest.mark.parametrize("M", [1, 8])
def test_awq_folded_stack_layer(M):
    """One layer of the 40-layer stack with the AWQ fold: calibration
    statistic -> s = importance^0.5 -> fold into the producer's gamma ->
    pack W diag(s) -> decode on X' = X * gamma'.  The oracle repeats the
    chain from the same generator inputs on sampled output rows."""
    spec = gen.WORKLOADS["stack40_decode"]
    for layer in spec["layers"]:
        K = layer.K
        Xc = gen.activations(spec["calib_tokens"], K, "stack40", layer.name, role="Xcal", device=DEV)
        W = gen.weights(layer.N, K, "stack40", layer.name, device=DEV)
        X = gen.activations(M, K, "stack40", layer.name, device=DEV)
        s = w4.w4a16_awq_scale(w4.w4a16_awq_importance(Xc), spec["awq_alpha"])
        gamma = torch.ones(K, dtype=torch.bfloat16, device=DEV)
        w4.w4a16_awq_fold(s, gamma)
        Xp = w4.w4a16_scale_channels(X, gamma)
        p = w4.w4a16_pack(W, awq_s=s)
        y = w4.w4a16_gemv(Xp, p)
        torch.cuda.synchronize()

        s_ref = O.awq_scale(O.awq_importance(gen.bits(Xc)), spec["awq_alpha"])
        g_ref = O.awq_fold(s_ref, O.f32_to_bf16_rne(np.ones(K, np.float32)))
        Xp_ref = O.apply_channel_scale(gen.bits(X), g_ref)
        rows = sample_rows(layer.N, 64, seed=layer.N + M)
        ridx = torch.as_tensor(rows, device=DEV)
        y_ref, mag = reference(Xp_ref, gen.bits(W[ridx]), awq_s=s_ref)
        # the per-element half-ulp bound needs identical codes, which holds
        # when both sides produced the same float32 s (the common case)
        same_s = np.array_equal(s.cpu().numpy(), s_ref)
        assert_output_close(y[:, ridx], y_ref, mag, label=f"{layer.name} M={M}", strict=same_s)
        del W, p
        torch.cuda.empty_cache()


def _salient_case(seed, N=64, K=512, T=64):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.02, size=(N, K))
    sal = rng.choice(K, 5, replace=False)
    x = rng.normal(0, 1, size=(T, K))
    x[:, sal] *= 20.0
    return O.f32_to_bf16_rne(w.astype(np.float32)), O.f32_to_bf16_rne(x.astype(np.float32))


@pytest.mark.parametrize("case", ["salient", "generated"])
def test_awq_search_matches_oracle(case):
    """The search on the library's kernels against the oracle's: every error
    within 3% (the GPU outputs are BF16-rounded, the oracle's are fp64), and
    the chosen exponent is one whose oracle error is within 2% of the
    oracle's best."""
    alphas = np.linspace(0, 1, 11)
    if case == "salient":
        Wb, Xb = _salient_case(18)
        Xeb = None
    else:
        N, K = 256, 1024
        Wb = gen.bits(gen.weights(N, K, "awq", "search", device=DEV))
        Xb = gen.bits(gen.activations(128, K, "awq", "search", role="Xcal", device=DEV))
        Xeb = gen.bits(gen.activations(96, K, "awq", "search", device=DEV))
    W = gen.from_bits(Wb, DEV)
    Xc = gen.from_bits(Xb, DEV)
    Xe = None if Xeb is None else gen.from_bits(Xeb, DEV)
    best, errs = w4.w4a16_awq_search(W, Xc, alphas, Xe)
    torch.cuda.synchronize()
    ref, ref_best = O.awq_search(Wb, Xb, alphas, Xeb)
    assert np.allclose(errs, ref, rtol=3e-2), (errs, ref)
    assert ref[best] <= ref[ref_best] * 1.02, (best, ref_best, ref)


def test_search_error_entry_point():
    """w4a16_awq_search_error against the plain definition of the relative
    L2 distance, in float64, on strided outputs."""
    M, N = 37, 1000
    a = gen.activations(M, N, "awq", "err_a", device=DEV)
    b = gen.activations(M, N + 24, "awq", "err_b", device=DEV)[:, 8:N + 8]
    e = w4.w4a16_awq_search_error(a, b)
    torch.cuda.synchronize()
    ya = O.bf16_to_f32(gen.bits(a)).astype(np.float64)
    yb = O.bf16_to_f32(gen.bits(b)).astype(np.float64)
    want = np.sqrt(((ya - yb) ** 2).sum() / (yb ** 2).sum())
    assert abs(float(e.item()) - want) <= 1e-12 * want
    # deterministic, and zero for identical outputs
    assert float(w4.w4a16_awq_search_error(a, b).item()) == float(e.item())
    assert float(w4.w4a16_awq_search_error(b, b).item()) == 0.0
