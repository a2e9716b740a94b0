"""The allocation-free chain entry point (w4a16_chain_run_noalloc) through
the C ABI against the prepared-plan path (w4a16_chain_prepare + run) on the
same chains: two calls in a row, the second with a smaller chain and input;
outputs equal bit for bit (the same kernel, the same arithmetic)."""
import pytest
import torch

from synth import gen

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def decoder(layers, tag):
    hidden, qh, kvh, hd, inter = 1024, 8, 2, 128, 2816
    lin = []
    for d in range(layers):
        for name, N, K, kind, params in (
                ("qkv", (qh + 2 * kvh) * hd, hidden, "x0" if d == 0 else "prev", None),
                ("o", hidden, qh * hd, "attn1", ((qh + kvh) * hd, hd, qh // kvh)),
                ("gate_up", 2 * inter, hidden, "prev", None),
                ("down", hidden, inter, "swiglu", None)):
            W = gen.weights(N, K, "noalloc", f"{tag}{name}{d}", shift=True, device=DEV)
            g = (gen.channel_vector(K, "noalloc", f"{tag}{name}{d}", "g") * 0.5).to(torch.bfloat16).to(DEV)
            lin.append(dict(p=w4.w4a16_pack(W), input=kind, params=params, gamma=g))
            del W
    return lin


def test_noalloc_matches_prepared_chain_twice():
    for layers, M in ((2, 2), (1, 1)):          # the second call: a smaller chain and input
        lin = decoder(layers, f"L{layers}")
        X0 = gen.activations(M, 1024, "noalloc", f"x{layers}", device=DEV)
        plan = w4.w4a16_chain_prepare(lin, M)
        ref = [y.clone() for y in w4.w4a16_chain_run(plan, X0)]
        torch.cuda.synchronize()
        assert w4.w4a16_chain_status(plan) == 0
        outs, status = w4.w4a16_chain_run_noalloc(lin, X0)
        torch.cuda.synchronize()
        assert status == 0
        assert len(outs) == len(ref)
        for a, b in zip(outs, ref):
            assert torch.equal(a, b)


def test_noalloc_rejects_too_many_linears():
    lin = decoder(1, "big")
    X0 = gen.activations(1, 1024, "noalloc", "xbig", device=DEV)
    # one more linear than the fixed device array holds descriptors for
    chain = [lin[0]] + [dict(p=lin[2]["p"], input="x0")] * 256
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_chain_run_noalloc(chain, X0)
    assert e.value.status == 3
