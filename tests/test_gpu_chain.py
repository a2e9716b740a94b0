"""Chains of dependent linears in one persistent launch (w4a16_chain_*) on
the GPU against the CPU oracle's chain (oracle.chain_ref): every linear's
output, with the glue between them (as is, SwiGLU, single-key attention)
and producer weights."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import gen
from parity import ACC_REL, BF16_HALF_ULP_REL, assert_output_close

pytestmark = pytest.mark.gpu

w4 = pytest.importorskip("int4_weight_only_gemv_amd")
DEV = "cuda"


def build(spec, cfg, M, seed_tag=""):
    """spec: list of (name, N, K, input, params, with_gamma).  Returns the
    library's chain linears, the oracle's linears and X0 (BF16, on the GPU)."""
    lib_lin, ora_lin = [], []
    for name, N, K, kind, params, with_gamma in spec:
        W = gen.weights(N, K, cfg, name + seed_tag, shift=True, device=DEV)
        p = w4.w4a16_pack(W)
        codes, scales, zeros = O.quantize_pack(gen.bits(W))   # the oracle packs the same weights itself
        del W
        g = None
        if with_gamma:
            g = (gen.channel_vector(K, cfg, name + seed_tag, "gamma") * 0.5).to(torch.bfloat16).to(DEV)
        lib_lin.append(dict(p=p, input=kind, params=params, gamma=g))
        ora_lin.append(dict(codes=codes, scales=scales, zeros=zeros, kind=kind, params=params,
                            gamma=None if g is None else gen.bits(g)))
    k_in = max(K for _, _, K, kind, _, _ in spec if kind == "x0")
    X0 = gen.activations(M, k_in, cfg, "x0" + seed_tag, device=DEV)
    return lib_lin, ora_lin, X0


def check_chain(spec, cfg, M, label):
    """Every linear of a chain against the oracle's chain.  Two chains that
    store every output in BF16 drift apart: wherever an exact output lies
    closer to a rounding boundary than the float32 accumulation error, the
    two stored values are neighbours, and such an input element shifts every
    output of the next linear a little, which the following linears pass on.
    Derived tolerance for linear l (0-based): the stored BF16 output alone is
    within 2e-3 relative L2 of the exact one; the drift adds about as much per
    earlier linear in quadrature, and SwiGLU, a product of two drifting
    values, up to sqrt(2) more:
        relative L2 <= 2e-3 f_l,   f_l = sqrt(l + 1) sqrt(2)^(SwiGLU inputs up to l),
    and per element |err| <= 1e-2 f_l (|ref| + rms(ref)) (the method's
    per-element gate, drifting the same way, with the output's own scale in
    place of 1: the chain has no normalisation, so its activations grow
    along it).  The first linear (fed
    by the chain's input) meets the single-linear bound of every other test;
    the glue itself is checked strictly by test_glue_isolated."""
    lib_lin, ora_lin, X0 = build(spec, cfg, M)
    plan = w4.w4a16_chain_prepare(lib_lin, M)
    ys = w4.w4a16_chain_run(plan, X0)
    torch.cuda.synchronize()
    assert w4.w4a16_chain_status(plan) == 0
    ref = O.chain_ref(gen.bits(X0), ora_lin)
    swiglus = 0
    for l, ((x, y_ref, _), L) in enumerate(zip(ref, ora_lin)):
        mag = np.abs(O.bf16_to_f32(x).astype(np.float64)) @ np.abs(O.dequantize(L["codes"], L["scales"], L["zeros"])).T
        name = f"{label} linear {l} ({spec[l][0]})"
        if l == 0:
            assert_output_close(ys[l], y_ref, mag, label=name)
            continue
        swiglus += L["kind"] == "swiglu"
        yv = O.bf16_to_f32(gen.bits(ys[l])).astype(np.float64)
        err = np.abs(yv - y_ref)
        rel = float(np.linalg.norm(err) / np.linalg.norm(y_ref))
        f = np.sqrt(l + 1) * np.sqrt(2.0) ** swiglus
        rms = float(np.sqrt(np.mean(y_ref ** 2)))
        elem = float(np.max(err / (np.abs(y_ref) + rms)))
        print(f"{name}: rel_l2 {rel:.3e}, scaled per-element {elem:.3e} (drift factor {f:.2f})", flush=True)
        assert rel <= O.REL_L2_TOL * f, f"{name}: relative L2 {rel} above {O.REL_L2_TOL * f}"
        assert elem <= O.ELEM_TOL * f, f"{name}: per-element {elem} above {O.ELEM_TOL * f}"
    return plan, ys, X0


def small_decoder(layers=2, hidden=1024, q_heads=8, kv_heads=2, head_dim=128, inter=2816):
    spec = []
    group = q_heads // kv_heads
    for d in range(layers):
        qkv_n = (q_heads + 2 * kv_heads) * head_dim
        spec += [
            (f"qkv{d}", qkv_n, hidden, "x0" if d == 0 else "prev", None, True),
            (f"o{d}", hidden, q_heads * head_dim, "attn1", ((q_heads + kv_heads) * head_dim, head_dim, group), False),
            (f"gate_up{d}", 2 * inter, hidden, "prev", None, True),
            (f"down{d}", hidden, inter, "swiglu", None, False),
        ]
    return spec


@pytest.mark.parametrize("M", [1, 2])
def test_small_decoder_chain(M):
    check_chain(small_decoder(), "chain_small", M, f"small decoder M={M}")


def test_ragged_chain():
    # tiny N (most blocks own no rows), K not a multiple of 2048, the chain's
    # input taken again in the middle, SwiGLU and an attention gather with a
    # group of three
    spec = [
        ("a", 300, 640, "x0", None, False),
        ("b", 6, 256, "prev", None, True),
        ("c", 4100, 1152, "x0", None, True),
        ("d", 517, 2048, "swiglu", None, False),
        ("e", 2000, 384, "attn1", (300, 64, 3), False),
        ("f", 37, 1920, "prev", None, False),
    ]
    for M in (1, 2):
        check_chain(spec, "chain_ragged", M, f"ragged M={M}")


def test_attention_gather_element_by_element():
    # value blocks that start off a multiple of 4 inputs, or heads that are
    # not a multiple of 8 inputs, are gathered element by element
    spec = [
        ("a", 700, 256, "x0", None, False),
        ("b", 300, 640, "attn1", (301, 20, 4), True),    # 32 heads of 20 over 8 kv heads, odd offset
        ("c", 500, 256, "attn1", (2, 64, 2), False),     # 4 heads of 64 over 2 kv heads, offset 2
    ]
    for M in (1, 2):
        check_chain(spec, "chain_gather", M, f"gather M={M}")


@pytest.mark.parametrize("M", [1, 2])
def test_long_inputs_staged_in_several_passes(M):
    # inputs longer than one staging pass (2048 octets of 8 per row set):
    # SwiGLU over 17408 (M = 1) or 9216 (M = 2) inputs, then a plain one
    K = 17408 if M == 1 else 9216
    spec = [
        ("a", 2 * K, 256, "x0", None, False),
        ("b", 400, K, "swiglu", None, True),
        ("c", 256, 384, "prev", None, False),
    ]
    check_chain(spec, "chain_long", M, f"long inputs M={M}")


def test_paired_swiglu_producer_with_few_rows():
    # [gate | up] of 2 x 256 rows: 64 gate batches, so most blocks own none;
    # the consumer's producer weight is applied where the input is formed
    spec = [
        ("a", 512, 384, "x0", None, False),
        ("b", 300, 256, "swiglu", None, True),
        ("c", 2 * 640, 300 - 300 % 128, "prev", None, False),
        ("d", 200, 640, "swiglu", None, False),
    ]
    for M in (1, 2):
        check_chain(spec, "chain_pair_few", M, f"paired few rows M={M}")


def test_longest_input_at_two_rows():
    # the documented maximum input length (32768) at M = 2 (its LDS plan is
    # exactly the 160 KiB a block may hold)
    spec = [
        ("a", 32768, 256, "x0", None, False),
        ("b", 260, 32768, "prev", None, True),
    ]
    check_chain(spec, "chain_max_k", 2, "K = 32768 M=2")


def test_llama8b_decoder_layer_chain():
    # the Llama-3-8B-shaped layer: 32 q / 8 kv heads of 128, SwiGLU 14336
    spec = [
        ("qkv", 6144, 4096, "x0", None, True),
        ("o", 4096, 4096, "attn1", (5120, 128, 4), False),
        ("gate_up", 28672, 4096, "prev", None, True),
        ("down", 4096, 14336, "swiglu", None, False),
    ]
    check_chain(spec, "chain_llama8b", 1, "llama8b layer")


@pytest.mark.parametrize("M", [1, 2])
def test_chain_equals_single_linear_kernels(M):
    # no glue arithmetic: a chain of linears fed as is (and a producer weight)
    # reproduces the one-launch-per-linear path bit for bit
    spec = [("p", 1000, 4096, "x0", None, True), ("q", 3000, 896, "prev", None, False),
            ("r", 700, 2944, "prev", None, False)]
    lib_lin, _, X0 = build(spec, "chain_eq", M)
    plan = w4.w4a16_chain_prepare(lib_lin, M)
    ys = w4.w4a16_chain_run(plan, X0)
    x = w4.w4a16_scale_channels(X0[:, :4096].contiguous(), lib_lin[0]["gamma"])
    y0 = w4.w4a16_gemv(x, lib_lin[0]["p"])
    y1 = w4.w4a16_gemv(y0[:, :896].contiguous(), lib_lin[1]["p"])
    y2 = w4.w4a16_gemv(y1[:, :2944].contiguous(), lib_lin[2]["p"])
    torch.cuda.synchronize()
    for a, b in zip(ys, (y0, y1, y2)):
        assert torch.equal(a, b)


def test_chain_deterministic_and_reusable():
    spec = small_decoder(layers=1)
    lib_lin, _, X0 = build(spec, "chain_det", 1)
    plan = w4.w4a16_chain_prepare(lib_lin, 1)
    first = [y.clone() for y in w4.w4a16_chain_run(plan, X0)]
    for _ in range(3):
        again = w4.w4a16_chain_run(plan, X0)
    torch.cuda.synchronize()
    assert w4.w4a16_chain_status(plan) == 0
    for a, b in zip(first, again):
        assert torch.equal(a, b)


def test_barrier_timeout_is_reported_and_cleared():
    # a spin limit of zero: every block that has to wait gives up at once, so
    # the run ends (with invalid outputs) and reports a timeout; after the
    # status call has cleared the state, a run reproduces a clean run's
    # outputs bit for bit
    spec = small_decoder(layers=3)
    lib_lin, _, X0 = build(spec, "chain_timeout", 1)
    plan = w4.w4a16_chain_prepare(lib_lin, 1)
    clean = [y.clone() for y in w4.w4a16_chain_run(plan, X0)]
    assert w4.w4a16_chain_status(plan) == 0
    plan.plan.spin_limit = 0
    w4.w4a16_chain_run(plan, X0)
    assert w4.w4a16_chain_status(plan) == w4.CHAIN_TIMEOUT
    assert w4.w4a16_chain_status(plan) == 0
    plan.plan.spin_limit = 1 << 22
    ys = w4.w4a16_chain_run(plan, X0)
    torch.cuda.synchronize()
    assert w4.w4a16_chain_status(plan) == 0
    for a, b in zip(clean, ys):
        assert torch.equal(a, b)


def _exact_first_linear(N, K, seed):
    """BF16 weights [N][K] with one on-grid weight 15/16 per row (at input
    p(n)) and zeros elsewhere, and inputs on the grid k/4 (|k| <= 15): every
    float32 sum the kernels form is exact, so the first output is exactly
    15/16 x[p(n)] on both sides."""
    rng = np.random.default_rng(seed)
    w = np.zeros((N, K), np.float32)
    pos = rng.integers(0, K, size=N)
    w[np.arange(N), pos] = 15 / 16
    return torch.from_numpy(w).to(torch.bfloat16)


@pytest.mark.parametrize("kind", ["prev", "swiglu", "attn1"])
@pytest.mark.parametrize("M", [1, 2])
def test_glue_isolated(kind, M):
    """One glue between an exact first linear and a random second one: the
    second output meets the single-linear bound against the oracle.  The only
    allowance is for SwiGLU values the oracle finds within 2^-18 (relative)
    of a BF16 rounding boundary, where float32 and float64 evaluation may
    round apart: there the input may differ by one BF16 ulp."""
    K1, N1 = 1024, 4608
    W1 = _exact_first_linear(N1, K1, seed=M)
    x0 = (np.random.default_rng(7 + M).integers(-15, 16, size=(M, K1)) / 4.0).astype(np.float32)
    X0 = torch.from_numpy(x0).to(torch.bfloat16).to(DEV)
    if kind == "prev":
        K2, params, gam = 4480, None, True
    elif kind == "swiglu":
        K2, params, gam = 2304, None, False
    else:
        K2, params, gam = 1536, (3072, 128, 3), True     # v at 3072, 12 heads of 128 over 4 kv heads
    N2 = 1000
    W2 = gen.weights(N2, K2, "glue", kind, shift=True)
    g = (gen.channel_vector(K2, "glue", kind, "gamma") * 0.5).to(torch.bfloat16) if gam else None
    lib_lin = [dict(p=w4.w4a16_pack(W1.to(DEV)), input="x0"),
               dict(p=w4.w4a16_pack(W2.to(DEV)), input=kind, params=params,
                    gamma=None if g is None else g.to(DEV))]
    c1 = O.quantize_pack(gen.bits(W1))
    c2 = O.quantize_pack(gen.bits(W2))
    ora = [dict(codes=c1[0], scales=c1[1], zeros=c1[2], kind="x0"),
           dict(codes=c2[0], scales=c2[1], zeros=c2[2], kind=kind, params=params,
                gamma=None if g is None else gen.bits(g))]
    plan = w4.w4a16_chain_prepare(lib_lin, M)
    ys = w4.w4a16_chain_run(plan, X0)
    torch.cuda.synchronize()
    assert w4.w4a16_chain_status(plan) == 0
    ref = O.chain_ref(gen.bits(X0), ora)
    # the first output is exact
    assert np.array_equal(O.bf16_to_f32(gen.bits(ys[0])).astype(np.float64), ref[0][1])
    x2, y2_ref, _ = ref[1]
    w_hat = np.abs(O.dequantize(*c2))
    mag = np.abs(O.bf16_to_f32(x2).astype(np.float64)) @ w_hat.T
    extra = np.zeros_like(mag)
    if kind == "swiglu":
        y1 = O.bf16_to_f32(ref[0][2]).astype(np.float64)
        v = O.silu_ref(y1[:, :K2]) * y1[:, K2:2 * K2]
        xb = O.bf16_to_f32(x2).astype(np.float64)
        ulp = np.abs(xb) * 2.0 ** -7 + 1e-38
        # the BF16 value toward zero from v, and the midpoint above it
        _, e = np.frexp(v)
        step = np.ldexp(1.0, e - 8)                 # BF16 spacing at |v|
        lo = np.trunc(v / step) * step
        mid = lo + np.sign(v) * step / 2
        near = np.abs(v - mid) <= np.abs(v) * 2.0 ** -18
        extra = (ulp * near) @ w_hat.T
    err = np.abs(O.bf16_to_f32(gen.bits(ys[1])).astype(np.float64) - y2_ref)
    from parity import BF16_HALF_ULP_REL as H, ACC_REL as A
    bound = H * np.abs(y2_ref) * (1 + 1e-3) + A * mag + extra + 1e-30
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (kind, M, worst, err[worst], bound[worst])
    rel, elem = O.output_errors(O.bf16_to_f32(gen.bits(ys[1])).astype(np.float64), y2_ref)
    assert rel <= O.REL_L2_TOL and elem <= O.ELEM_TOL
