"""The CPU oracle against facts fixed outside itself (see oracle_pins.py)."""
import numpy as np
import pytest

import oracle as O
from synth import gen
import oracle_pins as P


def test_bf16_rne_matches_torch():
    P.check_bf16_rne_matches_torch()


def test_bf16_rtz_hand():
    P.check_bf16_rtz_hand()


def test_round_half_away():
    P.check_round_half_away()


def test_hand_groups():
    P.check_hand_groups()


def test_dequant_closed_form():
    P.check_dequant_closed_form()


def test_pack_layout():
    P.check_pack_layout()


def test_all_codes_on_grid():
    P.check_all_codes_on_grid()


def test_on_grid_matmul_exact():
    P.check_on_grid_matmul_exact()


def test_brute_force_tiny():
    assert P.check_brute_force() == 0


def test_brute_force_three_groups():
    # K = 384: three groups per row, so a wrong group index shows up
    assert P.check_brute_force(seed=11, M=3, K=384, N=5) == 0


def test_grouped_hand():
    P.check_grouped_hand()


@pytest.mark.parametrize("group", [32, 64])
def test_grouped_all_codes_on_grid(group):
    P.check_all_codes_on_grid(seed=30 + group, N=16, K=512, group=group)


@pytest.mark.parametrize("group", [32, 64])
def test_grouped_brute_force(group):
    assert P.check_brute_force(seed=40 + group, M=3, K=256, N=4, group=group) == 0


@pytest.mark.parametrize("group", [32, 64])
def test_grouped_min_max_codes_generated(group):
    W = gen.weights(64, 1024, "pins", f"g{group}", shift=True)
    assert P.check_min_max_codes(gen.bits(W), group=group) > 0.99


def test_int8_on_grid_and_layout():
    P.check_int8_on_grid_and_layout()


def test_int8_brute_force():
    P.check_int8_brute_force()


def test_awq_prescale():
    P.check_awq_prescale_power_of_two()


def test_awq_fold_hand():
    P.check_awq_fold_hand()


def test_awq_importance_and_scale():
    P.check_awq_importance_and_scale()


def test_awq_equivalence():
    P.check_awq_equivalence_unquantised()


def test_storage_cost():
    P.check_storage_cost()


def test_output_gate():
    P.check_output_gate()


@pytest.mark.parametrize("shift", [False, True])
def test_min_max_codes_generated(shift):
    """Every group of generated weights maps its minimum to code 0 and, when
    it straddles zero, its maximum to code 15."""
    W = gen.weights(256, 4096, "pins", "layer", shift=shift)
    frac = P.check_min_max_codes(gen.bits(W))
    assert frac > 0.99


def test_min_max_codes_awq_prescaled():
    W = gen.weights(128, 1024, "pins", "awq")
    s = gen.channel_vector(1024, "pins", "awq", "s").numpy()
    q, s_bits, z = O.quantize(gen.bits(W), awq_s=s)
    w = (O.bf16_to_f32(gen.bits(W)) * s).astype(np.float32).reshape(128, 8, 128)
    qg = q.reshape(128, 8, 128)
    qmin = np.take_along_axis(qg, w.argmin(-1)[..., None], -1)
    qmax = np.take_along_axis(qg, w.argmax(-1)[..., None], -1)
    assert np.all(qmin == 0) and np.all(qmax == 15)


def test_generator_deterministic():
    a = gen.bits(gen.weights(64, 256, 1, "qkv"))
    b = gen.bits(gen.weights(64, 256, 1, "qkv"))
    c = gen.bits(gen.weights(64, 256, 2, "qkv"))
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    x = gen.bits(gen.activations(3, 256, 1, "qkv"))
    assert np.array_equal(x, gen.bits(gen.activations(3, 256, 1, "qkv")))
    S = gen.salient_channels(4096, 1, "qkv").numpy()
    assert len(S) == 41 and len(np.unique(S)) == 41


def test_dequant_bf16_hand():
    P.check_dequant_bf16_hand()


def test_dequant_bf16_vs_torch():
    P.check_dequant_bf16_vs_torch()


def test_dense_brute_force():
    P.check_dense_brute_force()


def test_dense_matches_fused_on_grid():
    P.check_dense_matches_fused_on_grid()


def test_symmetric_hand():
    P.check_symmetric_hand()


def test_symmetric_invariants():
    P.check_symmetric_invariants()


def test_symmetric_brute_force():
    P.check_symmetric_brute_force()


def test_i64_container():
    P.check_i64_container()


def test_awq_search_alpha_zero_is_plain():
    P.check_awq_search_alpha_zero_is_plain()


def test_awq_search_protects_salient():
    P.check_awq_search_protects_salient()


def test_f64_to_bf16_single_rounding():
    P.check_f64_to_bf16_single_rounding()


def test_silu_identities():
    P.check_silu_identities()


def test_chain_input_hand():
    P.check_chain_input_hand()


def test_chain_two_linears_exact():
    P.check_chain_two_linears_exact()
