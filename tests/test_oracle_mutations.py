"""Plant plausible mistakes in the CPU oracle and check that a pin catches
each one.  The mutations live only here, on the CPU, inside monkeypatch."""
import numpy as np
import pytest

import oracle
import oracle.w4a16_ref as R
import oracle_pins as P

ALL_PINS = [
    P.check_hand_groups, P.check_dequant_closed_form, P.check_pack_layout,
    P.check_all_codes_on_grid, P.check_on_grid_matmul_exact,
    lambda: P.check_brute_force(seed=11, M=3, K=384, N=5),
    P.check_awq_prescale_power_of_two, P.check_awq_fold_hand,
    P.check_awq_importance_and_scale, P.check_awq_equivalence_unquantised,
    P.check_storage_cost,
    P.check_dequant_bf16_hand, P.check_dequant_bf16_vs_torch,
    P.check_dense_brute_force, P.check_dense_matches_fused_on_grid,
    P.check_symmetric_hand, P.check_symmetric_invariants, P.check_symmetric_brute_force,
    P.check_i64_container,
    P.check_awq_search_alpha_zero_is_plain, P.check_awq_search_protects_salient,
    P.check_grouped_hand,
    lambda: P.check_all_codes_on_grid(seed=21, N=8, K=256, group=32),
    lambda: P.check_brute_force(seed=22, M=2, K=128, N=3, group=32),
    P.check_int8_on_grid_and_layout, P.check_int8_brute_force,
    P.check_f64_to_bf16_single_rounding, P.check_silu_identities, P.check_chain_input_hand,
    P.check_chain_two_linears_exact,
]


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(R, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _some_pin_fails():
    failed = 0
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, OverflowError, ZeroDivisionError, IndexError):
            failed += 1
    return failed


def _half_even(v):
    return np.round(np.asarray(v, dtype=np.float32).astype(np.float64))


def _scale_rne(x):
    return R.f32_to_bf16_rne(x)


def _pack_reversed(q):
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    q8 = q.reshape(N, K // 8, 8)
    w = np.zeros((N, K // 8), np.uint32)
    for j in range(8):
        w |= q8[:, :, 7 - j] << np.uint32(4 * j)
    return w


def _dequant_sign(codes, scales, zeros):
    q = R.unpack_codes(codes).astype(np.float64)
    K = q.shape[1]
    s = R.bf16_to_f32(scales).astype(np.float64)
    z = np.asarray(zeros, np.float64)
    g = np.arange(K) // 128
    return (z[:, g] - q) * s[:, g]


def _dequant_group_index(codes, scales, zeros):
    q = R.unpack_codes(codes).astype(np.float64)
    K = q.shape[1]
    s = R.bf16_to_f32(scales).astype(np.float64)
    z = np.asarray(zeros, np.float64)
    g = np.arange(K) % s.shape[1]
    return (q - z[:, g]) * s[:, g]


def _matmul_transposed(X_bits, codes, scales, zeros, rows=None):
    if rows is not None:
        codes, scales, zeros = codes[rows], scales[rows], zeros[rows]
    w = R.dequantize(codes, scales, zeros)
    x = R.bf16_to_f32(X_bits).astype(np.float64)
    return (w @ x.T)


def _scale_zero_clamped(wg, qmax=15):
    s_bits, s, z = ORIG["group_scale_zero"](wg, qmax)
    return s_bits, s, np.clip(z, 0, qmax)


def _scale_zero_no_degenerate(wg, qmax=15):
    w = np.asarray(wg, dtype=np.float32)
    mn, mx = w.min(-1), w.max(-1)
    t = ((mx - mn) / np.float32(15)).astype(np.float32)
    s_bits = R.f32_to_bf16_rtz(t)
    s = R.bf16_to_f32(s_bits)
    z = R.round_half_away((-mn / s).astype(np.float32)).astype(np.int64)
    return s_bits, s, z


def _scale_zero_div16(wg, qmax=15):
    w = np.asarray(wg, dtype=np.float32)
    mn, mx = w.min(-1), w.max(-1)
    t = ((mx - mn) / np.float32(16)).astype(np.float32)
    s_bits = R.f32_to_bf16_rtz(t)
    s = R.bf16_to_f32(s_bits)
    s_bits = np.where(s < R.FLT_MIN, np.uint16(0x3F80), s_bits).astype(np.uint16)
    s = R.bf16_to_f32(s_bits)
    z = R.round_half_away((-mn / s).astype(np.float32)).astype(np.int64)
    return s_bits, s, z


def _codes_against_unrounded(wg, s, z, qmax=15):
    w = np.asarray(wg, dtype=np.float32)
    mn, mx = w.min(-1), w.max(-1)
    t = ((mx - mn) / np.float32(15)).astype(np.float32)
    t = np.where(t > 0, t, s).astype(np.float32)
    r = R.round_half_away((w / t[..., None]).astype(np.float32)).astype(np.int64)
    return np.clip(r + z[..., None], 0, 15).astype(np.uint8)


def _quantize_ignores_awq(W_bits, awq_s=None, group=128):
    return ORIG["quantize"](W_bits, None, group)


def _quantize_ignores_group(W_bits, awq_s=None, group=128):
    return ORIG["quantize"](W_bits, awq_s)


def _quantize_int8_div256(W_bits, awq_s=None):
    N, K = W_bits.shape
    wg = R.bf16_to_f32(W_bits).reshape(N, K // 128, 128)
    s_bits, s, z = R.group_scale_zero(wg, 256)
    return R.group_codes(wg, s, z, 255).reshape(N, K), s_bits, z.astype(np.int32)


def _pack_int8_reversed(q):
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    q4 = q.reshape(N, K // 4, 4)
    words = np.zeros((N, K // 4), dtype=np.uint32)
    for j in range(4):
        words |= q4[:, :, 3 - j] << np.uint32(8 * j)
    return words


def _dequant_group_128(codes, scales, zeros):
    # the group index taken as k // 128 whatever the shapes say
    q = R.unpack_codes(codes).astype(np.float64)
    K = q.shape[1]
    s = R.bf16_to_f32(scales).astype(np.float64)
    z = np.asarray(zeros, np.float64)
    g = np.arange(K) // 128
    return (q - z[:, g]) * s[:, g]


def _fold_multiplies(s, gamma_bits):
    g = R.bf16_to_f32(gamma_bits)
    return R.f32_to_bf16_rne((g * np.asarray(s, np.float32)).astype(np.float32))


def _importance_no_abs(Xcal_bits):
    return R.bf16_to_f32(Xcal_bits).astype(np.float64).mean(axis=0)


def _dequant_bf16_truncated(codes, scales, zeros):
    q = R.unpack_codes(codes).astype(np.int64)
    K = q.shape[1]
    s = R.bf16_to_f32(scales)
    z = np.asarray(zeros, np.int64)
    g = np.arange(K) // 128
    return R.f32_to_bf16_rtz(np.multiply((q - z[:, g]).astype(np.float32), s[:, g], dtype=np.float32))


def _dequant_bf16_zero_added(codes, scales, zeros):
    q = R.unpack_codes(codes).astype(np.int64)
    K = q.shape[1]
    s = R.bf16_to_f32(scales)
    z = np.asarray(zeros, np.int64)
    g = np.arange(K) // 128
    return R.f32_to_bf16_rne(np.multiply((q + z[:, g]).astype(np.float32), s[:, g], dtype=np.float32))


def _dense_drops_last_k(X_bits, W_bits, rows=None):
    W = np.asarray(W_bits)
    if rows is not None:
        W = W[rows]
    x = R.bf16_to_f32(X_bits).astype(np.float64)[:, :-1]
    w = R.bf16_to_f32(W).astype(np.float64)[:, :-1]
    return x @ w.T


def _sym_scale_div8(wg):
    w = np.asarray(wg, dtype=np.float32)
    a = np.abs(w).max(axis=-1).astype(np.float32)
    s_bits = R.f32_to_bf16_rtz((a / np.float32(8)).astype(np.float32))
    s_bits = np.where(R.bf16_to_f32(s_bits) < R.FLT_MIN, np.uint16(0x3F80), s_bits).astype(np.uint16)
    return s_bits, R.bf16_to_f32(s_bits)


def _sym_scale_max_only(wg):
    w = np.asarray(wg, dtype=np.float32)
    a = w.max(axis=-1).astype(np.float32)
    s_bits = R.f32_to_bf16_rtz((a / np.float32(7)).astype(np.float32))
    s_bits = np.where(R.bf16_to_f32(s_bits) < R.FLT_MIN, np.uint16(0x3F80), s_bits).astype(np.uint16)
    return s_bits, R.bf16_to_f32(s_bits)


def _i64_high_nibble_first(q):
    q = np.asarray(q, dtype=np.uint64)
    N, K = q.shape
    q16 = q.reshape(N, K // 16, 16)
    words = np.zeros((N, K // 16), dtype=np.uint64)
    for j in range(16):
        words |= (q16[:, :, j ^ 1] & np.uint64(0xF)) << np.uint64(4 * j)
    return words.view(np.int64)


def _search_multiplies_x(W_bits, Xcal_bits, alphas, X_bits=None):
    X_bits = Xcal_bits if X_bits is None else X_bits
    imp = R.awq_importance(Xcal_bits)
    yd = R.dense_matmul_ref(X_bits, W_bits)
    errs = []
    for a in alphas:
        s = R.awq_scale(imp, a)
        codes, scales, zeros = R.quantize_pack(W_bits, s)
        g = R.f32_to_bf16_rne(np.asarray(s, np.float32))
        y = R.matmul_ref(R.apply_channel_scale(X_bits, g), codes, scales, zeros)
        errs.append(np.linalg.norm(y - yd) / np.linalg.norm(yd))
    errs = np.asarray(errs)
    return errs, int(np.argmin(errs))


def _bf16_via_f32(x):
    return R.f32_to_bf16_rne(np.asarray(x, np.float64).astype(np.float32))


def _silu_sign(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(g))


_chain_input_orig = R.chain_input


def _chain_attn_mod(kind, y_prev_bits, K, params=None, gamma_bits=None, x0_bits=None):
    if kind == "attn1":
        v_off, hd, group = params
        y = R.bf16_to_f32(np.asarray(y_prev_bits)).astype(np.float64)
        k = np.arange(K)
        x = y[:, v_off + (k // hd % group) * hd + k % hd]
        return R.f64_to_bf16_rne(x)
    return _chain_input_orig(kind, y_prev_bits, K, params, gamma_bits, x0_bits)


def _chain_swiglu_swapped(kind, y_prev_bits, K, params=None, gamma_bits=None, x0_bits=None):
    if kind == "swiglu":
        y = R.bf16_to_f32(np.asarray(y_prev_bits)).astype(np.float64)
        return R.f64_to_bf16_rne(R.silu_ref(y[:, K:2 * K]) * y[:, :K])
    return _chain_input_orig(kind, y_prev_bits, K, params, gamma_bits, x0_bits)


def _chain_ignores_gamma(kind, y_prev_bits, K, params=None, gamma_bits=None, x0_bits=None):
    return _chain_input_orig(kind, y_prev_bits, K, params, None, x0_bits)


def _chain_ref_feeds_x0(x0_bits, linears):
    out = []
    for L in linears:
        K = L["codes"].shape[1] * 8
        x = R.chain_input("x0", None, K, None, L.get("gamma"), x0_bits)
        y = R.matmul_ref(x, L["codes"], L["scales"], L["zeros"])
        out.append((x, y, R.f64_to_bf16_rne(y)))
    return out


ORIG = {n: getattr(R, n) for n in ["group_scale_zero", "quantize"]}

MUTATIONS = {
    "ties_to_even": ("round_half_away", _half_even),
    "scale_round_nearest": ("f32_to_bf16_rtz", _scale_rne),
    "nibble_order_reversed": ("pack_codes", _pack_reversed),
    "dequant_sign_flipped": ("dequantize", _dequant_sign),
    "dequant_wrong_group": ("dequantize", _dequant_group_index),
    "matmul_transposed": ("matmul_ref", _matmul_transposed),
    "zero_point_clamped": ("group_scale_zero", _scale_zero_clamped),
    "no_degenerate_rule": ("group_scale_zero", _scale_zero_no_degenerate),
    "divide_by_16": ("group_scale_zero", _scale_zero_div16),
    "codes_vs_unrounded_scale": ("group_codes", _codes_against_unrounded),
    "awq_scale_ignored": ("quantize", _quantize_ignores_awq),
    "fold_multiplies": ("awq_fold", _fold_multiplies),
    "importance_without_abs": ("awq_importance", _importance_no_abs),
    "dequant_bf16_truncated": ("dequantize_bf16", _dequant_bf16_truncated),
    "dequant_bf16_zero_added": ("dequantize_bf16", _dequant_bf16_zero_added),
    "dense_drops_last_k": ("dense_matmul_ref", _dense_drops_last_k),
    "symmetric_divide_by_8": ("group_scale_symmetric", _sym_scale_div8),
    "symmetric_scale_from_max_not_magnitude": ("group_scale_symmetric", _sym_scale_max_only),
    "i64_high_nibble_first": ("pack_codes_i64", _i64_high_nibble_first),
    "awq_search_multiplies_x": ("awq_search", _search_multiplies_x),
    "quantize_ignores_group": ("quantize", _quantize_ignores_group),
    "dequant_group_always_128": ("dequantize", _dequant_group_128),
    "int8_divide_by_256": ("quantize_int8", _quantize_int8_div256),
    "int8_bytes_reversed": ("pack_codes_int8", _pack_int8_reversed),
    "bf16_store_rounds_twice": ("f64_to_bf16_rne", _bf16_via_f32),
    "silu_sign_flipped": ("silu_ref", _silu_sign),
    "attention_head_modulo": ("chain_input", _chain_attn_mod),
    "swiglu_halves_swapped": ("chain_input", _chain_swiglu_swapped),
    "chain_ignores_gamma": ("chain_input", _chain_ignores_gamma),
    "chain_feeds_x0_everywhere": ("chain_ref", _chain_ref_feeds_x0),
}


def test_unmutated_oracle_passes_all_pins():
    assert _some_pin_fails() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(monkeypatch, name):
    target, fn = MUTATIONS[name]
    _patch(monkeypatch, target, fn)
    assert _some_pin_fails() > 0, f"no pin catches mutation {name}"
