"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Every mutation below is a plausible slip: a dropped term, a wrong sign or
index, a transposed operand.  The test swaps the oracle function for the
mutant, runs the pins that should notice, and expects an assertion failure.
"""
import math

import numpy as np
import pytest

from oracle import kvq_oracle as O
import tests.test_oracle_pins as P


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _signs_after_h(x, signs):
    d = x.shape[-1]
    return O.walsh_hadamard(np.asarray(x, np.float64)) * np.asarray(signs, np.float64) * (1.0 / np.sqrt(d))


def _no_scale(x, signs):
    return O.walsh_hadamard(np.asarray(x, np.float64) * np.asarray(signs, np.float64))


def _values_rotate_wrong_way(v, modality, rot, codebook):
    return _orig_qv(v, modality, np.swapaxes(np.asarray(rot), -1, -2), codebook)


def _keys_map_to_unit(k, signs, codebook, group=32):
    """Maps the group range onto [-1, 1] instead of [c0, c3]."""
    y = O.randomized_hadamard(k, signs)
    L, d = y.shape
    codes, lo, hi = _orig_qk(k, signs, codebook, group)
    gi = np.arange(L) // group
    LO, HI = lo.astype(np.float64)[gi], hi.astype(np.float64)[gi]
    with np.errstate(divide="ignore", invalid="ignore"):
        z = -1.0 + (y - LO) * 2.0 / (HI - LO)
    bad = O.nearest_level(np.nan_to_num(z), codebook)
    bad[HI == LO] = 0
    return bad, lo, hi


def _decode_rotates_with_transpose(q_rot, k_codes, lo16, hi16, v_codes, norms16, modality, rot, codebook, scale,
                                   retained=None):
    return _orig_dh(q_rot, k_codes, lo16, hi16, v_codes, norms16, modality,
                    np.swapaxes(np.asarray(rot), -1, -2), codebook, scale, retained)


def _decode_drops_scale(q_rot, k_codes, lo16, hi16, v_codes, norms16, modality, rot, codebook, scale,
                        retained=None):
    return _orig_dh(q_rot, k_codes, lo16, hi16, v_codes, norms16, modality, rot, codebook, 1.0, retained)


def _decode_ignores_retained_set(q_rot, k_codes, lo16, hi16, v_codes, norms16, modality, rot, codebook, scale,
                                 retained=None):
    if retained is not None and not np.any(retained):
        return np.zeros(q_rot.shape[-1])
    return _orig_dh(q_rot, k_codes, lo16, hi16, v_codes, norms16, modality, rot, codebook, scale)


def _rotate_query_wrong_head(q, signs, n_kv_heads):
    hq = q.shape[0]
    out = np.empty_like(np.asarray(q, np.float64))
    for i in range(hq):
        out[i] = O.randomized_hadamard(q[i], signs[i % n_kv_heads])
    return out


def _dequant_keys_off_by_one_level(codes, lo16, hi16, codebook, group=32):
    return _orig_dk(np.minimum(codes + 1, 3).astype(np.uint8), lo16, hi16, codebook, group)


def _ties_go_down(z, codebook):
    """Wrong threshold side: a value exactly on a threshold takes the lower level."""
    b = O.decision_thresholds(codebook)
    return (np.asarray(z)[..., None] > b).sum(axis=-1).astype(np.uint8)


def _keys_per_group_scalar_stats(k, signs, codebook, group=32):
    """One min / max per group over every channel instead of per channel."""
    y = O.randomized_hadamard(k, signs)
    L, d = y.shape
    ng = -(-L // group)
    c = np.asarray(codebook, np.float32).astype(np.float64)
    codes = np.zeros((L, d), np.uint8)
    lo16 = np.zeros((ng, d), np.float16)
    hi16 = np.zeros((ng, d), np.float16)
    for g in range(ng):
        yg = y[g * group:(g + 1) * group]
        lo16[g] = np.float16(yg.min())
        hi16[g] = np.float16(yg.max())
        LO, HI = lo16[g].astype(np.float64), hi16[g].astype(np.float64)
        z = c[0] + (yg - LO) * (c[-1] - c[0]) / np.where(HI > LO, HI - LO, 1.0)
        codes[g * group:(g + 1) * group] = np.where(HI > LO, O.nearest_level(z, codebook), 0)
    return codes, lo16, hi16


def _key_z_from_unrounded_range(k, signs, lo16, hi16, codebook, group=32):
    """z taken against the exact group min / max instead of the stored fp16 LO / HI."""
    y = O.randomized_hadamard(k, signs)
    ng = -(-y.shape[0] // group)
    lo = np.stack([y[g * group:(g + 1) * group].min(0) for g in range(ng)])
    hi = np.stack([y[g * group:(g + 1) * group].max(0) for g in range(ng)])
    return _orig_knv(k, signs, lo, hi, codebook, group)


def _key_z_on_unit_range(k, signs, lo16, hi16, codebook, group=32):
    """z mapped onto [-1, 1] instead of [c0, c3]."""
    z = _orig_knv(k, signs, lo16, hi16, codebook, group)
    c = np.asarray(codebook, np.float32).astype(np.float64)
    return -1.0 + (z - c[0]) * 2.0 / (c[-1] - c[0])


def _bf16_as_upper_fp16(bits):
    """Reads the raw 16 bits as IEEE half precision instead of bfloat16."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _bf16_truncated_fraction(bits):
    """Drops the lowest fraction bit of every bfloat16 value."""
    u = (np.asarray(bits, dtype=np.uint16) & np.uint16(0xFFFE)).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


_orig_qv = O.quantize_values
_orig_qk = O.quantize_keys
_orig_dh = O.decode_attention_head
_orig_dk = O.dequantize_keys
_orig_knv = O.key_normalized_values

MUTANTS = [
    ("randomized_hadamard", _signs_after_h, [(P.test_randomized_hadamard_is_H_times_D, 64)]),
    ("randomized_hadamard", _no_scale, [(P.test_randomized_hadamard_orthonormal_and_roundtrip, 64)]),
    ("quantize_values", _values_rotate_wrong_way, [(P.test_value_codes_roundtrip_when_value_sits_on_levels, 64)]),
    ("quantize_keys", _keys_map_to_unit, [(P.test_key_code_is_nearest_reconstruction_level, 0, 256)]),
    ("decode_attention_head", _decode_rotates_with_transpose,
     [(P.test_decode_equals_dense_attention_over_dequantized_cache, 37)]),
    ("decode_attention_head", _decode_drops_scale,
     [(P.test_decode_equals_dense_attention_over_dequantized_cache, 37)]),
    ("decode_attention_head", _decode_ignores_retained_set,
     [(P.test_decode_over_a_retained_position_set, "random")]),
    ("rotate_query", _rotate_query_wrong_head,
     [(P.test_decode_equals_dense_attention_over_dequantized_cache, 37)]),
    ("dequantize_keys", _dequant_keys_off_by_one_level, [(P.test_key_group_range_is_restored, 0, 300)]),
    ("nearest_level", _ties_go_down, [(P.test_nearest_level_ties_go_up,)]),
    ("quantize_keys", _keys_per_group_scalar_stats, [(P.test_key_group_range_is_restored, 0, 300)]),
    ("key_normalized_values", _key_z_from_unrounded_range, [(P.test_key_normalized_values_decide_the_codes, 0, 289)]),
    ("key_normalized_values", _key_z_on_unit_range, [(P.test_key_normalized_values_decide_the_codes, 0, 289),
                                                     (P.test_key_normalized_values_on_a_hand_worked_group,)]),
    ("bf16_to_f64", _bf16_as_upper_fp16, [(P.test_bf16_to_f64_on_every_bit_pattern,)]),
    ("bf16_to_f64", _bf16_truncated_fraction, [(P.test_bf16_to_f64_on_every_bit_pattern,)]),
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(O, name, mutant)
    for pin, *args in pins:
        assert _fails(pin, *args), f"{pin.__name__} did not notice {mutant.__name__}"


# ------------------------------------------------ value-basis calibration

from oracle import kvq_calib_oracle as CO  # noqa: E402
import tests.test_calib_pins as CP  # noqa: E402

_orig_ac = CO.attention_contribution
_orig_wc = CO.weighted_covariance
_orig_eb = CO.eigenbasis
_orig_qe = CO.value_quantization_error


def _contribution_over_queries(k, q_rows, scale):
    """Normalises each token's scores over the queries instead of the tokens."""
    s = scale * (np.asarray(q_rows, np.float64) @ np.asarray(k, np.float64).T)
    p = np.exp(s - s.max(axis=0, keepdims=True))
    p = p / p.sum(axis=0, keepdims=True)
    return p.mean(axis=0) / k.shape[0]


def _contribution_wrong_head(k, q, scale):
    n, hkv, d = k.shape
    nq, hq, _ = q.shape
    out = np.zeros((hkv, n))
    for h in range(hkv):
        rows = q[:, h::hkv, :].reshape(-1, d)       # heads h, h + Hkv, ... instead of a contiguous group
        out[h] = CO.attention_contribution(k[:, h, :], rows, scale)
    return out


def _covariance_uncentred(v, modality, w):
    Cm, W, mu = _orig_wc(v, modality, w)
    for m in range(3):
        if W[m] > 0:
            Cm[m] = Cm[m] + np.outer(mu[m], mu[m])
    return Cm, W, mu


def _covariance_squared_weights(v, modality, w):
    return _orig_wc(v, modality, np.asarray(w, np.float64) ** 2)


def _covariance_divides_by_count(v, modality, w):
    Cm, W, mu = _orig_wc(v, modality, w)
    for m in range(3):
        cnt = int((np.asarray(modality) == m).sum())
        if W[m] > 0:
            Cm[m] = Cm[m] * W[m] / cnt
    return Cm, W, mu


def _eigenbasis_ascending(C):
    R, lam = _orig_eb(C)
    return R[:, ::-1].copy(), lam[::-1].copy()


def _eigenbasis_rows(C):
    R, lam = _orig_eb(C)
    return R.T.copy(), lam


def _eigenbasis_no_sign_rule(C):
    R, lam = _orig_eb(C)
    return -R, lam


def _error_reconstructs_with_transpose(v, modality, rot, codebook):
    """Quantizes with R_m^T v but reconstructs with R_m^T instead of R_m."""
    codes, norms = O.quantize_values(v, modality, rot, codebook)
    vt = O.dequantize_values_rotated(codes, norms, codebook)
    R = np.asarray(rot, np.float32).astype(np.float64)
    err = np.full(3, np.nan)
    for m in range(3):
        idx = np.asarray(modality) == m
        if idx.any():
            vh = vt[idx] @ R[m]
            err[m] = ((v[idx] - vh) ** 2).sum() / (v[idx] ** 2).sum()
    return err


CALIB_MUTANTS = [
    ("attention_contribution", _contribution_over_queries,
     [(CP.test_weights_of_each_head_sum_to_one_and_follow_permutation,), (CP.test_two_tokens_follow_the_logistic_function,)]),
    ("contribution_weights", _contribution_wrong_head, [(CP.test_query_heads_map_to_kv_head_floor_i_over_g,)]),
    ("weighted_covariance", _covariance_uncentred,
     [(CP.test_uniform_weights_give_population_covariance,), (CP.test_covariance_is_shift_invariant_and_per_modality,)]),
    ("weighted_covariance", _covariance_squared_weights,
     [(CP.test_doubled_weight_equals_duplicated_token_and_scale_invariance,)]),
    ("weighted_covariance", _covariance_divides_by_count,
     [(CP.test_covariance_recovers_constructed_matrix,)]),
    ("eigenbasis", _eigenbasis_ascending, [(CP.test_eigenbasis_of_diagonal_is_sorted_permutation,)]),
    ("eigenbasis", _eigenbasis_rows, [(CP.test_eigenbasis_recovers_known_basis_with_sign_rule,)]),
    ("eigenbasis", _eigenbasis_no_sign_rule, [(CP.test_eigenbasis_two_by_two_closed_form,),
                                              (CP.test_calibration_recovers_each_modality_basis_exactly,)]),
    ("value_quantization_error", _error_reconstructs_with_transpose,
     [(CP.test_error_harness_matches_the_quantizer_distortion,),
      (CP.test_error_harness_is_invariant_under_a_common_rotation,)]),
]


@pytest.mark.parametrize("name,mutant,pins", CALIB_MUTANTS, ids=[m[1].__name__ for m in CALIB_MUTANTS])
def test_planted_calibration_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(CO, name, mutant)
    for pin, *args in pins:
        assert _fails(pin, *args), f"{pin.__name__} did not notice {mutant.__name__}"


# ------------------------------------------- TurboQuant baseline and harness

import tests.test_turbo_pins as TP  # noqa: E402

_orig_qkt = O.quantize_keys_per_token
_orig_hvb = O.hadamard_value_basis
_orig_dkt = O.dequantize_keys_per_token
_orig_go = O.grouping_order


def _per_token_keys_without_sqrt_d(k, signs, codebook):
    L, d = k.shape
    y = O.randomized_hadamard(k, signs)
    n = np.sqrt(np.sum(np.asarray(k, np.float64) ** 2, axis=1))
    codes = np.zeros((L, d), np.uint8)
    ok = n > 0
    codes[ok] = O.nearest_level(y[ok] / n[ok][:, None], codebook)
    return codes, n.astype(np.float16)


def _hadamard_basis_transposed(signs):
    return _orig_hvb(signs).T


def _per_token_dequant_drops_norm(codes, norms16, codebook):
    return _orig_dkt(codes, np.ones_like(norms16), codebook)


def _modality_order_loses_time(modality, order, seed=0):
    """Modality blocks, but each in reverse stream order."""
    if order == "modality":
        return np.lexsort((-np.arange(len(modality)), modality))
    return _orig_go(modality, order, seed)


TURBO_MUTANTS = [
    ("quantize_keys_per_token", _per_token_keys_without_sqrt_d,
     [(TP.test_per_token_key_codes_and_norms,), (TP.test_per_token_keys_reach_the_quantizer_distortion, 64)]),
    ("hadamard_value_basis", _hadamard_basis_transposed, [(TP.test_hadamard_value_basis_is_the_randomized_hadamard,)]),
    ("dequantize_keys_per_token", _per_token_dequant_drops_norm,
     [(TP.test_per_token_keys_reach_the_quantizer_distortion, 128)]),
    ("grouping_order", _modality_order_loses_time,
     [(TP.test_grouping_orders_are_permutations_with_the_stated_structure,)]),
]


@pytest.mark.parametrize("name,mutant,pins", TURBO_MUTANTS, ids=[m[1].__name__ for m in TURBO_MUTANTS])
def test_planted_baseline_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(O, name, mutant)
    for pin, *args in pins:
        assert _fails(pin, *args), f"{pin.__name__} did not notice {mutant.__name__}"
