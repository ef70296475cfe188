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


_orig_qv = O.quantize_values
_orig_qk = O.quantize_keys
_orig_dh = O.decode_attention_head
_orig_dk = O.dequantize_keys

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
]


@pytest.mark.parametrize("name,mutant,pins", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(O, name, mutant)
    for pin, *args in pins:
        assert _fails(pin, *args), f"{pin.__name__} did not notice {mutant.__name__}"
