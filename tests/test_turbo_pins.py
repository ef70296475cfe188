"""Pins of the TurboQuant baseline codec and the key-grouping harness (CPU).

The per-token key codec is checked against the exact distortion of the
4-level quantizer for an isotropic source and a dense brute-force decode;
the shared Hadamard value basis against the transform it stands for; the
grouping harness against its definition's special cases (identity order,
block-constant keys, permutations, stationary streams).
"""
import math

import numpy as np
import pytest

from oracle import kvq_oracle as O
from tests.test_calib_pins import _sphere_marginal_distortion

CB = (-1.5104, -0.4528, 0.4528, 1.5104)


def _signs(rng, d):
    return np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)


def test_hadamard_value_basis_is_the_randomized_hadamard():
    rng = np.random.default_rng(0)
    d = 64
    s = _signs(rng, d)
    R = O.hadamard_value_basis(s)
    v = rng.standard_normal((5, d))
    np.testing.assert_allclose(v @ R, O.randomized_hadamard(v, s), atol=1e-14)
    np.testing.assert_allclose(R.T @ R, np.eye(d), atol=1e-14)


@pytest.mark.parametrize("d", [64, 128])
def test_per_token_keys_reach_the_quantizer_distortion(d):
    # isotropic keys: every normalised rotated coordinate follows the sphere
    # marginal, so the relative error is that law's 4-level distortion
    rng = np.random.default_rng(d)
    k = rng.standard_normal((3000, d)) * 2.5
    err = O.per_token_key_error(k, _signs(rng, d), CB)
    assert abs(err - _sphere_marginal_distortion(d, CB)) < 0.002


def test_per_token_key_codes_and_norms():
    rng = np.random.default_rng(1)
    d = 64
    s = _signs(rng, d)
    k = rng.standard_normal((40, d))
    k[3] = 0.0
    codes, norms = O.quantize_keys_per_token(k, s, CB)
    np.testing.assert_array_equal(norms, np.sqrt((k * k).sum(1)).astype(np.float16))
    assert not codes[3].any() and norms[3] == 0
    z = O.key_per_token_normalized_values(k, s)
    np.testing.assert_array_equal(codes[np.arange(40) != 3], O.nearest_level(z[np.arange(40) != 3], CB))
    # the normalised rotated key has norm sqrt(d)
    np.testing.assert_allclose(np.sqrt((z[np.arange(40) != 3] ** 2).sum(1)), math.sqrt(d), rtol=1e-12)


def test_per_token_decode_equals_dense_brute_force():
    # materialise every key and value in the original domain, attend densely
    rng = np.random.default_rng(2)
    d, L = 64, 57
    s = _signs(rng, d)
    k = rng.standard_normal((L, d)) * 1.7
    v = rng.standard_normal((L, d))
    mod = rng.integers(0, 3, L).astype(np.uint8)
    rot = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(3)]).astype(np.float32)
    kc, kn = O.quantize_keys_per_token(k, s, CB)
    vc, vn = O.quantize_values(v, mod, rot, CB)
    q = rng.standard_normal(d)
    scale = 1 / math.sqrt(d)
    got = O.decode_attention_head_per_token_keys(O.randomized_hadamard(q, s), kc, kn, vc, vn, mod, rot, CB, scale)
    lev = np.asarray(CB, np.float32).astype(np.float64)
    K = O.inverse_randomized_hadamard(kn.astype(np.float64)[:, None] / math.sqrt(d) * lev[kc], s)
    vt = O.dequantize_values_rotated(vc, vn, CB)
    R = rot.astype(np.float64)
    V = np.stack([R[mod[t]] @ vt[t] for t in range(L)])
    sc = scale * (K @ q)
    p = np.exp(sc - sc.max())
    p /= p.sum()
    np.testing.assert_allclose(got, p @ V, rtol=0, atol=1e-12)


def test_grouping_orders_are_permutations_with_the_stated_structure():
    rng = np.random.default_rng(3)
    mod = rng.integers(0, 3, 500).astype(np.uint8)
    for order in O.GROUP_ORDERS:
        perm = O.grouping_order(mod, order, seed=5)
        np.testing.assert_array_equal(np.sort(perm), np.arange(500))
    np.testing.assert_array_equal(O.grouping_order(mod, "temporal"), np.arange(500))
    pm = O.grouping_order(mod, "modality")
    assert np.all(np.diff(mod[pm].astype(int)) >= 0)                       # modality blocks
    for m in range(3):
        blk = pm[mod[pm] == m]
        assert np.all(np.diff(blk) > 0)                                      # time order inside
    ps = O.grouping_order(mod, "modality_shuffled", seed=5)
    assert np.all(np.diff(mod[ps].astype(int)) >= 0)
    assert not np.all(np.diff(ps[mod[ps] == 0]) > 0)                        # shuffled inside


def test_temporal_grouping_error_is_the_codec_error():
    rng = np.random.default_rng(4)
    d, L = 64, 300
    s = _signs(rng, d)
    k = rng.standard_normal((L, d))
    mod = rng.integers(0, 3, L).astype(np.uint8)
    codes, lo, hi = O.quantize_keys(k, s, CB)
    y = O.randomized_hadamard(k, s)
    yh = O.dequantize_keys(codes, lo, hi, CB)
    assert O.key_grouping_error(k, mod, s, CB, "temporal") == ((y - yh) ** 2).sum() / (y ** 2).sum()


def test_block_constant_keys_have_only_rounding_error_unless_shuffled():
    rng = np.random.default_rng(5)
    d, L = 64, 32 * 20
    s = _signs(rng, d)
    k = np.repeat(rng.standard_normal((20, d)) * 3, 32, axis=0)     # one key per aligned group
    mod = np.zeros(L, np.uint8)
    # each group's range collapses (HI == LO): the only error left is the fp16
    # rounding of the statistics
    y = O.randomized_hadamard(k, s)
    r16 = y.astype(np.float16).astype(np.float64)
    assert O.key_grouping_error(k, mod, s, CB, "temporal") == ((y - r16) ** 2).sum() / (y ** 2).sum()
    assert O.key_grouping_error(k, mod, s, CB, "shuffled", seed=1) > 0.01


def test_stationary_keys_give_the_same_error_in_every_order():
    rng = np.random.default_rng(6)
    d, L = 64, 32 * 150
    s = _signs(rng, d)
    k = rng.standard_normal((L, d))
    mod = rng.integers(0, 3, L).astype(np.uint8)
    errs = [O.key_grouping_error(k, mod, s, CB, o, seed=2) for o in O.GROUP_ORDERS]
    assert max(errs) - min(errs) < 0.02 * min(errs)


@pytest.mark.parametrize("cfg_id", [0, 2])
def test_generated_hadamard_bases_equal_the_oracle_basis(cfg_id):
    """The shared-rotation baseline's value bases are an input built by the
    stream generator (Sylvester doubling); they equal the oracle's pinned
    randomized-Hadamard basis rounded once to fp32, for every KV head and
    modality, and the generator's matrix is scipy's Hadamard."""
    import scipy.linalg
    from omnistream import generate, hadamard_value_bases, sylvester_hadamard
    w = generate(cfg_id, length=64)
    d = w.cfg.head_dim
    np.testing.assert_array_equal(sylvester_hadamard(d), scipy.linalg.hadamard(d))
    R = hadamard_value_bases(w)
    assert R.shape == (w.cfg.n_kv_heads, 3, d, d) and R.dtype == np.float32
    for h in range(w.cfg.n_kv_heads):
        ref = O.hadamard_value_basis(w.signs[h]).astype(np.float32)
        for m in range(3):
            np.testing.assert_array_equal(R[h, m], ref)
