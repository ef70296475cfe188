"""Pins of the value-basis calibration oracle (CPU only).

Each test checks the oracle against something other than itself: closed
forms (two-token softmax, 2 x 2 eigenproblem, a covariance built to be
exactly Q diag(lam) Q^T), invariants (weights sum to one, shift and scale
invariance, a doubled weight equals a duplicated token), special cases that
reduce to a library routine (uniform weights give numpy's population
covariance), and the Lloyd-Max distortion of a Gaussian source for the
error harness.
"""
import math

import numpy as np
import pytest

from oracle import kvq_calib_oracle as C
from oracle import kvq_oracle as O
from omnistream import calibration_queries, generate


# ------------------------------------------------------------ contribution

def test_zero_queries_give_uniform_weights():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((37, 2, 16))
    q = np.zeros((3, 4, 16))
    w = C.contribution_weights(k, q, 0.25)
    assert w.shape == (2, 37)
    np.testing.assert_allclose(w, 1.0 / 37, rtol=0, atol=1e-16)


def test_two_tokens_follow_the_logistic_function():
    # softmax over two tokens is the logistic function of the score difference
    rng = np.random.default_rng(1)
    d = 8
    k = rng.standard_normal((2, 1, d))
    q = rng.standard_normal((5, 3, d))
    scale = 0.3
    w = C.contribution_weights(k, q, scale)[0]
    rows = q.reshape(15, d)
    ds = scale * (rows @ (k[1, 0] - k[0, 0]))
    expect1 = np.mean([1.0 / (1.0 + math.exp(-x)) for x in ds])
    assert abs(w[1] - expect1) < 1e-15
    assert abs(w[0] - (1.0 - expect1)) < 1e-15


def test_weights_of_each_head_sum_to_one_and_follow_permutation():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((50, 2, 32)) * 2
    q = rng.standard_normal((4, 6, 32))
    w = C.contribution_weights(k, q, 1 / math.sqrt(32))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    perm = rng.permutation(50)
    w2 = C.contribution_weights(k[perm], q, 1 / math.sqrt(32))
    np.testing.assert_allclose(w2, w[:, perm], rtol=1e-13, atol=0)


def test_query_heads_map_to_kv_head_floor_i_over_g():
    # zeroing the queries of KV head 1's group (heads 3..5 of 6, G = 3) makes
    # only KV head 1's weights uniform
    rng = np.random.default_rng(3)
    k = rng.standard_normal((20, 2, 16)) * 3
    q = rng.standard_normal((2, 6, 16))
    q[:, 3:6] = 0
    w = C.contribution_weights(k, q, 0.5)
    np.testing.assert_allclose(w[1], 1 / 20, atol=1e-16)
    assert np.abs(w[0] - 1 / 20).max() > 1e-3


def test_dominant_token_takes_all_weight():
    d = 16
    k = np.zeros((10, 1, d))
    k[4, 0, 0] = 100.0
    q = np.zeros((2, 1, d))
    q[:, 0, 0] = 1.0
    w = C.contribution_weights(k, q, 1.0)[0]
    others = np.delete(w, 4)
    assert w[4] > 1 - 1e-15 and others.max() < 1e-40 and others.max() > 0


# -------------------------------------------------------------- covariance

def _exact_stream(rng, n, Q, lam, mean):
    """n tokens whose centred, uniform-weight covariance is exactly
    Q diag(lam) Q^T: orthonormal score columns orthogonal to the all-ones
    vector, scaled so that sum_t x_t x_t^T / n = Q diag(lam) Q^T."""
    d = Q.shape[0]
    a = rng.standard_normal((n, d + 1))
    a[:, 0] = 1.0
    basis, _ = np.linalg.qr(a)
    xi = basis[:, 1:] * math.sqrt(n)                   # xi^T xi = n I, 1^T xi = 0
    return mean[None, :] + (xi * np.sqrt(lam)[None, :]) @ Q.T


def test_uniform_weights_give_population_covariance():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((300, 24)) * rng.uniform(0.1, 3, 24) + 0.7
    mod = np.zeros(300, np.uint8)
    w = np.full(300, 1 / 300)
    Cm, W, mu = C.weighted_covariance(v, mod, w)
    np.testing.assert_allclose(Cm[0], np.cov(v.T, bias=True), rtol=0, atol=1e-13)
    np.testing.assert_allclose(mu[0], v.mean(axis=0), rtol=0, atol=1e-14)
    assert abs(W[0] - 1.0) < 1e-14
    assert not Cm[1].any() and not Cm[2].any() and W[1] == 0 and W[2] == 0


def test_covariance_recovers_constructed_matrix():
    rng = np.random.default_rng(5)
    d = 16
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.linspace(5.0, 0.1, d)
    v = _exact_stream(rng, 200, Q, lam, rng.standard_normal(d) * 4)
    Cm, _, _ = C.weighted_covariance(v, np.zeros(200, np.uint8), np.full(200, 0.37))
    np.testing.assert_allclose(Cm[0], (Q * lam) @ Q.T, rtol=0, atol=1e-12)


def test_doubled_weight_equals_duplicated_token_and_scale_invariance():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((40, 8))
    mod = np.zeros(40, np.uint8)
    w = rng.uniform(0.1, 1.0, 40)
    w2 = w.copy()
    w2[7] *= 2
    C2, _, _ = C.weighted_covariance(v, mod, w2)
    vd = np.vstack([v, v[7:8]])
    Cd, _, _ = C.weighted_covariance(vd, np.zeros(41, np.uint8), np.append(w, w[7]))
    np.testing.assert_allclose(C2[0], Cd[0], rtol=0, atol=1e-14)
    C5, _, _ = C.weighted_covariance(v, mod, w * 5.0)
    C1, _, _ = C.weighted_covariance(v, mod, w)
    np.testing.assert_allclose(C5[0], C1[0], rtol=0, atol=1e-14)


def test_covariance_is_shift_invariant_and_per_modality():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((90, 8))
    mod = np.repeat(np.array([0, 1, 2], np.uint8), 30)
    w = rng.uniform(0.1, 1.0, 90)
    C0, W0, _ = C.weighted_covariance(v, mod, w)
    v2 = v.copy()
    v2[mod == 1] += 10.0                        # shift one modality only
    v2[mod == 2] *= 3.0                         # scale another
    C1, W1, _ = C.weighted_covariance(v2, mod, w)
    np.testing.assert_allclose(C1[0], C0[0], atol=1e-13)
    np.testing.assert_allclose(C1[1], C0[1], atol=1e-12)
    np.testing.assert_allclose(C1[2], 9.0 * C0[2], atol=1e-12)
    np.testing.assert_allclose(W1, W0, atol=0)
    # a modality byte outside 0..2 takes no part
    mod3 = mod.copy()
    mod3[:5] = 3
    C3, W3, _ = C.weighted_covariance(v, mod3, w)
    Cr, Wr, _ = C.weighted_covariance(v[5:], mod[5:], w[5:])
    np.testing.assert_allclose(C3, Cr, atol=1e-14)
    np.testing.assert_allclose(W3, Wr, atol=1e-15)


# --------------------------------------------------------------- eigenbasis

def test_eigenbasis_of_diagonal_is_sorted_permutation():
    lam = np.array([0.5, 3.0, -1.0, 2.0])
    R, l = C.eigenbasis(np.diag(lam))
    np.testing.assert_array_equal(l, [3.0, 2.0, 0.5, -1.0])
    np.testing.assert_array_equal(R, np.eye(4)[:, [1, 3, 0, 2]])


def test_eigenbasis_two_by_two_closed_form():
    a, b, c = 2.0, -0.75, 0.5
    R, l = C.eigenbasis(np.array([[a, b], [b, c]]))
    r = math.sqrt(((a - c) / 2) ** 2 + b * b)
    np.testing.assert_allclose(l, [(a + c) / 2 + r, (a + c) / 2 - r], rtol=0, atol=1e-15)
    # the top eigenvector solves (a - l1) x + b y = 0
    x, y = R[:, 0]
    assert abs((a - l[0]) * x + b * y) < 1e-15 and abs(math.hypot(x, y) - 1) < 1e-15
    assert abs(x) >= abs(y) and x > 0


def test_eigenbasis_recovers_known_basis_with_sign_rule():
    rng = np.random.default_rng(8)
    d = 32
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = np.sort(rng.uniform(0.1, 10, d))[::-1] + np.arange(d)[::-1] * 0.05
    R, l = C.eigenbasis((Q * lam) @ Q.T)
    np.testing.assert_allclose(l, lam, rtol=0, atol=1e-12)
    for j in range(d):
        i = int(np.argmax(np.abs(Q[:, j])))
        qj = Q[:, j] * np.sign(Q[i, j])
        np.testing.assert_allclose(R[:, j], qj, rtol=0, atol=1e-10)
    np.testing.assert_allclose(R.T @ R, np.eye(d), atol=1e-13)


def test_eigenbasis_of_zero_is_identity():
    R, l = C.eigenbasis(np.zeros((8, 8)))
    np.testing.assert_array_equal(R, np.eye(8))
    np.testing.assert_array_equal(l, 0)


# ----------------------------------------------------------------- pipeline

def test_calibration_recovers_each_modality_basis_exactly():
    # uniform contribution (zero queries) over streams built to have exactly
    # Q_m diag(lam_m) Q_m^T as each modality's covariance
    rng = np.random.default_rng(9)
    d, n_per = 16, 64
    Qs = [np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(3)]
    lams = [np.sort(rng.uniform(0.2, 6, d))[::-1] + np.arange(d)[::-1] * 0.1 for _ in range(3)]
    v = np.concatenate([_exact_stream(rng, n_per, Qs[m], lams[m], rng.standard_normal(d)) for m in range(3)])
    mod = np.repeat(np.arange(3, dtype=np.uint8), n_per)
    order = rng.permutation(3 * n_per)            # interleave the modalities
    v, mod = v[order], mod[order]
    k = rng.standard_normal((3 * n_per, 1, d))
    q = np.zeros((2, 2, d))
    rot, lam, w, _ = C.calibrate_value_bases(k, v[:, None, :], mod, q, 0.25)
    for m in range(3):
        np.testing.assert_allclose(lam[0, m], lams[m], rtol=0, atol=1e-11)
        for j in range(d):
            i = int(np.argmax(np.abs(Qs[m][:, j])))
            np.testing.assert_allclose(rot[0, m][:, j], Qs[m][:, j] * np.sign(Qs[m][i, j]), rtol=0, atol=1e-6)


def test_calibration_on_generator_stream_finds_its_spectrum():
    # the generator draws v ~ N(0, Q_m diag(lam_m) Q_m^T) independently of the
    # keys, so the weighted covariance estimates Q_m diag(lam_m) Q_m^T: the
    # true covariance's Rayleigh quotient along each calibrated direction
    # tracks the sorted true spectrum (video: ~1,570 tokens at d = 64)
    w = generate(0)
    k = O.as_f64(w.k[0], w.dtype)
    v = O.as_f64(w.v[0], w.dtype)
    q = O.as_f64(calibration_queries(w, 8), w.dtype)
    rot, lam, _, _ = C.calibrate_value_bases(k, v, w.modality[0], q, 1 / math.sqrt(64))
    spec = w.meta["value_spectrum"][0, 0]
    true_c = (w.rot[0, 0].astype(np.float64) * spec) @ w.rot[0, 0].astype(np.float64).T
    R = rot[0, 0].astype(np.float64)
    rq = np.einsum("ij,ik,kj->j", R, true_c, R)
    srt = np.sort(spec)[::-1]
    assert abs(rq[0] - srt[0]) < 0.15 * srt[0]
    assert np.abs(rq - srt).max() < 0.25 * srt[0]
    # and the estimated eigenvalues are those of the estimate, in order
    assert np.all(np.diff(lam[0, 0]) <= 0)


# ------------------------------------------------------------- error harness

def _sphere_marginal_distortion(d, cb):
    """E[(z - c(z))^2] for z = sqrt(d) t, t one coordinate of a uniform point
    on the unit sphere in R^d (density proportional to (1 - t^2)^((d - 3) / 2)),
    c the nearest of the levels cb: the codec's per-coordinate distortion for
    isotropic values, whose normalised coordinates follow exactly this law.
    Tends to the Gaussian Lloyd-Max distortion 0.1175 as d grows."""
    from scipy import integrate, special
    c = np.asarray(cb, np.float64)
    b = (c[:-1] + c[1:]) / 2
    lognorm = special.gammaln(d / 2) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2)
    f = lambda t: math.exp(lognorm + (d - 3) / 2 * math.log1p(-t * t))
    edges = [-1.0] + list(b / math.sqrt(d)) + [1.0]
    tot = 0.0
    for k in range(len(c)):
        val, _ = integrate.quad(lambda t: (math.sqrt(d) * t - c[k]) ** 2 * f(t), edges[k], edges[k + 1],
                                epsabs=1e-13, epsrel=1e-12)
        tot += val
    return tot


def test_error_harness_matches_the_quantizer_distortion():
    # isotropic Gaussian values: the normalised coordinates in any orthonormal
    # basis follow the sphere marginal, so the relative error is that law's
    # 4-level distortion (0.1127 at d = 64, 0.1151 at d = 128)
    cb = (-1.5104, -0.4528, 0.4528, 1.5104)
    assert abs(_sphere_marginal_distortion(100000, cb) - 0.1175) < 2e-4   # Gaussian limit
    rng = np.random.default_rng(10)
    for d, n in ((64, 4000), (128, 2000)):
        v = rng.standard_normal((n, d))
        signs = np.where(rng.random(d) < 0.5, -1.0, 1.0)
        H = O.hadamard_value_basis(signs)                  # r = v @ H = H_d (s * v) / sqrt(d)
        R = np.linalg.qr(rng.standard_normal((d, d)))[0]
        rot = np.stack([H, R, H]).astype(np.float32)
        mod = np.repeat(np.array([0, 1], np.uint8), [n // 2, n - n // 2])
        err = C.value_quantization_error(v, mod, rot, cb)
        expect = _sphere_marginal_distortion(d, cb)
        assert abs(err[0] - expect) < 0.002 and abs(err[1] - expect) < 0.002, (d, err, expect)
        assert np.isnan(err[2])


def test_error_harness_is_invariant_under_a_common_rotation():
    # rotating every value by P and every basis to P R leaves the codes, and
    # so the relative error, unchanged (a transposed basis anywhere breaks it)
    rng = np.random.default_rng(11)
    d, n = 32, 600
    v = rng.standard_normal((n, d)) * rng.uniform(0.3, 2.0, d)
    mod = rng.integers(0, 3, n).astype(np.uint8)
    R = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(3)])
    P = np.linalg.qr(rng.standard_normal((d, d)))[0]
    cb = (-1.5104, -0.4528, 0.4528, 1.5104)
    R32 = R.astype(np.float32).astype(np.float64)
    e1 = C.value_quantization_error(v, mod, R32.astype(np.float32), cb)
    PR = np.einsum("ij,mjk->mik", P, R32)
    e2 = C.value_quantization_error(v @ P.T, mod, PR, cb)
    assert np.all(e1 > 0.05) and np.all(e1 < 0.6)
    np.testing.assert_allclose(e1, e2, rtol=1e-3)
