"""Pins of the 3- and 4-bit fixed codebooks and of the oracle's codecs at
those widths (CPU only).

The codebooks are pinned to J. Max's published table of optimum Gaussian
quantizers (tests/golden/lloyd_max_gaussian.txt, four significant figures)
and to the Lloyd-Max conditions themselves; the oracle's key codec, value
codec and decode, written for any number of levels, are pinned at 8 and 16
levels against brute force, the range-restoring property and the exact
distortion of the quantizer.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import scipy.stats
from scipy import integrate

from omnistream import lloyd_max_codebook
from oracle import kvq_oracle as O
from tests.test_calib_pins import _sphere_marginal_distortion

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lloyd_max_gaussian.txt")


def _golden():
    table = {}
    for line in open(GOLDEN):
        if not line.strip() or line.startswith("#"):
            continue
        n, kind, *vals = line.split()
        table[(int(n), kind)] = [float(v) for v in vals]
    return table


def _distortion(c):
    c = np.asarray(c, np.float64)
    b = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
    return sum(integrate.quad(lambda x, k=k: (x - c[k]) ** 2 * scipy.stats.norm.pdf(x), b[k], b[k + 1],
                              epsabs=1e-14)[0] for k in range(len(c)))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_matches_max_table(bits):
    n = 1 << bits
    t = _golden()
    c = lloyd_max_codebook(bits).astype(np.float64)
    assert c.shape == (n,) and np.all(np.diff(c) > 0)
    np.testing.assert_allclose(c, -c[::-1], atol=0)                       # symmetric
    np.testing.assert_allclose(c[n // 2:], t[(n, "outputs")], atol=1e-3)
    np.testing.assert_allclose(O.decision_thresholds(c.astype(np.float32))[n // 2:], t[(n, "thresholds")], atol=1e-3)
    np.testing.assert_allclose(_distortion(c), t[(n, "distortion")][0], rtol=1e-3)


@pytest.mark.parametrize("bits", [3, 4])
def test_codebook_is_lloyd_max_fixed_point(bits):
    c = lloyd_max_codebook(bits)
    b = np.concatenate([[-np.inf], O.decision_thresholds(c), [np.inf]])
    phi, Phi = scipy.stats.norm.pdf, scipy.stats.norm.cdf
    means = (phi(b[:-1]) - phi(b[1:])) / (Phi(b[1:]) - Phi(b[:-1]))
    np.testing.assert_allclose(means, c.astype(np.float64), atol=2e-6)


@pytest.mark.parametrize("bits", [3, 4])
def test_key_codec_restores_range_and_takes_nearest_level(bits):
    cb = lloyd_max_codebook(bits)
    c = cb.astype(np.float64)
    rng = np.random.default_rng(bits)
    d, L = 64, 200
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    k = rng.standard_normal((L, d)) * 3 + rng.standard_normal(d)
    codes, lo, hi = O.quantize_keys(k, s, cb)
    assert codes.max() == len(c) - 1
    kh = O.dequantize_keys(codes, lo, hi, cb)
    y = k @ (scipy.linalg.hadamard(d) * s[None, :]).T / math.sqrt(d)
    gi = np.arange(L) // 32
    LO, HI = lo.astype(np.float64)[gi], hi.astype(np.float64)[gi]
    for g in range(lo.shape[0]):
        sl = slice(32 * g, 32 * g + 32)
        np.testing.assert_array_equal(kh[sl].min(0), lo[g].astype(np.float64))
        np.testing.assert_array_equal(kh[sl].max(0), hi[g].astype(np.float64))
    levels = LO[..., None] + (c - c[0])[None, None, :] * ((HI - LO) / (c[-1] - c[0]))[..., None]
    dist = np.abs(y[..., None] - levels)
    srt = np.sort(dist, axis=-1)
    clear = srt[..., 1] - srt[..., 0] > 1e-9
    np.testing.assert_array_equal(codes[clear], np.argmin(dist, axis=-1)[clear])


@pytest.mark.parametrize("bits", [3, 4])
def test_value_codec_reaches_the_quantizer_distortion(bits):
    cb = lloyd_max_codebook(bits)
    rng = np.random.default_rng(10 + bits)
    d, n = 128, 2000
    v = rng.standard_normal((n, d))
    R = np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(3)]).astype(np.float32)
    mod = np.zeros(n, np.uint8)
    codes, norms = O.quantize_values(v, mod, R, cb)
    vh = O.dequantize_values_rotated(codes, norms, cb) @ R[0].astype(np.float64).T
    err = ((v - vh) ** 2).sum() / (v ** 2).sum()
    expect = _sphere_marginal_distortion(d, tuple(cb.astype(np.float64)))
    assert abs(err - expect) < 0.03 * expect


@pytest.mark.parametrize("bits", [3, 4])
def test_decode_equals_dense_attention_at_more_bits(bits):
    cb = lloyd_max_codebook(bits)
    c = cb.astype(np.float64)
    rng = np.random.default_rng(20 + bits)
    d, L, hq, hkv = 64, 70, 4, 2
    s = np.where(rng.random((hkv, d)) < 0.5, -1, 1).astype(np.int8)
    R = np.stack([np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(3)])
                  for _ in range(hkv)]).astype(np.float32)
    k = rng.standard_normal((L, hkv, d)) * 2
    v = rng.standard_normal((L, hkv, d))
    mod = rng.integers(0, 3, L).astype(np.uint8)
    q = rng.standard_normal((hq, d))
    caches = O.quantize_session(k, v, mod, s, R, cb)
    scale = 1 / math.sqrt(d)
    got = O.decode_attention(O.rotate_query(q, s, hkv), caches, R, cb, scale)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    for i in range(hq):
        h = i // (hq // hkv)
        C = caches[h]
        M = H @ np.diag(s[h].astype(np.float64)) / math.sqrt(d)
        gi = np.arange(L) // 32
        LO, HI = C["lo"].astype(np.float64)[gi], C["hi"].astype(np.float64)[gi]
        K = (LO + (c[C["k_codes"]] - c[0]) / (c[-1] - c[0]) * (HI - LO)) @ M
        V = np.stack([R[h, mod[t]].astype(np.float64) @ (C["norms"][t].astype(np.float64) / math.sqrt(d)
                      * c[C["v_codes"][t]]) for t in range(L)])
        p = scipy.special.softmax(scale * (K @ q[i]))
        np.testing.assert_allclose(got[i], p @ V, rtol=0, atol=1e-12)
