"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-type the oracle's formulas: each compares it with a library
routine, a closed form, an invariant the pages state, a special case, or a
brute force computed a different way.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import scipy.stats

from oracle import kvq_oracle as O
from omnistream import generate, lloyd_max_codebook_2bit

CB = lloyd_max_codebook_2bit()


# ---------------------------------------------------------------- Hadamard

@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128])
def test_walsh_hadamard_is_sylvester_matrix(d):
    """The butterfly transform equals scipy's Sylvester-construction matrix."""
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, size=(5, d)).astype(np.float64)
    H = scipy.linalg.hadamard(d).astype(np.float64)
    np.testing.assert_array_equal(O.walsh_hadamard(x), x @ H.T)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_randomized_hadamard_is_H_times_D(d):
    """Signs first, then H, then 1/sqrt(d): y = H D x / sqrt(d)."""
    rng = np.random.default_rng(100 + d)
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((7, d))
    M = scipy.linalg.hadamard(d) @ np.diag(s.astype(np.float64)) / math.sqrt(d)
    np.testing.assert_allclose(O.randomized_hadamard(x, s), x @ M.T, rtol=0, atol=1e-13)


@pytest.mark.parametrize("d", [64, 128])
def test_randomized_hadamard_orthonormal_and_roundtrip(d):
    rng = np.random.default_rng(200 + d)
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    M = O.randomized_hadamard(np.eye(d), s)          # rows = images of basis vectors
    np.testing.assert_allclose(M @ M.T, np.eye(d), atol=1e-15)
    x = rng.standard_normal((3, d))
    np.testing.assert_allclose(O.inverse_randomized_hadamard(O.randomized_hadamard(x, s), s), x,
                               atol=1e-14)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    assert abs(O.randomized_hadamard(q, s) @ O.randomized_hadamard(k, s) - q @ k) < 1e-12


def test_hadamard_of_bf16_data_is_exact():
    """bf16 inputs: the unnormalised transform is exact in fp64 (every partial
    sum is representable), so it equals an exact rational computation."""
    from fractions import Fraction
    from omnistream import bf16_bits_to_f64, f64_to_bf16_bits
    rng = np.random.default_rng(7)
    x = bf16_bits_to_f64(f64_to_bf16_bits(rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3, 128)))
    H = scipy.linalg.hadamard(128)
    exact = [sum(Fraction(float(x[j])) * int(H[i, j]) for j in range(128)) for i in range(128)]
    got = O.walsh_hadamard(x)
    assert all(Fraction(float(g)) == e for g, e in zip(got, exact))


# ---------------------------------------------------------------- codebook

def test_codebook_is_lloyd_max_fixed_point_for_standard_normal():
    """Each level is the conditional mean of N(0,1) over its decision cell
    (cells bounded by midpoints): the Lloyd-Max optimality conditions."""
    c = CB.astype(np.float64)
    b = np.concatenate([[-np.inf], O.decision_thresholds(CB), [np.inf]])
    phi, Phi = scipy.stats.norm.pdf, scipy.stats.norm.cdf
    means = (phi(b[:-1]) - phi(b[1:])) / (Phi(b[1:]) - Phi(b[:-1]))
    np.testing.assert_allclose(means, c, atol=1e-4)


def test_nearest_level_equals_bruteforce_argmin():
    rng = np.random.default_rng(3)
    z = rng.normal(0, 2, size=200000)
    c = CB.astype(np.float64)
    dist = np.abs(z[:, None] - c[None, :])
    srt = np.sort(dist, axis=1)
    clear = srt[:, 1] - srt[:, 0] > 1e-12
    np.testing.assert_array_equal(O.nearest_level(z, CB)[clear], np.argmin(dist, axis=1)[clear])


def test_nearest_level_ties_go_up():
    b = O.decision_thresholds(CB)
    np.testing.assert_array_equal(O.nearest_level(b, CB), [1, 2, 3])
    np.testing.assert_array_equal(O.nearest_level(np.nextafter(b, -np.inf), CB), [0, 1, 2])


def test_fp16_storage_rounds_to_nearest_even():
    """Stored statistics use numpy's direct double->half conversion; pin its
    rounding on exact midpoints and one ulp either side."""
    one_ulp = 2.0 ** -10                       # fp16 ulp in [1, 2)
    mid_even = 1.0 + one_ulp / 2               # between 1.0 (even) and 1+ulp (odd)
    mid_odd = 1.0 + 1.5 * one_ulp              # between 1+ulp (odd) and 1+2ulp (even)
    h = lambda x: float(np.float64(x).astype(np.float16))
    assert h(mid_even) == 1.0
    assert h(mid_odd) == 1.0 + 2 * one_ulp
    assert h(np.nextafter(mid_even, 2.0)) == 1.0 + one_ulp
    assert h(np.nextafter(mid_odd, 0.0)) == 1.0 + one_ulp
    # double rounding through fp32 would get this one wrong
    x = 1.0 + one_ulp / 2 + 2.0 ** -40
    assert h(x) == 1.0 + one_ulp


# ------------------------------------------------------------------- keys

def _keys(cfg_id, L):
    w = generate(cfg_id, length=L)
    k = O.as_f64(w.k[0], w.dtype)
    return w, k


@pytest.mark.parametrize("cfg_id,L", [(0, 300), (1, 400)])
def test_key_group_range_is_restored(cfg_id, L):
    """Dequantized group minimum/maximum equal the stored LO/HI exactly, and
    LO/HI are the fp16 images of the true rotated group extremes
    (OmniKVQuant key bullet: the local statistics restore the range)."""
    w, k = _keys(cfg_id, L)
    for h in range(w.cfg.n_kv_heads):
        codes, lo, hi = O.quantize_keys(k[:, h], w.signs[h], CB)
        kh = O.dequantize_keys(codes, lo, hi, CB)
        y = k[:, h] @ (scipy.linalg.hadamard(k.shape[-1]) * w.signs[h][None, :]).T / math.sqrt(k.shape[-1])
        for g in range(lo.shape[0]):
            sl = slice(32 * g, 32 * g + 32)
            LO, HI = lo[g].astype(np.float64), hi[g].astype(np.float64)
            var = HI > LO
            np.testing.assert_array_equal(kh[sl].min(0)[var], LO[var])
            np.testing.assert_array_equal(kh[sl].max(0)[var], HI[var])
            ulp = np.spacing(np.abs(y[sl]).max(0).astype(np.float16)).astype(np.float64)
            assert np.all(np.abs(LO - y[sl].min(0)) <= ulp / 2 + 1e-12)
            assert np.all(np.abs(HI - y[sl].max(0)) <= ulp / 2 + 1e-12)


@pytest.mark.parametrize("cfg_id,L", [(0, 256), (2, 512)])
def test_key_code_is_nearest_reconstruction_level(cfg_id, L):
    """In the rotated domain each key element takes the reconstruction level
    (of the four its group offers) nearest to it: brute force over levels."""
    w, k = _keys(cfg_id, L)
    c = CB.astype(np.float64)
    d = k.shape[-1]
    M = scipy.linalg.hadamard(d) / math.sqrt(d)
    for h in range(w.cfg.n_kv_heads):
        codes, lo, hi = O.quantize_keys(k[:, h], w.signs[h], CB)
        y = (k[:, h] * w.signs[h]) @ M.T
        gi = np.arange(L) // 32
        LO, HI = lo.astype(np.float64)[gi], hi.astype(np.float64)[gi]
        levels = LO[..., None] + (c - c[0])[None, None, :] * ((HI - LO) / (c[-1] - c[0]))[..., None]
        dist = np.abs(y[..., None] - levels)
        srt = np.sort(dist, axis=-1)
        clear = (srt[..., 1] - srt[..., 0] > 1e-9) & (HI > LO)
        np.testing.assert_array_equal(codes[clear], np.argmin(dist, axis=-1)[clear])
        assert clear.mean() > 0.99
        np.testing.assert_array_equal(codes[HI == LO], 0)


def test_key_single_token_and_constant_groups_give_code_zero():
    d = 64
    s = np.ones(d, np.int8)
    k = np.random.default_rng(0).standard_normal((33, d))       # last group has one token
    codes, lo, hi = O.quantize_keys(k, s, CB)
    assert lo.shape == (2, d)
    np.testing.assert_array_equal(lo[1], hi[1])
    np.testing.assert_array_equal(codes[32], 0)
    kc = np.tile(k[:1], (32, 1))                                  # all-equal group
    codes, lo, hi = O.quantize_keys(kc, s, CB)
    np.testing.assert_array_equal(codes, 0)


# ------------------------------------------------------------------ values

def _orthogonal(rng, d):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return (q * np.sign(np.diag(r))).astype(np.float32)


@pytest.mark.parametrize("d", [64, 128])
def test_value_codes_roundtrip_when_value_sits_on_levels(d):
    """v = R_m c[codes] (per-modality bases): the quantizer must recover the
    codes, which pins the rotation direction (R_m^T on the way in), the
    modality's basis, and the sqrt(d)/||v|| normalisation."""
    rng = np.random.default_rng(d)
    R = np.stack([_orthogonal(rng, d) for _ in range(3)])
    L = 90
    mod = rng.integers(0, 3, size=L).astype(np.uint8)
    c = CB.astype(np.float64)
    n_outer = round((d - d * c[2] ** 2) / (c[3] ** 2 - c[2] ** 2))    # makes ||c[codes]|| ~ sqrt(d)
    codes = np.empty((L, d), np.uint8)
    for t in range(L):
        outer = rng.permutation(d) < n_outer
        sign = rng.random(d) < 0.5
        codes[t] = np.where(outer, np.where(sign, 3, 0), np.where(sign, 2, 1))
    v = np.stack([R[mod[t]].astype(np.float64) @ c[codes[t]] for t in range(L)]) * 3.7
    got, norms = O.quantize_values(v, mod, R, CB)
    np.testing.assert_array_equal(got, codes)
    np.testing.assert_array_equal(norms, np.linalg.norm(v, axis=1).astype(np.float16))
    # the wrong basis must not round-trip
    wrong, _ = O.quantize_values(v, (mod + 1) % 3, R, CB)
    assert (wrong != codes).mean() > 0.3


def test_value_reconstruction_error_is_quantizer_error():
    """With orthogonal R_m the value error equals the rotated-domain error
    (Method: reconstructed values use their modality's rotation)."""
    w = generate(1, length=300)
    v = O.as_f64(w.v[0], w.dtype)[:, 0]
    mod = w.modality[0]
    R = w.rot[0].astype(np.float64)
    codes, norms = O.quantize_values(v, mod, w.rot[0], CB)
    vt = O.dequantize_values_rotated(codes, norms, CB)
    vhat = np.stack([R[mod[t]] @ vt[t] for t in range(len(mod))])
    r = np.stack([R[mod[t]].T @ v[t] for t in range(len(mod))])
    np.testing.assert_allclose(np.linalg.norm(vhat - v, axis=1), np.linalg.norm(vt - r, axis=1),
                               rtol=1e-5)
    z = O.value_normalized_values(v, mod, w.rot[0])
    dist = np.abs(z[..., None] - CB.astype(np.float64))
    clear = np.sort(dist, -1)[..., 1] - np.sort(dist, -1)[..., 0] > 1e-9
    np.testing.assert_array_equal(codes[clear], dist.argmin(-1)[clear])


def test_zero_value_gives_zero_codes_and_norm():
    d = 64
    R = np.stack([np.eye(d, dtype=np.float32)] * 3)
    v = np.zeros((2, d))
    v[1, 3] = 2.0
    codes, norms = O.quantize_values(v, np.array([0, 1], np.uint8), R, CB)
    np.testing.assert_array_equal(codes[0], 0)
    assert norms[0] == 0 and norms[1] == 2.0


# ------------------------------------------------------------------ decode

def _tiny_case(seed, L, d=64, hq=4, hkv=2):
    rng = np.random.default_rng(seed)
    s = np.where(rng.random((hkv, d)) < 0.5, -1, 1).astype(np.int8)
    R = np.stack([np.stack([_orthogonal(rng, d) for _ in range(3)]) for _ in range(hkv)])
    k = rng.standard_normal((L, hkv, d)) * 2 + rng.standard_normal(d)
    v = rng.standard_normal((L, hkv, d))
    mod = rng.integers(0, 3, size=L).astype(np.uint8)
    q = rng.standard_normal((hq, d))
    caches = O.quantize_session(k, v, mod, s, R, CB)
    return s, R, mod, q, caches


def _dense_bruteforce(q, s, R, mod, caches, scale, keep=None):
    """Undo every rotation explicitly (scipy Hadamard matrix, R_m matrices),
    then run textbook softmax attention on the dequantized dense cache (over
    the positions in `keep` only, when given)."""
    hq, d = q.shape
    hkv = len(caches)
    g = hq // hkv
    c = CB.astype(np.float64)
    out = np.zeros((hq, d))
    H = scipy.linalg.hadamard(d).astype(np.float64)
    for i in range(hq):
        h = i // g
        C = caches[h]
        L = C["k_codes"].shape[0]
        M = H @ np.diag(s[h].astype(np.float64)) / math.sqrt(d)      # y = M k
        gi = np.arange(L) // 32
        LO, HI = C["lo"].astype(np.float64)[gi], C["hi"].astype(np.float64)[gi]
        krot = LO + (c[C["k_codes"]] - c[0]) / (c[3] - c[0]) * (HI - LO)
        K = krot @ M                                                   # k = M^T y, row form
        V = np.stack([R[h, mod[t]].astype(np.float64) @ (C["norms"][t].astype(np.float64)
                      / math.sqrt(d) * c[C["v_codes"][t]]) for t in range(L)])
        sel = np.arange(L) if keep is None else np.flatnonzero(keep[:L])
        if sel.size == 0:
            continue
        p = scipy.special.softmax(scale * (K[sel] @ q[i]))
        out[i] = p @ V[sel]
    return out


@pytest.mark.parametrize("L", [1, 5, 37, 96])
def test_decode_equals_dense_attention_over_dequantized_cache(L):
    s, R, mod, q, caches = _tiny_case(L, L)
    scale = 1 / math.sqrt(64)
    got = O.decode_attention(O.rotate_query(q, s, 2), caches, R, CB, scale)
    ref = _dense_bruteforce(q, s, R, mod, caches, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_decode_special_cases():
    s, R, mod, q, caches = _tiny_case(11, 40)
    scale = 0.125
    c = CB.astype(np.float64)
    vhat = lambda h, t: R[h, mod[t]].astype(np.float64) @ (
        caches[h]["norms"][t].astype(np.float64) / 8.0 * c[caches[h]["v_codes"][t]])
    # q = 0: uniform attention -> the mean reconstructed value
    o = O.decode_attention(np.zeros_like(q), caches, R, CB, scale)
    for i in range(4):
        np.testing.assert_allclose(o[i], np.mean([vhat(i // 2, t) for t in range(40)], 0), atol=1e-13)
    # one cached position -> that value, whatever the query
    one = [{k: (v[:1] if k != "lo" and k != "hi" else v[:1]) for k, v in C.items()} for C in caches]
    for C in one:
        C["modality"] = mod[:1]
    o = O.decode_attention(O.rotate_query(q, s, 2), one, R, CB, scale)
    for i in range(4):
        np.testing.assert_allclose(o[i], vhat(i // 2, 0), atol=1e-14)
    # empty context -> zeros
    empty = [{k: v[:0] for k, v in C.items()} for C in caches]
    np.testing.assert_array_equal(O.decode_attention(q, empty, R, CB, scale), 0)


def test_decode_single_modality_uses_only_that_basis():
    s, R, mod, q, caches = _tiny_case(5, 64)
    for C in caches:
        C["modality"] = np.full(64, 1, np.uint8)
    R2 = R.copy()
    R2[:, 0] = 0.0
    R2[:, 2] = 0.0
    a = O.decode_attention(O.rotate_query(q, s, 2), caches, R, CB, 0.125)
    b = O.decode_attention(O.rotate_query(q, s, 2), caches, R2, CB, 0.125)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("pattern", ["pages", "random"])
def test_decode_over_a_retained_position_set(pattern):
    """A sparse page set: the masked decode equals textbook attention over the
    retained positions alone; keeping everything changes nothing; keeping
    nothing gives zeros."""
    L = 160
    s, R, mod, q, caches = _tiny_case(7, L)
    scale = 1 / math.sqrt(64)
    rng = np.random.default_rng(11)
    if pattern == "pages":       # whole 32-position blocks kept or dropped
        keep = np.repeat(rng.random(L // 32) < 0.5, 32)
        keep[:32] = True
    else:
        keep = rng.random(L) < 0.3
    qr = O.rotate_query(q, s, 2)
    got = O.decode_attention(qr, caches, R, CB, scale, retained=keep)
    ref = _dense_bruteforce(q, s, R, mod, caches, scale, keep)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))
    np.testing.assert_array_equal(O.decode_attention(qr, caches, R, CB, scale, retained=np.ones(L, bool)),
                                  O.decode_attention(qr, caches, R, CB, scale))
    np.testing.assert_array_equal(O.decode_attention(qr, caches, R, CB, scale, retained=np.zeros(L, bool)), 0)


# ------------------------------------------- input conversion, value bases

def test_bf16_to_f64_on_every_bit_pattern():
    """All 65,536 bfloat16 bit patterns: the oracle's fp64 image equals torch's
    bfloat16 -> float32 conversion (NaNs compared by class, zeros by sign),
    and a few patterns worked by hand from the format (sign, 8-bit exponent
    with bias 127, 7-bit fraction) come out exactly."""
    import torch
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(bits)
    with np.errstate(invalid="ignore"):
        ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127                       # exponent all ones, fraction nonzero, both signs
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    hand = {0x3F80: 1.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
            0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: np.inf, 0xFF80: -np.inf, 0x8000: -0.0,
            0x3E80: 0.25, 0x4049: 3.140625}
    for b, v in hand.items():
        g = O.bf16_to_f64(np.array([b], np.uint16))[0]
        assert g == v and np.signbit(g) == np.signbit(v), (hex(b), g, v)


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_generated_value_bases_are_orthogonal(cfg_id):
    """Every generated fp32 value basis R_{h,m} is orthogonal to 1e-6: the
    oracle inverts the forward map R_m^T with R_m (Sec. 2, values bullet: the
    reconstructed values use the modality's rotation), which needs
    R_m^T R_m = R_m R_m^T = I.  The bases depend only on the configuration's
    seed, so a short stream gives the full configuration's bases."""
    w = generate(cfg_id, length=64, batch=1, len_range=(64, 64) if cfg_id == 3 else None)
    hkv, d = w.cfg.n_kv_heads, w.cfg.head_dim
    assert w.rot.shape == (hkv, 3, d, d) and w.rot.dtype == np.float32
    I = np.eye(d)
    for h in range(hkv):
        for m in range(3):
            R = w.rot[h, m].astype(np.float64)
            assert np.abs(R.T @ R - I).max() < 1e-6, (h, m)
            assert np.abs(R @ R.T - I).max() < 1e-6, (h, m)
    # the three modalities of a head have different bases (per-modality rotation)
    for h in range(hkv):
        assert np.abs(w.rot[h, 0] - w.rot[h, 1]).max() > 0.1 and np.abs(w.rot[h, 1] - w.rot[h, 2]).max() > 0.1


# ------------------------------------- the z each key code is decided on

@pytest.mark.parametrize("cfg_id,L", [(0, 289), (1, 333), (2, 97)])
def test_key_normalized_values_decide_the_codes(cfg_id, L):
    """key_normalized_values reports the z each key code is decided on:
    nearest_level(z) reproduces quantize_keys' codes wherever z is defined,
    z is NaN exactly where the stored range is empty (HI == LO: here the
    single-position last group), and z stays inside [c0, c3] up to the fp16
    rounding of LO / HI (Sec. 2 Method, key bullet)."""
    w, k = _keys(cfg_id, L)
    c = CB.astype(np.float64)
    gi = np.arange(L) // 32
    for h in range(w.cfg.n_kv_heads):
        codes, lo, hi = O.quantize_keys(k[:, h], w.signs[h], CB)
        z = O.key_normalized_values(k[:, h], w.signs[h], lo, hi, CB)
        empty = (lo.astype(np.float64) == hi.astype(np.float64))[gi]
        if L % 32 == 1:
            assert empty[-1].all()
        np.testing.assert_array_equal(np.isnan(z), empty)
        np.testing.assert_array_equal(O.nearest_level(z[~empty], CB), codes[~empty])
        # y lies in [true min, true max]; LO / HI are those within half an fp16 ulp
        LO, HI = lo.astype(np.float64)[gi], hi.astype(np.float64)[gi]
        ulp = np.spacing(np.maximum(np.abs(LO), np.abs(HI)).astype(np.float16)).astype(np.float64)
        slack = (c[-1] - c[0]) * ulp / np.where(empty, 1.0, HI - LO)
        ok = ~empty
        assert np.all(z[ok] >= c[0] - slack[ok] - 1e-12) and np.all(z[ok] <= c[-1] + slack[ok] + 1e-12)


def test_key_normalized_values_on_a_hand_worked_group():
    """Rotated keys placed at known fractions f of an fp16-exact group range:
    the position at the group minimum has z = c0, the maximum z = c3, and
    fraction f gives z = c0 + f (c3 - c0), so the quarter points of the range
    fall on the levels' affine images (the range maps onto [c0, c3])."""
    d = 64
    rng = np.random.default_rng(21)
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    LO = np.round(rng.uniform(-4, 0, d) * 8) / 8                 # fp16-exact
    HI = LO + np.round(rng.uniform(0.5, 6, d) * 8) / 8
    fr = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 0.125, 0.375, 0.625])
    f = fr[np.arange(32)[:, None] % 8 + 0 * np.arange(d)[None, :]]
    f[0], f[1] = 0.0, 1.0                                         # both extremes present in every channel
    y = LO + f * (HI - LO)                                        # exact in fp64
    M = scipy.linalg.hadamard(d) @ np.diag(s.astype(np.float64)) / math.sqrt(d)
    k = y @ M                                                     # M^T y: the key whose rotation is y
    codes, lo, hi = O.quantize_keys(k, s, CB)
    np.testing.assert_array_equal(lo[0].astype(np.float64), LO)
    np.testing.assert_array_equal(hi[0].astype(np.float64), HI)
    z = O.key_normalized_values(k, s, lo, hi, CB)
    c = CB.astype(np.float64)
    np.testing.assert_allclose(z, c[0] + f * (c[-1] - c[0]), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(codes[f == 0.0], 0)
    np.testing.assert_array_equal(codes[f == 1.0], 3)
