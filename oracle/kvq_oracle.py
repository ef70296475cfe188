"""fp64 CPU oracle for rotation-based 2-bit KV-cache quantization with fused
decode attention (the OmniKVQuant method).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The library's product path never calls
it, and it shares no code, constant or helper with the HIP path.

Sources (the OmniKVQuant page, paperlayer.ai summary of arXiv 2609.11582):
  * Sec. 2 Method, "TurboQuant" bullet: rotate toward Gaussian-like
    coordinates with a randomized Hadamard transform, separate magnitude from
    direction, quantize rotated coordinates with a fixed codebook, reconstruct.
  * Sec. 2 Method, first "OmniKVQuant" bullet: min-max scale rotated keys in
    short consecutive-token groups, store the group statistics, apply the
    shared fixed codebook; the statistics restore the range on reconstruction;
    the Hadamard basis is kept.
  * Sec. 2 Method, second "OmniKVQuant" bullet: a value rotation per modality;
    reconstructed values use their modality's rotation.
  * Sec. 1 Introduction, "Implementation" bullet: decode unpacks the 2-bit
    cache inside attention, rotates one query per head, and applies the inverse
    value rotations once, after aggregation.

Everything is float64.  Inputs are exact float64 images of the fp32/bf16
data.  Stored statistics (key min/max, value norms) are rounded once to fp16
with round-to-nearest-even (numpy's direct double->half conversion).

Readings where the pages are silent (each repeated in the design notes):
  * Hadamard: Sylvester natural order, signs applied first,
    y = (1/sqrt(d)) * H_d (s * x); the 1/sqrt(d) is one fp64 multiply after
    the unnormalised transform.
  * Key statistics are per (32-token group, rotated channel): lo/hi = min/max
    over the group's present tokens, stored as fp16.
  * The group range [LO, HI] maps affinely onto [c0, c3]; a value's code is
    the number of decision thresholds (midpoints of adjacent levels) it
    reaches (ties go up); HI == LO gives code 0.
  * Values: n = ||v||, r = R_m^T v, z = sqrt(d) * r / n, nearest level; the
    stored norm is fp16(n); reconstruction is R_m (N / sqrt(d)) c[code].
  * Query head i uses KV head floor(i / G); scores use scale 1/sqrt(d) unless
    given; an empty context attends to nothing and yields zeros.
  * Sparse page sets (a retained-page list or mask; OmniTide page, Sec. 6
    OmniPage: an emptied page is skipped whole): positions outside the
    retained set are left out before the softmax, exactly as if they had
    never been cached.
  * TurboQuant baseline (Sec. 2 Method, TurboQuant bullet; Sec. 1 Problem
    bullet: one fixed scale per token rather than local ranges): a key is
    coded like a value, with the randomized Hadamard as its rotation:
    n = ||k||, z = sqrt(d) H_d (s * k) / sqrt(d) / n, nearest level, fp16(n);
    values use the same randomized Hadamard for every modality.
  * Key-grouping harness (Sec. 3, "Key Adaptation" bullet): the 32-token
    min-max groups are formed over the stream taken in a given order
    (temporal; modality-only, i.e. sorted by modality keeping time order;
    shuffled within each modality; shuffled globally), and the relative
    squared error of the reconstructed rotated keys is reported.
"""
from __future__ import annotations

import numpy as np

GROUP_TOKENS = 32
N_MODALITIES = 3


# ------------------------------------------------------------------ inputs

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 data given as raw uint16 bits."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ------------------------------------------------------- Hadamard rotation

def walsh_hadamard(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis (Sylvester
    natural order: H_1 = [1], H_2n = [[H, H], [H, -H]]), by butterflies."""
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    if d & (d - 1):
        raise ValueError("head dimension must be a power of two")
    lead = x.shape[:-1]
    h = 1
    while h < d:
        y = x.reshape(lead + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        x = y.reshape(lead + (d,))
        h *= 2
    return x


def randomized_hadamard(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = (1/sqrt(d)) H_d (s * x) over the last axis: the randomized Hadamard
    rotation (Method, TurboQuant bullet; kept for keys by OmniKVQuant)."""
    d = x.shape[-1]
    return walsh_hadamard(np.asarray(x, np.float64) * np.asarray(signs, np.float64)) * (1.0 / np.sqrt(d))


def inverse_randomized_hadamard(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x = s * (1/sqrt(d)) H_d y (H_d is symmetric and H_d H_d = d I)."""
    d = y.shape[-1]
    return walsh_hadamard(y) * (1.0 / np.sqrt(d)) * np.asarray(signs, np.float64)


# ------------------------------------------------------------------ codebook

def decision_thresholds(codebook: np.ndarray) -> np.ndarray:
    """Midpoints between adjacent levels, in fp64 from the fp32 levels."""
    c = np.asarray(codebook, dtype=np.float32).astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


def nearest_level(z: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Index of the nearest codebook level: the number of thresholds z reaches
    (a value exactly on a threshold takes the upper level)."""
    b = decision_thresholds(codebook)
    return (np.asarray(z)[..., None] >= b).sum(axis=-1).astype(np.uint8)


# ------------------------------------------------------------------- keys

def quantize_keys(k: np.ndarray, signs: np.ndarray, codebook: np.ndarray,
                  group: int = GROUP_TOKENS):
    """Quantize one KV head's keys.

    k: [L, d] float64 raw keys.  Returns codes [L, d] uint8, lo/hi
    [ceil(L/group), d] float16 (the stored group statistics).
    Method, OmniKVQuant key bullet: rotate, min-max scale within short
    consecutive-token groups, store the statistics, apply the fixed codebook.
    """
    y = randomized_hadamard(k, signs)
    L, d = y.shape
    ng = -(-L // group)
    c = np.asarray(codebook, np.float32).astype(np.float64)
    c0, c3 = c[0], c[-1]
    codes = np.zeros((L, d), np.uint8)
    lo16 = np.zeros((ng, d), np.float16)
    hi16 = np.zeros((ng, d), np.float16)
    for g in range(ng):
        yg = y[g * group:(g + 1) * group]
        lo16[g] = yg.min(axis=0).astype(np.float16)
        hi16[g] = yg.max(axis=0).astype(np.float16)
        LO = lo16[g].astype(np.float64)
        HI = hi16[g].astype(np.float64)
        span = HI - LO
        ok = span > 0
        z = np.zeros_like(yg)
        z[:, ok] = c0 + (yg[:, ok] - LO[ok]) * (c3 - c0) / span[ok]
        cg = nearest_level(z, codebook)
        cg[:, ~ok] = 0
        codes[g * group:(g + 1) * group] = cg
    return codes, lo16, hi16


def key_normalized_values(k: np.ndarray, signs: np.ndarray, lo16: np.ndarray,
                          hi16: np.ndarray, codebook: np.ndarray,
                          group: int = GROUP_TOKENS) -> np.ndarray:
    """The fp64 value z each key element's code is decided on (NaN where the
    group range is empty).  Used to find elements near a decision threshold."""
    y = randomized_hadamard(k, signs)
    c = np.asarray(codebook, np.float32).astype(np.float64)
    c0, c3 = c[0], c[-1]
    gi = np.arange(y.shape[0]) // group
    LO = lo16.astype(np.float64)[gi]
    HI = hi16.astype(np.float64)[gi]
    span = HI - LO
    with np.errstate(divide="ignore", invalid="ignore"):
        z = c0 + (y - LO) * (c3 - c0) / span
    z[span == 0] = np.nan
    return z


def dequantize_keys(codes: np.ndarray, lo16: np.ndarray, hi16: np.ndarray,
                    codebook: np.ndarray, group: int = GROUP_TOKENS) -> np.ndarray:
    """Rotated-domain key reconstruction k_hat = LO + (c[code]-c0)(HI-LO)/(c3-c0):
    code 0 gives LO and code 3 gives HI, restoring the group's range."""
    c = np.asarray(codebook, np.float32).astype(np.float64)
    gi = np.arange(codes.shape[0]) // group
    LO = lo16.astype(np.float64)[gi]
    HI = hi16.astype(np.float64)[gi]
    return LO + (c[codes] - c[0]) * (HI - LO) / (c[-1] - c[0])


# ------------------------------------------------------------------ values

def quantize_values(v: np.ndarray, modality: np.ndarray, rot: np.ndarray,
                    codebook: np.ndarray):
    """Quantize one KV head's values with per-modality rotations.

    v: [L, d] float64; modality: [L] in {0,1,2}; rot: [3, d, d] (R_m, columns
    form the basis).  Returns codes [L, d] uint8 and norms [L] float16.
    Method, TurboQuant bullet (magnitude/direction split, fixed codebook on
    rotated coordinates) with the rotation replaced by the modality's R_m
    (OmniKVQuant value bullet).
    """
    L, d = v.shape
    R = np.asarray(rot, np.float32).astype(np.float64)
    n = np.sqrt(np.sum(v * v, axis=1))
    norms = n.astype(np.float16)
    r = np.zeros_like(v)
    for m in range(N_MODALITIES):
        idx = modality == m
        if idx.any():
            r[idx] = v[idx] @ R[m]          # r_j = sum_i R_ij v_i, i.e. R_m^T v
    codes = np.zeros((L, d), np.uint8)
    ok = n > 0
    z = np.sqrt(d) * r[ok] / n[ok][:, None]
    codes[ok] = nearest_level(z, codebook)
    return codes, norms


def value_normalized_values(v: np.ndarray, modality: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """The fp64 value z each value element's code is decided on (NaN for n == 0)."""
    L, d = v.shape
    R = np.asarray(rot, np.float32).astype(np.float64)
    n = np.sqrt(np.sum(v * v, axis=1))
    r = np.zeros_like(v)
    for m in range(N_MODALITIES):
        idx = modality == m
        if idx.any():
            r[idx] = v[idx] @ R[m]
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.sqrt(d) * r / n[:, None]
    z[n == 0] = np.nan
    return z


def dequantize_values_rotated(codes: np.ndarray, norms16: np.ndarray,
                              codebook: np.ndarray) -> np.ndarray:
    """v_tilde = (N / sqrt(d)) c[code], still in the modality's rotated frame."""
    d = codes.shape[1]
    c = np.asarray(codebook, np.float32).astype(np.float64)
    return (norms16.astype(np.float64) / np.sqrt(d))[:, None] * c[codes]


# ------------------------------------------------------------------- decode

def rotate_query(q: np.ndarray, signs: np.ndarray, n_kv_heads: int) -> np.ndarray:
    """q: [Hq, d] float64 -> q_rot [Hq, d]: each query rotated once with the
    Hadamard signs of its KV head (Introduction, Implementation bullet)."""
    hq = q.shape[0]
    g = hq // n_kv_heads
    out = np.empty_like(np.asarray(q, np.float64))
    for i in range(hq):
        out[i] = randomized_hadamard(q[i], signs[i // g])
    return out


def decode_attention_head(q_rot: np.ndarray, k_codes, lo16, hi16, v_codes, norms16,
                          modality, rot, codebook, scale: float, retained=None) -> np.ndarray:
    """One query head over one KV head's packed cache, in the rotated domain.

    scores s_t = scale * <q_rot, k_hat_t>; p = softmax(s) over the cached
    positions; A_m = sum over modality-m positions of p_t v_tilde_t; output
    o = sum_m R_m A_m (the inverse value rotation applied once per modality,
    after aggregation).

    retained: optional boolean mask over positions (a sparse page set: the
    positions kept, e.g. on the pages a retention policy kept).  Positions
    outside it take no part: the softmax runs over the retained positions
    only, and no retained position yields zeros."""
    L = k_codes.shape[0]
    d = q_rot.shape[-1]
    keep = np.ones(L, bool) if retained is None else np.asarray(retained, bool)[:L]
    if L == 0 or not keep.any():
        return np.zeros(d)
    k_hat = dequantize_keys(k_codes, lo16, hi16, codebook)
    s = scale * (k_hat @ q_rot)
    p = np.zeros(L)
    p[keep] = np.exp(s[keep] - s[keep].max())
    p = p / p.sum()
    v_t = dequantize_values_rotated(v_codes, norms16, codebook)
    R = np.asarray(rot, np.float32).astype(np.float64)
    o = np.zeros(d)
    for m in range(N_MODALITIES):
        idx = (modality == m) & keep
        if idx.any():
            o += R[m] @ (p[idx] @ v_t[idx])
    return o


def decode_attention(q_rot: np.ndarray, caches: list, rot: np.ndarray, codebook,
                     scale: float, retained=None) -> np.ndarray:
    """q_rot: [Hq, d]; caches: per KV head dicts with k_codes, lo, hi, v_codes,
    norms and the shared modality; rot: [Hkv, 3, d, d]; retained: optional
    position mask (see decode_attention_head).  Returns [Hq, d]."""
    hq, d = q_rot.shape
    hkv = len(caches)
    g = hq // hkv
    out = np.zeros((hq, d))
    for i in range(hq):
        c = caches[i // g]
        out[i] = decode_attention_head(q_rot[i], c["k_codes"], c["lo"], c["hi"],
                                       c["v_codes"], c["norms"], c["modality"],
                                       rot[i // g], codebook, scale, retained)
    return out


# --------------------------------------------------------- whole sessions

def quantize_session(k: np.ndarray, v: np.ndarray, modality: np.ndarray,
                     signs: np.ndarray, rot: np.ndarray, codebook) -> list:
    """k, v: [L, Hkv, d] float64 -> per KV head packed-cache dicts (logical layout)."""
    hkv = k.shape[1]
    out = []
    for h in range(hkv):
        kc, lo, hi = quantize_keys(k[:, h], signs[h], codebook)
        vc, nrm = quantize_values(v[:, h], modality, rot[h], codebook)
        out.append(dict(k_codes=kc, lo=lo, hi=hi, v_codes=vc, norms=nrm, modality=modality))
    return out


# ------------------------------------------------------ TurboQuant baseline

def quantize_keys_per_token(k: np.ndarray, signs: np.ndarray, codebook) -> tuple:
    """TurboQuant key codec for one KV head (Sec. 2 Method, TurboQuant bullet):
    magnitude n = ||k|| apart, direction rotated by the randomized Hadamard,
    z = sqrt(d) y / n on the fixed codebook.  k: [L, d] float64.  Returns
    codes [L, d] uint8 and norms [L] float16; n == 0 gives codes 0."""
    L, d = k.shape
    y = randomized_hadamard(k, signs)
    n = np.sqrt(np.sum(np.asarray(k, np.float64) ** 2, axis=1))
    codes = np.zeros((L, d), np.uint8)
    ok = n > 0
    codes[ok] = nearest_level(np.sqrt(d) * y[ok] / n[ok][:, None], codebook)
    return codes, n.astype(np.float16)


def key_per_token_normalized_values(k: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """The fp64 value z each per-token key code is decided on (NaN for n == 0)."""
    d = k.shape[1]
    y = randomized_hadamard(k, signs)
    n = np.sqrt(np.sum(np.asarray(k, np.float64) ** 2, axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.sqrt(d) * y / n[:, None]
    z[n == 0] = np.nan
    return z


def dequantize_keys_per_token(codes: np.ndarray, norms16: np.ndarray, codebook) -> np.ndarray:
    """Rotated-domain reconstruction y_hat = (N / sqrt(d)) c[code]."""
    return dequantize_values_rotated(codes, norms16, codebook)


def hadamard_value_basis(signs: np.ndarray) -> np.ndarray:
    """R [d, d] with R^T v = H_d (s * v) / sqrt(d): the shared randomized
    Hadamard of TurboQuant written as a value basis (columns = basis)."""
    d = len(signs)
    # row i of the transform of the identity is s_i H_d[:, i] / sqrt(d): the
    # matrix D H_d / sqrt(d), whose columns give v @ R = H_d (s * v) / sqrt(d)
    return randomized_hadamard(np.eye(d), signs)


def decode_attention_head_per_token_keys(q_rot, k_codes, k_norms16, v_codes, norms16, modality, rot,
                                         codebook, scale: float, retained=None) -> np.ndarray:
    """decode_attention_head with TurboQuant keys: k_hat_t = (N_t / sqrt(d)) c[code]
    in the rotated domain; values and the softmax as before."""
    L = k_codes.shape[0]
    d = q_rot.shape[-1]
    keep = np.ones(L, bool) if retained is None else np.asarray(retained, bool)[:L]
    if L == 0 or not keep.any():
        return np.zeros(d)
    k_hat = dequantize_keys_per_token(k_codes, k_norms16, codebook)
    s = scale * (k_hat @ q_rot)
    p = np.zeros(L)
    p[keep] = np.exp(s[keep] - s[keep].max())
    p = p / p.sum()
    v_t = dequantize_values_rotated(v_codes, norms16, codebook)
    R = np.asarray(rot, np.float32).astype(np.float64)
    o = np.zeros(d)
    for m in range(N_MODALITIES):
        idx = (modality == m) & keep
        if idx.any():
            o += R[m] @ (p[idx] @ v_t[idx])
    return o


# ----------------------------------------------------- key-grouping harness

GROUP_ORDERS = ("temporal", "modality", "modality_shuffled", "shuffled")


def grouping_order(modality: np.ndarray, order: str, seed: int = 0) -> np.ndarray:
    """Token order in which the 32-token key groups are formed.
    temporal: stream order; modality: all tokens of modality 0, then 1, then
    2, each in stream order; modality_shuffled: the same blocks, each in a
    random order; shuffled: one random order over the whole stream."""
    L = len(modality)
    rng = np.random.default_rng(seed)
    if order == "temporal":
        return np.arange(L)
    if order == "modality":
        return np.argsort(modality, kind="stable")
    if order == "modality_shuffled":
        return np.concatenate([rng.permutation(np.flatnonzero(modality == m)) for m in range(N_MODALITIES)])
    if order == "shuffled":
        return rng.permutation(L)
    raise ValueError(order)


def key_grouping_error(k: np.ndarray, modality: np.ndarray, signs: np.ndarray, codebook,
                       order: str, seed: int = 0) -> float:
    """Relative squared error sum ||y - y_hat||^2 / sum ||y||^2 of one KV
    head's rotated keys when the min-max groups are formed in `order`."""
    perm = grouping_order(modality, order, seed)
    kp = np.asarray(k, np.float64)[perm]
    codes, lo, hi = quantize_keys(kp, signs, codebook)
    y = randomized_hadamard(kp, signs)
    y_hat = dequantize_keys(codes, lo, hi, codebook)
    return float(((y - y_hat) ** 2).sum() / (y ** 2).sum())


def per_token_key_error(k: np.ndarray, signs: np.ndarray, codebook) -> float:
    """The same relative error for TurboQuant's per-token key codec."""
    codes, norms = quantize_keys_per_token(k, signs, codebook)
    y = randomized_hadamard(k, signs)
    y_hat = dequantize_keys_per_token(codes, norms, codebook)
    return float(((y - y_hat) ** 2).sum() / (y ** 2).sum())
