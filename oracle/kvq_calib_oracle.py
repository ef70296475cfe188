"""fp64 CPU oracle for the value-basis calibration of the OmniKVQuant method.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The library's product path never calls
it, and it shares no code, constant or helper with the HIP path.

Source (the OmniKVQuant page, paperlayer.ai summary of arXiv 2609.11582,
Sec. 2 Method, second "OmniKVQuant" bullet): for values, directions are
weighted by how much they contribute to attention outputs, a covariance
matrix is formed separately for each modality, and its eigenbasis is that
modality's rotation; reconstruction uses the modality's rotation.  Sec. 3
Experiments, "Value Rotation" bullet, compares per-modality, pooled and
shared rotations by their value quantization error.

Readings where the page is silent (each repeated in the design notes):
  * Contribution of a calibration token t to attention outputs: the mean,
    over the calibration queries and the query heads of its KV group, of the
    attention probability the token receives, with full-precision keys:
    w_t = mean_{queries i, heads g} softmax_t(scale * <q_{i,g}, k_t>).
    (Rotating keys and queries with the same orthogonal map does not change
    the scores, so the unrotated vectors are used.)
  * Covariance of modality m: the w-weighted, centred second moment
    C_m = sum_t w_t (v_t - mu_m)(v_t - mu_m)^T / W_m over the tokens of
    modality m, with W_m = sum_t w_t and mu_m = sum_t w_t v_t / W_m.  A
    modality with W_m == 0 has C_m = 0 and mu_m = 0.  Tokens whose modality
    byte is not 0, 1 or 2 take no part.
  * Eigenbasis: the columns of R_m are unit eigenvectors of C_m ordered by
    decreasing eigenvalue; each column's largest-magnitude component (the
    first such component on a tie) is made positive.  C_m = 0 gives the
    identity.  R_m is handed to the cache as fp32 (rounded once).

Everything is float64; inputs are exact float64 images of fp32/bf16 data.
The eigendecomposition step is numpy's symmetric eigensolver (LAPACK).
"""
from __future__ import annotations

import numpy as np

N_MODALITIES = 3


def attention_contribution(k: np.ndarray, q_rows: np.ndarray, scale: float) -> np.ndarray:
    """Weights of one KV head's calibration tokens.

    k: [n, d] float64 keys; q_rows: [R, d] float64, every (query, head of the
    group) pair as one row.  Returns w: [n], the mean over rows of each row's
    softmax over tokens; the weights of a head sum to one (n > 0)."""
    n = k.shape[0]
    if n == 0:
        return np.zeros(0)
    s = scale * (np.asarray(q_rows, np.float64) @ np.asarray(k, np.float64).T)     # [R, n]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return p.mean(axis=0)


def contribution_weights(k: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    """k: [n, Hkv, d] float64; q: [nq, Hq, d] float64 calibration queries.
    Query head i belongs to KV head floor(i / G).  Returns [Hkv, n]."""
    n, hkv, d = k.shape
    nq, hq, _ = q.shape
    g = hq // hkv
    out = np.zeros((hkv, n))
    for h in range(hkv):
        rows = q[:, h * g:(h + 1) * g, :].reshape(nq * g, d)
        out[h] = attention_contribution(k[:, h, :], rows, scale)
    return out


def weighted_covariance(v: np.ndarray, modality: np.ndarray, w: np.ndarray):
    """One KV head: v [n, d] float64, modality [n] uint8, w [n] float64.
    Returns (C [3, d, d], W [3], mu [3, d]) per the reading above."""
    n, d = v.shape
    C = np.zeros((N_MODALITIES, d, d))
    W = np.zeros(N_MODALITIES)
    mu = np.zeros((N_MODALITIES, d))
    for m in range(N_MODALITIES):
        idx = np.asarray(modality) == m
        wm = np.asarray(w, np.float64)[idx]
        W[m] = wm.sum()
        if W[m] == 0.0:
            continue
        vm = np.asarray(v, np.float64)[idx]
        mu[m] = (wm @ vm) / W[m]
        x = vm - mu[m]
        C[m] = (x.T * wm) @ x / W[m]
    return C, W, mu


def eigenbasis(C: np.ndarray):
    """Symmetric C [d, d] -> (R [d, d] float64 with unit eigenvector columns
    in decreasing eigenvalue order and the sign rule above, lam [d])."""
    C = np.asarray(C, np.float64)
    d = C.shape[0]
    if not C.any():
        return np.eye(d), np.zeros(d)
    lam, U = np.linalg.eigh(C)
    order = np.argsort(-lam, kind="stable")
    lam, U = lam[order], U[:, order].copy()
    for j in range(d):
        i = int(np.argmax(np.abs(U[:, j])))
        if U[i, j] < 0:
            U[:, j] = -U[:, j]
    return U, lam


def calibrate_value_bases(k: np.ndarray, v: np.ndarray, modality: np.ndarray, q: np.ndarray,
                          scale: float):
    """The whole calibration: k, v [n, Hkv, d] float64, modality [n], q
    [nq, Hq, d] float64.  Returns (rot [Hkv, 3, d, d] float32 as the cache
    takes it, lam [Hkv, 3, d], weights [Hkv, n], C [Hkv, 3, d, d])."""
    n, hkv, d = v.shape
    w = contribution_weights(k, q, scale)
    rot = np.zeros((hkv, N_MODALITIES, d, d), np.float32)
    lam = np.zeros((hkv, N_MODALITIES, d))
    Cs = np.zeros((hkv, N_MODALITIES, d, d))
    for h in range(hkv):
        C, _, _ = weighted_covariance(v[:, h, :], modality, w[h])
        Cs[h] = C
        for m in range(N_MODALITIES):
            R, lam[h, m] = eigenbasis(C[m])
            rot[h, m] = R.astype(np.float32)
    return rot, lam, w, Cs


def value_quantization_error(v: np.ndarray, modality: np.ndarray, rot: np.ndarray, codebook) -> np.ndarray:
    """Relative squared reconstruction error of the 2-bit value codec per
    modality, sum ||v - v_hat||^2 / sum ||v||^2 (NaN for an empty modality).
    v: [n, d] float64 of one KV head; rot: [3, d, d] (columns = basis).  The
    codec is the TurboQuant-style one of the decode path: z = sqrt(d) R^T v / ||v||,
    nearest level, fp16 norm, v_hat = R (N / sqrt(d)) c[code]."""
    from oracle import kvq_oracle as O
    n, d = v.shape
    codes, norms = O.quantize_values(v, modality, rot, codebook)
    vt = O.dequantize_values_rotated(codes, norms, codebook)
    R = np.asarray(rot, np.float32).astype(np.float64)
    err = np.full(N_MODALITIES, np.nan)
    for m in range(N_MODALITIES):
        idx = np.asarray(modality) == m
        if idx.any():
            vh = vt[idx] @ R[m].T
            err[m] = ((v[idx] - vh) ** 2).sum() / (v[idx] ** 2).sum()
    return err
