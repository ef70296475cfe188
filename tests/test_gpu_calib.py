"""GPU parity of the value-basis calibration against the fp64 oracle.

Each step is checked on its own, fed the oracle's inputs (so a mistake in
one step cannot hide behind another), then the three steps together:
  - contribution weights: elementwise, relative 1e-11 (fp64 on both sides,
    different summation orders);
  - covariances: elementwise within 1e-12 of each matrix's largest entry,
    weight sums relative 1e-13, and exactly symmetric;
  - eigenbases: eigenvalues within 1e-12 of the largest; an eigenvector is
    unique (up to sign) only when its eigenvalue is separated from the
    others, so columns are compared where the relative gap exceeds 1e-6
    (within 1e-6, fp32 output), and every column is checked for validity:
    residual |C r - lam r| <= 1e-5 |C|, orthonormality 1e-6, and the sign
    rule (largest-magnitude component positive).
"""
import math

import numpy as np
import pytest

from omnistream import calibration_queries, generate
from oracle import kvq_calib_oracle as CO
from oracle import kvq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kvq_amd._lib as L
    L.load()


def _say(*a):
    print(*a, flush=True)


def _t(x, dtype, device="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def _stream(cfg_id, length, n_q_heads=None):
    w = generate(cfg_id, length=length, n_q_heads=n_q_heads)
    return w, w.k[0], w.v[0], w.modality[0]


# ------------------------------------------------------------ contribution

@pytest.mark.parametrize("cfg_id,length,nq,hq", [(0, 2048, 4, None), (1, 5000, 8, None), (2, 3001, 3, 28),
                                                 (1, 1, 2, None), (1, 300, 1, 2)])
def test_contribution_matches_oracle(cfg_id, length, nq, hq):
    import decode_attention_kvq_amd as K
    w, k, _, _ = _stream(cfg_id, length, hq)
    q = calibration_queries(w, nq)
    _say(f"calib contribution cfg{cfg_id} n={length} nq={nq} hq={w.cfg.n_q_heads}")
    got = K.kvq_calib_contribution(_t(k, w.dtype), _t(q, w.dtype)).cpu().numpy()
    ref = CO.contribution_weights(O.as_f64(k, w.dtype), O.as_f64(q, w.dtype), 1 / math.sqrt(w.cfg.head_dim))
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=0)
    np.testing.assert_allclose(got.sum(axis=1), 1.0, atol=1e-12)


def test_contribution_is_independent_of_token_order_and_repeats_bitwise():
    import decode_attention_kvq_amd as K
    w, k, _, _ = _stream(1, 1000)
    q = _t(calibration_queries(w, 4), w.dtype)
    kt = _t(k, w.dtype)
    _say("calib contribution repeat")
    a = K.kvq_calib_contribution(kt, q).cpu().numpy()
    b = K.kvq_calib_contribution(kt, q).cpu().numpy()
    np.testing.assert_array_equal(a, b)


# -------------------------------------------------------------- covariance

@pytest.mark.parametrize("cfg_id,length", [(0, 2048), (1, 5000), (1, 1), (2, 777)])
def test_covariance_matches_oracle(cfg_id, length):
    import decode_attention_kvq_amd as K
    w, k, v, mod = _stream(cfg_id, length)
    rng = np.random.default_rng(cfg_id * 1000 + length)
    weights = rng.uniform(0.0, 1.0, (w.cfg.n_kv_heads, length))
    mod = mod.copy()
    if length > 10:
        mod[rng.choice(length, size=max(1, length // 50), replace=False)] = 7   # bytes outside 0..2 take no part
    _say(f"calib covariance cfg{cfg_id} n={length}")
    cov, ws = K.kvq_calib_covariance(_t(v, w.dtype), _t(mod, "u8"), torch.from_numpy(weights).cuda())
    cov, ws = cov.cpu().numpy(), ws.cpu().numpy()
    v64 = O.as_f64(v, w.dtype)
    for h in range(w.cfg.n_kv_heads):
        C, W, _ = CO.weighted_covariance(v64[:, h], mod, weights[h])
        np.testing.assert_allclose(ws[h], W, rtol=1e-13, atol=0)
        for m in range(3):
            np.testing.assert_array_equal(cov[h, m], cov[h, m].T)
            tol = 1e-12 * max(np.abs(C[m]).max(), 1e-300)
            assert np.abs(cov[h, m] - C[m]).max() <= tol, (h, m)


def test_covariance_of_absent_modalities_is_zero():
    import decode_attention_kvq_amd as K
    w, k, v, mod = _stream(1, 640)
    mod = np.zeros_like(mod)                   # video only
    weights = np.full((w.cfg.n_kv_heads, 640), 1 / 640)
    _say("calib covariance video only")
    cov, ws = K.kvq_calib_covariance(_t(v, w.dtype), _t(mod, "u8"), torch.from_numpy(weights).cuda())
    cov, ws = cov.cpu().numpy(), ws.cpu().numpy()
    assert not cov[:, 1:].any() and not ws[:, 1:].any()
    np.testing.assert_allclose(ws[:, 0], 1.0, atol=1e-13)


# -------------------------------------------------------------- eigenbasis

def _check_eigenbasis(C, R, lam, ref_R, ref_lam, where="", lam_tol=1e-12):
    d = C.shape[0]
    scale = max(np.abs(ref_lam).max(), 1e-300)
    np.testing.assert_allclose(lam, ref_lam, rtol=0, atol=lam_tol * scale, err_msg=where)
    assert np.all(np.diff(lam) <= 0), where
    R64 = R.astype(np.float64)
    np.testing.assert_allclose(R64.T @ R64, np.eye(d), atol=1e-6, err_msg=where)
    res = C @ R64 - R64 * lam[None, :]
    assert np.abs(res).max() <= 1e-5 * scale, where
    for j in range(d):
        col = R64[:, j]
        i = int(np.argmax(np.abs(col)))
        top2 = np.sort(np.abs(col))[-2:]
        assert col[i] > 0 or top2[1] - top2[0] < 1e-6, (where, j)
        others = np.delete(ref_lam, j)
        gap = np.abs(others - ref_lam[j]).min() / scale if d > 1 else 1.0
        if gap > 1e-6:
            c = ref_R[:, j] * (1.0 if np.dot(ref_R[:, j], col) >= 0 else -1.0)
            assert np.abs(col - c).max() <= 1e-6 + 1e-9 / gap, (where, j, gap)


@pytest.mark.parametrize("cfg_id,length", [(0, 2048), (1, 5000), (2, 3001)])
def test_eigenbasis_matches_oracle_on_stream_covariances(cfg_id, length):
    import decode_attention_kvq_amd as K
    w, k, v, mod = _stream(cfg_id, length)
    v64 = O.as_f64(v, w.dtype)
    weights = np.random.default_rng(length).uniform(0.1, 1.0, (w.cfg.n_kv_heads, length))
    Cs = np.stack([CO.weighted_covariance(v64[:, h], mod, weights[h])[0] for h in range(w.cfg.n_kv_heads)])
    _say(f"calib eigenbasis cfg{cfg_id} n={length} count={Cs.shape[0] * 3}")
    R, lam = K.kvq_calib_eigenbasis(torch.from_numpy(Cs).cuda())
    R, lam = R.cpu().numpy(), lam.cpu().numpy()
    for h in range(Cs.shape[0]):
        for m in range(3):
            ref_R, ref_lam = CO.eigenbasis(Cs[h, m])
            _check_eigenbasis(Cs[h, m], R[h, m], lam[h, m], ref_R, ref_lam, f"h{h} m{m}")


@pytest.mark.parametrize("d", [64, 128])
def test_eigenbasis_special_matrices(d):
    import decode_attention_kvq_amd as K
    rng = np.random.default_rng(d)
    Q = np.linalg.qr(rng.standard_normal((d, d)))[0]
    lam_known = np.sort(rng.uniform(0.01, 10.0, d))[::-1] + np.arange(d)[::-1] * 1e-3
    mats = [
        (Q * lam_known) @ Q.T,                             # known basis, distinct eigenvalues
        np.zeros((d, d)),                                  # empty modality: identity
        np.diag(np.repeat([3.0, 1.0], d // 2)),            # repeated eigenvalues
        np.diag(rng.uniform(-1, 1, d)),                    # already diagonal, mixed signs
        np.ones((d, d)),                                   # rank one
    ]
    Cs = np.stack(mats)
    Cs = (Cs + np.swapaxes(Cs, 1, 2)) / 2
    _say(f"calib eigenbasis special d={d}")
    R, lam = K.kvq_calib_eigenbasis(torch.from_numpy(Cs).cuda())
    R, lam = R.cpu().numpy(), lam.cpu().numpy()
    for i, C in enumerate(Cs):
        ref_R, ref_lam = CO.eigenbasis(C)
        _check_eigenbasis(C, R[i], lam[i], ref_R, ref_lam, f"matrix {i}")
    np.testing.assert_array_equal(R[1], np.eye(d, dtype=np.float32))
    for j in range(d):
        i = int(np.argmax(np.abs(Q[:, j])))
        np.testing.assert_allclose(R[0][:, j], Q[:, j] * np.sign(Q[i, j]), atol=2e-6)


# ---------------------------------------------------------------- pipeline

@pytest.mark.parametrize("cfg_id,length,nq", [(1, 16384, 8), (2, 81920, 8)])
def test_full_calibration_matches_oracle(cfg_id, length, nq):
    """Contribution -> covariance -> eigenbasis on the GPU, against the oracle's
    whole calibration, at the stream sizes of the 16K and 80K workloads."""
    import decode_attention_kvq_amd as K
    w, k, v, mod = _stream(cfg_id, length)
    q = calibration_queries(w, nq)
    _say(f"calib pipeline cfg{cfg_id} n={length} nq={nq}")
    wt = K.kvq_calib_contribution(_t(k, w.dtype), _t(q, w.dtype))
    cov, _ = K.kvq_calib_covariance(_t(v, w.dtype), _t(mod, "u8"), wt)
    R, lam = K.kvq_calib_eigenbasis(cov)
    torch.cuda.synchronize()
    R, lam, cov = R.cpu().numpy(), lam.cpu().numpy(), cov.cpu().numpy()
    ref_rot, ref_lam, ref_w, ref_C = CO.calibrate_value_bases(
        O.as_f64(k, w.dtype), O.as_f64(v, w.dtype), mod, O.as_f64(q, w.dtype), 1 / math.sqrt(w.cfg.head_dim))
    np.testing.assert_allclose(wt.cpu().numpy(), ref_w, rtol=1e-11, atol=0)
    for h in range(w.cfg.n_kv_heads):
        for m in range(3):
            tol = 1e-11 * max(np.abs(ref_C[h, m]).max(), 1e-300)
            assert np.abs(cov[h, m] - ref_C[h, m]).max() <= tol
            ref_R, _ = CO.eigenbasis(ref_C[h, m])
            # the GPU's covariance differs from the oracle's by rounding: eigenvalues within 1e-10
            _check_eigenbasis(ref_C[h, m], R[h, m], lam[h, m], ref_R, ref_lam[h, m], f"h{h} m{m}", lam_tol=1e-10)
