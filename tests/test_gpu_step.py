"""GPU checks of the fused decode step (kvq_decode_step): one call that
appends one position to every session, rotates the queries and attends every
position, including the new one.

Against the two calls it stands for (kvq_append_and_rotate, then
kvq_decode_attention) on a twin cache: the same cache bytes, lengths and
rotated queries, bit for bit, after every step, and outputs within 1e-3
normwise of each other.  Both sides attend the same codes; they differ in
rounding only.  The partition kernel feeds its value weights p * N and the
levels to the matrix cores as fp16 (relative rounding up to 2^-11 and
2^-12), while the fused step's merge weighs the open group in fp32, so
where the open group holds most of the softmax mass the two outputs may
differ by about 2^-11 + 2^-12 = 7.3e-4 (plus fp32 summation order; the
fused step may also split the context differently).
Against the fp64 oracle attending over the GPU's own codes: within the parity
bar, 2e-3 normwise per (session, query head).  The steps cross group
boundaries (32-position groups), start from empty and one-short-of-a-group
sessions, and include a session whose open group lies on an unmapped page.
"""
import numpy as np
import pytest

from omnistream import generate
from oracle import kvq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CACHE_KEYS = ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "seq_len", "k_tail")
TWIN_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kvq_amd._lib as L
    L.load()


def H():
    import tests.kvq_harness as h
    return h


def _say(*a):
    print(*a, flush=True)


def _step_inputs(h, w, pos):
    """Position pos[b] of every session's stream as [B, 1, Hkv, d] / [B, 1]."""
    B = w.cfg.batch
    k = torch.cat([h._kv_tensor(w.k[b][None, pos[b]:pos[b] + 1], w.dtype) for b in range(B)])
    v = torch.cat([h._kv_tensor(w.v[b][None, pos[b]:pos[b] + 1], w.dtype) for b in range(B)])
    m = torch.from_numpy(np.stack([w.modality[b][pos[b]:pos[b] + 1] for b in range(B)])).cuda()
    return k, v, m


def _assert_same_cache(a, b):
    x, y = a.host_arrays(), b.host_arrays()
    for key in CACHE_KEYS:
        np.testing.assert_array_equal(x[key], y[key], err_msg=key)
    assert a.lengths() == b.lengths()


STEP_CASES = [
    # (cfg_id, overrides, starting lengths (None: the workload's), steps,
    #  unmap the page of session 1's next position, query dtype)
    (0, dict(length=700), [655], 40, False, None),                  # d = 64, G = 2, fp32
    (1, dict(length=1200), [1000], 40, False, None),                # d = 128, G = 8, bf16
    (2, dict(length=2600), [2525], 36, False, None),                # G = 7 (the 80K shape)
    (3, dict(batch=3, len_range=(600, 1300)), [0, 31, 511], 40, True, None),   # paged, empty session
    (1, dict(length=1200, n_q_heads=32), [990], 6, False, None),    # G = 16: the two-call path
    (1, dict(length=1200), [1000], 6, False, "f32"),                # fp32 queries on a bf16 cache: two calls
]


@pytest.mark.parametrize("cfg_id,kw,start,steps,unmap,qdt", STEP_CASES,
                         ids=[f"cfg{c}-{'-'.join(str(x) for x in s)}-x{n}{'-unmapped' if u else ''}-{q or 'native'}"
                              for c, _, s, n, u, q in STEP_CASES])
def test_decode_step_equals_append_and_rotate_then_decode(cfg_id, kw, start, steps, unmap, qdt):
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(cfg_id, **kw)
    B = w.cfg.batch
    _say(f"decode step cfg{cfg_id} {kw} from {start} x{steps} unmap={unmap} q={qdt or w.dtype}")
    cfg, params, sep = h.build(w, upto=start)
    _, _, fus = h.build(w, upto=start)
    if unmap:
        # the page holding session 1's next positions: nothing is stored there
        # and the decodes skip it, on both sides
        pg = start[1] // w.page_tokens
        for c in (sep, fus):
            c.page_table[1, pg] = -1
    q = h.query_tensor(w)
    if qdt == "f32":
        q = q.float()
    scale = h.default_scale(w)
    L_end = max(start) + steps
    ws_sep = torch.zeros(K.kvq_decode_workspace_bytes(cfg, L_end), dtype=torch.uint8, device="cuda")
    ws_fus = torch.zeros(K.kvq_decode_step_workspace_bytes(cfg, L_end), dtype=torch.uint8, device="cuda")
    q_fus = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    worst = 0.0
    for j in range(steps):
        k, v, m = _step_inputs(h, w, [s + j for s in start])
        q_sep = K.kvq_append_and_rotate(cfg, sep, params, k, v, m, q)
        o_sep = K.kvq_decode_attention(cfg, sep, params, q_sep, scale, workspace=ws_sep)
        o_fus = K.kvq_decode_step(cfg, fus, params, k, v, m, q, q_fus, scale, workspace=ws_fus)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q_sep.cpu().numpy(), q_fus.cpu().numpy())
        a, b = o_sep.cpu().numpy().astype(np.float64), o_fus.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(b))
        err = max(float(h.normwise_rel_err(b[i], a[i]).max()) for i in range(B))
        worst = max(worst, err)
        assert err <= TWIN_TOL, (j, err)
        if j % 8 == 0 or j == steps - 1:
            _assert_same_cache(sep, fus)
    _say(f"fused vs two calls: worst normwise difference {worst:.2e} over {steps} steps")
    assert fus.lengths() == [s + steps for s in start]
    ref = h.oracle_decode_over_gpu_codes(w, cfg, fus, O.as_f64(w.q, w.dtype), range(B), scale)
    out = o_fus.cpu().numpy().astype(np.float64)
    err = max(float(h.normwise_rel_err(out[b], ref[b]).max()) for b in range(B))
    _say(f"fused step vs oracle: worst normwise rel err {err:.3e}")
    assert err <= h.ATTN_TOL


def test_captured_decode_step_replays():
    """A fused step captured in a HIP graph and replayed 45 times (the input
    buffers refilled eagerly between replays): each replay appends at, and
    attends up to, the device length of the replay; the cache equals one
    built by the two-call sequence, and sampled replays match the oracle."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(2, length=1500, n_q_heads=28)
    start, n_rep = 1400, 45
    _say(f"captured decode step cfg2 from {start} x{n_rep}")
    cfg, params, fus = h.build(w, upto=[start])
    _, _, sep = h.build(w, upto=[start])
    scale = h.default_scale(w)
    q = h.query_tensor(w)
    k_in, v_in, m_in = _step_inputs(h, w, [start])
    q_rot = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.zeros(K.kvq_decode_step_workspace_bytes(cfg, start + n_rep), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            K.kvq_decode_step(cfg, fus, params, k_in, v_in, m_in, q, q_rot, scale, out, ws)
    torch.cuda.synchronize()
    assert int(fus.seq_len.cpu()[0]) == start          # capture does not run the kernels
    q64 = O.as_f64(w.q, w.dtype)
    for j in range(n_rep):
        k, v, m = _step_inputs(h, w, [start + j])
        k_in.copy_(k)
        v_in.copy_(v)
        m_in.copy_(m)
        g.replay()
        q_sep = K.kvq_append_and_rotate(cfg, sep, params, k, v, m, q)
        o_sep = K.kvq_decode_attention(cfg, sep, params, q_sep, scale)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert float(h.normwise_rel_err(got[0], o_sep.cpu().numpy()[0].astype(np.float64)).max()) <= TWIN_TOL
        if j in (0, 17, n_rep - 1):
            ref = h.oracle_decode_over_gpu_codes(w, cfg, sep, q64, [0], scale)
            err = float(h.normwise_rel_err(got[0], ref[0]).max())
            _say(f"replay {j} at {start + j + 1} positions: worst normwise rel err {err:.3e}")
            assert err <= h.ATTN_TOL
    assert int(fus.seq_len.cpu()[0]) == start + n_rep
    fus.set_lengths([start + n_rep])
    _assert_same_cache(sep, fus)


def test_decode_step_at_full_80k_context():
    """The benchmark's launch: one fused step on the 81,920-position workload
    (28/4 heads) against the two calls on a twin cache: the same cache bytes
    and rotated queries, and outputs equal up to fp32 summation order (the
    two calls' decode is checked against the oracle at this size by the
    parity tests)."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(2, length=81920 + 40)
    n0 = 81920
    _say(f"decode step at {n0} positions")
    cfg, params, sep = h.build(w, upto=[n0], chunks=[8192])
    _, _, fus = h.build(w, upto=[n0], chunks=[8192])
    scale = h.default_scale(w)
    q = h.query_tensor(w)
    for j in range(3):
        k, v, m = _step_inputs(h, w, [n0 + j])
        q_sep = K.kvq_append_and_rotate(cfg, sep, params, k, v, m, q)
        o_sep = K.kvq_decode_attention(cfg, sep, params, q_sep, scale)
        q_fus = torch.empty_like(q_sep)
        o_fus = K.kvq_decode_step(cfg, fus, params, k, v, m, q, q_fus, scale)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q_sep.cpu().numpy(), q_fus.cpu().numpy())
        err = float(h.normwise_rel_err(o_fus.cpu().numpy()[0].astype(np.float64),
                                       o_sep.cpu().numpy()[0].astype(np.float64)).max())
        _say(f"step {j}: fused vs two calls worst normwise difference {err:.2e}")
        assert err <= TWIN_TOL
    _assert_same_cache(sep, fus)
