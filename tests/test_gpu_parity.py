"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bar: key/value codes and fp16 statistics bit-exact (codes may differ only
within 1e-6 of a decision threshold, counted, < 1e-5 of all elements);
rotated queries bit-exact (one fp32 rounding of the fp64 transform);
decode outputs within 2e-3 normwise relative error per (session, query head)
of the oracle attending over the same packed codes.
"""
import math

import numpy as np
import pytest

from omnistream import generate
from oracle import kvq_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


# ------------------------------------------------------------ query rotation

@pytest.mark.parametrize("cfg_id", [0, 1, 2, 4])
def test_rotate_query_bit_exact(cfg_id):
    import decode_attention_kvq_amd as K
    w = generate(cfg_id, length=64)
    _say(f"rotate_query cfg{cfg_id}")
    cfg, params, cache = H().build(w)
    q_rot = K.kvq_rotate_query(cfg, params, H().query_tensor(w)).cpu().numpy()
    q64 = O.as_f64(w.q, w.dtype)
    for b in range(w.cfg.batch):
        ref = O.rotate_query(q64[b], w.signs, w.cfg.n_kv_heads).astype(np.float32)
        np.testing.assert_array_equal(q_rot[b], ref)


# ----------------------------------------------------- quantize-append + decode

CASES = [
    # (cfg_id, overrides) -- several tiles and a ragged tail at each size
    (0, dict()),
    (1, dict(length=3001)),
    (2, dict(length=5000)),
    (3, dict(batch=3, len_range=(700, 2600))),
    (4, dict(length=1500)),
    # GQA groups above 8 (the one-role partition kernel): 16, 12 and 10 heads
    (1, dict(length=3001, n_q_heads=32)),
    (0, dict(length=1000, n_q_heads=12)),
    (3, dict(batch=2, len_range=(700, 1900), n_q_heads=20)),
    # page sizes: one group per page, a size that is not a power of two, large pages
    (1, dict(length=3001, page_tokens=32)),
    (3, dict(batch=3, len_range=(700, 2600), page_tokens=96)),
    (0, dict(length=2100, page_tokens=512)),
]


def _case_id(c, kw):
    s = f"cfg{c}"
    if "n_q_heads" in kw:
        s += f"-G{kw['n_q_heads']}"
    if "page_tokens" in kw:
        s += f"-P{kw['page_tokens']}"
    return s


@pytest.mark.parametrize("cfg_id,kw", CASES, ids=[_case_id(c, kw) for c, kw in CASES])
def test_append_and_decode_parity(cfg_id, kw):
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(cfg_id, **kw)
    _say(f"append+decode cfg{cfg_id} {kw} lengths={w.lengths.tolist()}")
    cfg, params, cache = h.build(w)
    total, mism = h.check_codes(w, cfg, cache, range(w.cfg.batch))
    _say(f"codes: {total} elements, {mism} boundary mismatches")
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale).cpu().numpy()
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), range(w.cfg.batch), scale)
    worst = 0.0
    for b in range(w.cfg.batch):
        err = h.normwise_rel_err(out[b].astype(np.float64), ref[b])
        worst = max(worst, float(err.max()))
    _say(f"decode worst normwise rel err {worst:.3e}")
    assert worst <= h.ATTN_TOL


# An asymmetric codebook (c0 + c3 != 0): the decode then carries the
# codebook's midpoint through the per-modality weight sums of the partials.
ASYM_CODEBOOK = np.array([-1.2, -0.35, 0.55, 1.8], dtype=np.float32)
ASYM_CASES = [
    (0, dict(length=1500)),                          # a few partitions per head: the all-heads merge
    (3, dict(batch=3, len_range=(200, 500))),         # a ragged batch, all-heads merge
    (2, dict(length=20000)),                         # 64 partitions per head: the per-head merge
    (3, dict(batch=3, len_range=(700, 2600))),        # a ragged batch, per-head merge
    (1, dict(length=3001, n_q_heads=32)),            # 16 heads per KV head: the one-role partition kernel
    (1, dict(length=1000, n_q_heads=32)),            # the same with few partitions: all-heads merge, 16 heads
]


@pytest.mark.parametrize("cfg_id,kw", ASYM_CASES, ids=[f"asym-{_case_id(c, kw)}-{i}" for i, (c, kw) in enumerate(ASYM_CASES)])
def test_asymmetric_codebook_parity(cfg_id, kw):
    import dataclasses
    import decode_attention_kvq_amd as K
    h = H()
    w = dataclasses.replace(generate(cfg_id, **kw), codebook=ASYM_CODEBOOK.copy())
    _say(f"asymmetric codebook cfg{cfg_id} {kw} lengths={w.lengths.tolist()}")
    cfg, params, cache = h.build(w)
    total, mism = h.check_codes(w, cfg, cache, range(w.cfg.batch))
    _say(f"codes: {total} elements, {mism} boundary mismatches")
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale).cpu().numpy()
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), range(w.cfg.batch), scale)
    worst = 0.0
    for b in range(w.cfg.batch):
        worst = max(worst, float(h.normwise_rel_err(out[b].astype(np.float64), ref[b]).max()))
    _say(f"decode worst normwise rel err {worst:.3e}")
    assert worst <= h.ATTN_TOL


FUSED_CASES = [
    # (cfg_id, overrides, positions appended, first session, query dtype)
    (0, dict(length=700), 1, 0, None),
    (1, dict(length=1200), 45, 0, None),
    (2, dict(length=900), 0, 0, None),
    (2, dict(length=900), 1, 0, "f32"),
    (3, dict(batch=3, len_range=(500, 1300)), 3, 1, None),
]


@pytest.mark.parametrize("cfg_id,kw,n_new,b0,qdt", FUSED_CASES,
                         ids=[f"cfg{c}-n{n}-b{b}-{q or 'native'}" for c, _, n, b, q in FUSED_CASES])
def test_append_and_rotate_equals_separate_calls(cfg_id, kw, n_new, b0, qdt):
    """kvq_append_and_rotate gives the same cache bytes, lengths and rotated
    queries as kvq_quantize_append followed by kvq_rotate_query."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(cfg_id, **kw)
    nb = w.cfg.batch - b0
    upto = [max(int(n) - n_new, 0) for n in w.lengths]
    _say(f"fused append+rotate cfg{cfg_id} {kw} n_new={n_new} b0={b0} q={qdt or w.dtype} upto={upto}")
    cfg, params, sep = h.build(w, upto=upto)
    _, _, fus = h.build(w, upto=upto)
    q = h.query_tensor(w)
    if qdt == "f32":
        q = q.float()
    # every appended session gets the positions that follow its own prefix
    ks = [h._kv_tensor(w.k[b][None, upto[b]:upto[b] + n_new], w.dtype) for b in range(b0, b0 + nb)]
    vs = [h._kv_tensor(w.v[b][None, upto[b]:upto[b] + n_new], w.dtype) for b in range(b0, b0 + nb)]
    ms = [torch.from_numpy(np.ascontiguousarray(w.modality[b][None, upto[b]:upto[b] + n_new])).cuda()
          for b in range(b0, b0 + nb)]
    k_new, v_new, m_new = torch.cat(ks), torch.cat(vs), torch.cat(ms)
    K.kvq_quantize_append(cfg, sep, params, k_new, v_new, m_new, b0=b0)
    q_sep = K.kvq_rotate_query(cfg, params, q)
    q_fus = K.kvq_append_and_rotate(cfg, fus, params, k_new, v_new, m_new, q, b0=b0)
    torch.cuda.synchronize()
    a, b = sep.host_arrays(), fus.host_arrays()
    for key in ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "seq_len", "k_tail"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    assert sep.lengths() == fus.lengths()
    np.testing.assert_array_equal(q_sep.cpu().numpy(), q_fus.cpu().numpy())
    if n_new:
        h.check_codes(w, cfg, fus, range(b0, b0 + nb), lengths=[upto[b] + n_new for b in range(w.cfg.batch)])


def test_chunked_append_equals_one_shot():
    """Appends of ragged sizes (re-quantizing the open group from the raw key
    tail each time) give the same cache bytes as one append of the stream."""
    h = H()
    w = generate(1, length=1111)
    _say("chunked append cfg1 1111")
    cfg, params, one = h.build(w)
    _, _, many = h.build(w, chunks=[1, 7, 31, 33, 64, 5, 100, 2, 32])
    a, b = one.host_arrays(), many.host_arrays()
    for key in ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "seq_len"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    h.check_codes(w, cfg, many, [0])


def test_paged_equals_contiguous():
    """The same sessions under a shuffled page table decode to the same output."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(3, batch=4, len_range=(300, 1500))
    _say("paged vs contiguous cfg3 b=4")
    ident = np.full_like(w.page_table, -1)
    off = 0
    for b in range(4):
        n = int((w.page_table[b] >= 0).sum())
        ident[b, :n] = np.arange(off, off + n)
        off += n
    cfg_p, params, cache_p = h.build(w)
    cfg_c, _, cache_c = h.build(w, page_table=ident)
    q_rot = K.kvq_rotate_query(cfg_p, params, h.query_tensor(w))
    out_p = K.kvq_decode_attention(cfg_p, cache_p, params, q_rot).cpu().numpy()
    out_c = K.kvq_decode_attention(cfg_c, cache_c, params, q_rot).cpu().numpy()
    np.testing.assert_array_equal(out_p, out_c)


# ------------------------------------------------ sparse page sets

RETAINED_CASES = [
    # (cfg_id, overrides, which logical pages lose their mapping)
    (3, dict(batch=3, len_range=(700, 2600)), "random"),
    (2, dict(length=5000), "alternate"),
    (1, dict(length=3001, page_tokens=32), "random"),
    (3, dict(batch=3, len_range=(700, 2600), page_tokens=96), "random"),
    (3, dict(batch=3, len_range=(400, 1200)), "session"),
]


def _evicted(pattern: str, b: int, npg: int, rng) -> np.ndarray:
    if pattern == "random":
        return rng.random(npg) < 0.4
    if pattern == "alternate":
        return np.arange(npg) % 2 == 1
    return np.full(npg, b == 1)          # "session": every page of session 1


@pytest.mark.parametrize("cfg_id,kw,pattern", RETAINED_CASES,
                         ids=[_case_id(c, kw) + f"-{p}" for c, kw, p in RETAINED_CASES])
def test_decode_over_retained_pages(cfg_id, kw, pattern):
    """A page-table entry of -1 drops that logical page from the decode: the
    softmax runs over the positions of the mapped pages only (the oracle with
    the same position mask), and a session with no mapped page gives zeros."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(cfg_id, **kw)
    rng = np.random.default_rng(17)
    cfg, params, cache = h.build(w)
    pt = cache.page_table.cpu().numpy()
    dropped = []
    for b in range(w.cfg.batch):
        npg = -(-int(w.lengths[b]) // w.page_tokens)
        ev = _evicted(pattern, b, npg, rng)
        pt[b, :npg][ev] = -1
        dropped.append(int(ev.sum()))
    cache.page_table.copy_(torch.from_numpy(pt))
    _say(f"retained pages cfg{cfg_id} {kw} {pattern}: lengths={w.lengths.tolist()} pages dropped={dropped}")
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale).cpu().numpy()
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), range(w.cfg.batch), scale)
    worst = 0.0
    for b in range(w.cfg.batch):
        if (pt[b] >= 0).sum() == 0:
            np.testing.assert_array_equal(out[b], 0.0)
            continue
        worst = max(worst, float(h.normwise_rel_err(out[b].astype(np.float64), ref[b]).max()))
    _say(f"decode worst normwise rel err {worst:.3e}")
    assert worst <= h.ATTN_TOL


@pytest.mark.parametrize("chunks", [[45, 300, 7, 256], [1, 1, 1, 61]], ids=["chunked", "one-position"])
def test_append_skips_unmapped_pages(chunks):
    """Positions appended while their logical page has no physical page are not
    stored: every mapped page holds the same bytes as in a build with all pages
    mapped, the pages nobody maps stay untouched, lengths still advance, and
    the decode equals the fully mapped cache's decode under the same sparse
    page table.  Both append paths: longer appends, and one-position appends
    (the decode step's, which read their inputs before the length is known)
    at every offset inside a group."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(3, batch=3, len_range=(900, 2600))
    rng = np.random.default_rng(23)
    sparse = w.page_table.copy()
    for b in range(w.cfg.batch):
        npg = -(-int(w.lengths[b]) // w.page_tokens)
        sparse[b, :npg][rng.random(npg) < 0.5] = -1
    num_pages = int(w.page_table.max()) + 1
    _say(f"append onto unmapped pages: lengths={w.lengths.tolist()} "
         f"unmapped={int((sparse < 0).sum() - (w.page_table < 0).sum())} chunks={chunks}")
    cfg, params, full = h.build(w, chunks=chunks)
    _, _, part = h.build(w, page_table=sparse, chunks=chunks, num_pages=num_pages)
    a, b = full.host_arrays(), part.host_arrays()
    np.testing.assert_array_equal(a["seq_len"], b["seq_len"])
    kept = np.unique(sparse[sparse >= 0])
    free = np.setdiff1d(np.arange(num_pages), kept)
    for key in ("k_codes", "k_stats", "v_codes", "v_norms", "modality"):
        pa, pb = a[key].reshape(num_pages, -1), b[key].reshape(num_pages, -1)
        np.testing.assert_array_equal(pa[kept], pb[kept], err_msg=key)
        assert not pb[free].any(), f"{key}: an unmapped page was written"
    full.page_table.copy_(torch.from_numpy(sparse))
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    np.testing.assert_array_equal(K.kvq_decode_attention(cfg, part, params, q_rot).cpu().numpy(),
                                  K.kvq_decode_attention(cfg, full, params, q_rot).cpu().numpy())


def test_empty_and_tiny_sessions():
    """Session lengths 0, 1, 31, 32, 33: empty gives zeros, one position gives
    that position's reconstructed value."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(3, batch=5, len_range=(40, 60))
    upto = [0, 1, 31, 32, 33]
    _say(f"tiny sessions {upto}")
    cfg, params, cache = h.build(w, upto=upto)
    h.check_codes(w, cfg, cache, [1, 2, 3, 4], lengths=upto)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot).cpu().numpy()
    np.testing.assert_array_equal(out[0], 0.0)
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), [1, 2, 3, 4],
                                         h.default_scale(w))
    for b in [1, 2, 3, 4]:
        assert h.normwise_rel_err(out[b].astype(np.float64), ref[b]).max() <= h.ATTN_TOL


def test_decode_is_repeatable_and_scale_respected():
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(1, length=2000)
    cfg, params, cache = h.build(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    a = K.kvq_decode_attention(cfg, cache, params, q_rot, 0.05).cpu().numpy()
    b = K.kvq_decode_attention(cfg, cache, params, q_rot, 0.05).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), [0], 0.05)
    assert h.normwise_rel_err(a[0].astype(np.float64), ref[0]).max() <= h.ATTN_TOL


def test_graph_replays_match_eager():
    """A captured decode (no memset nodes) replayed several times, with eager
    work in between, reproduces the eager output on every replay."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(2, length=3000)
    _say("graph replay cfg2 3000")
    cfg, params, cache = h.build(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    eager = K.kvq_decode_attention(cfg, cache, params, q_rot).clone()
    out = torch.empty_like(eager)
    ws = torch.zeros(K.kvq_decode_workspace_bytes(cfg, 3000), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            K.kvq_decode_attention(cfg, cache, params, q_rot, None, out, ws)
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        K.kvq_rotate_query(cfg, params, h.query_tensor(w), q_rot)   # eager work between replays
        torch.cuda.synchronize()


def test_many_partitions_merge():
    """A context long enough for more partitions than the merge keeps in
    flight at once (d = 64, one KV head: 70,000 positions)."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(0, length=70000)
    _say("many partitions cfg0 70000")
    cfg, params, cache = h.build(w, chunks=[4096])
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale).cpu().numpy()
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), [0], scale)
    err = float(h.normwise_rel_err(out[0].astype(np.float64), ref[0]).max())
    _say(f"decode worst normwise rel err {err:.3e}")
    assert err <= h.ATTN_TOL


def test_graph_replayed_single_token_appends():
    """A captured one-position append replayed 70 times (the input buffer is
    refilled eagerly between replays) advances the device length itself and
    leaves the same cache as appending the stream directly."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(1, length=200)
    _say("graph-replayed appends cfg1 130 -> 200")
    cfg, params, cache = h.build(w, upto=[130])
    k_in = h._kv_tensor(w.k[0][None, 130:131], w.dtype)
    v_in = h._kv_tensor(w.v[0][None, 130:131], w.dtype)
    m_in = torch.from_numpy(np.ascontiguousarray(w.modality[0][None, 130:131])).cuda()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            K.kvq_quantize_append(cfg, cache, params, k_in, v_in, m_in)
    torch.cuda.synchronize()
    assert int(cache.seq_len.cpu()[0]) == 130          # capture does not run the kernel
    for t in range(130, 200):
        k_in.copy_(h._kv_tensor(w.k[0][None, t:t + 1], w.dtype))
        v_in.copy_(h._kv_tensor(w.v[0][None, t:t + 1], w.dtype))
        m_in.copy_(torch.from_numpy(np.ascontiguousarray(w.modality[0][None, t:t + 1])).cuda())
        g.replay()
    torch.cuda.synchronize()
    assert int(cache.seq_len.cpu()[0]) == 200
    assert int(cache.append_tickets.cpu()[0]) == 0
    cache.set_lengths([200])
    _, _, ref = h.build(w)
    a, b = cache.host_arrays(), ref.host_arrays()
    for key in ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "seq_len"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


# ------------------------------------------------------- full-size workloads

ORACLE_THREADS = 16    # host threads for the oracle side of the full-size checks


def _decode_parity(w, cfg, params, cache, sessions, out=None):
    import decode_attention_kvq_amd as K
    h = H()
    scale = h.default_scale(w)
    if out is None:
        q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
        out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale).cpu().numpy()
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), sessions, scale,
                                         threads=ORACLE_THREADS)
    worst = max(float(h.normwise_rel_err(out[b].astype(np.float64), ref[b]).max()) for b in sessions)
    return worst


def test_full_80k_context():
    """The benchmark's workload at full size (81,920 positions, 28/4 heads):
    every code and statistic, and every head's output."""
    h = H()
    w = generate(2)
    _say(f"full 80K: {int(w.lengths[0])} positions")
    cfg, params, cache = h.build(w, chunks=[8192])
    total, mism = h.check_codes(w, cfg, cache, [0])
    _say(f"codes: {total} elements, {mism} boundary mismatches")
    worst = _decode_parity(w, cfg, params, cache, [0])
    _say(f"decode worst normwise rel err {worst:.3e}")
    assert worst <= h.ATTN_TOL


def test_full_16k_context():
    """The 16K workload at its full size (16,384 positions, 16/2 heads):
    every code and statistic, and every head's output."""
    h = H()
    w = generate(1)
    assert int(w.lengths[0]) == 16384
    _say(f"full 16K: {int(w.lengths[0])} positions")
    cfg, params, cache = h.build(w, chunks=[5000])
    total, mism = h.check_codes(w, cfg, cache, [0])
    _say(f"codes: {total} elements, {mism} boundary mismatches")
    worst = _decode_parity(w, cfg, params, cache, [0])
    _say(f"decode worst normwise rel err {worst:.3e}")
    assert worst <= h.ATTN_TOL


def test_full_batched_paged_sessions():
    """32 sessions of 8K..64K positions under a random page table, decoded in
    one launch: the codes and statistics of every session and every head's
    output against the oracle."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(3)
    _say(f"full batched: {w.cfg.batch} sessions, {int(w.lengths.sum())} positions")
    cfg, params, cache = h.build(w, chunks=[16384])
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, h.default_scale(w)).cpu().numpy()
    assert np.all(np.isfinite(out))
    sessions = list(range(w.cfg.batch))
    total, mism = h.check_codes(w, cfg, cache, sessions, threads=ORACLE_THREADS)
    _say(f"codes of all {len(sessions)} sessions: {total} elements, {mism} boundary mismatches")
    worst = _decode_parity(w, cfg, params, cache, sessions, out)
    _say(f"decode worst normwise rel err over all sessions {worst:.3e}")
    assert worst <= h.ATTN_TOL


def test_full_stream_loop_append():
    """A 131,072-position cache (32/8 heads), then one 1,024-position chunk
    (640 video + 25 audio + 359 text) appended in one call, then the decode."""
    h = H()
    w = generate(4)
    n0 = int(w.prefix_lengths[0])
    _say(f"stream loop: prefill {n0}, append {int(w.lengths[0]) - n0}")
    cfg, params, cache = h.build(w, upto=[n0 + 5], chunks=[16384])   # an open group before the chunk
    h.append_range(cfg, cache, params, w, 0, n0 + 5, int(w.lengths[0]))
    total, mism = h.check_codes(w, cfg, cache, [0])
    _say(f"codes: {total} elements, {mism} boundary mismatches")
    worst = _decode_parity(w, cfg, params, cache, [0])
    _say(f"decode worst normwise rel err {worst:.3e}")
    assert worst <= h.ATTN_TOL


def test_degenerate_inputs():
    """Zero value vectors (norm 0: codes 0), key channels constant over a
    whole group (HI == LO: codes 0), and a group that is all one value."""
    h = H()
    w = generate(1, length=700)
    k, v = w.k[0], w.v[0]
    v[100] = 0                                   # bf16 +0
    v[101:133] = 0
    k[64:96, 0, 5] = k[64, 0, 5]                 # channel 5 of KV head 0 constant in group 2
    k[160:192, 1, :] = k[160, 1, :]              # a whole group of identical keys (after rotation too)
    _say("degenerate inputs cfg1 700")
    cfg, params, cache = h.build(w, chunks=[97, 3, 600])
    total, mism = h.check_codes(w, cfg, cache, [0])
    worst = _decode_parity(w, cfg, params, cache, [0])
    _say(f"codes {total} ({mism} at thresholds), decode worst {worst:.3e}")
    assert worst <= h.ATTN_TOL
