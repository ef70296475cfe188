"""GPU checks of the decode beyond the workloads' own value scale and shapes:
small value norms, bf16 output, and a captured decode replayed after the
sessions have grown past the plan it was captured with.  Same bar as the
parity tests: outputs within 2e-3 normwise relative error per (session,
query head) of the fp64 oracle attending over the GPU's own codes.
"""
import dataclasses

import numpy as np
import pytest

from omnistream import bf16_bits_to_f64, f64_to_bf16_bits, generate
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


def _scaled_values(w, factor):
    """The workload with every value vector multiplied by `factor` (rounded
    back to the workload's dtype)."""
    if w.dtype == "bf16":
        v = [f64_to_bf16_bits(bf16_bits_to_f64(x) * factor) for x in w.v]
    else:
        v = [(x.astype(np.float64) * factor).astype(np.float32) for x in w.v]
    return dataclasses.replace(w, v=v)


def _decode_err(w, cfg, params, cache, out_dtype=torch.float32):
    import decode_attention_kvq_amd as K
    h = H()
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale, out_dtype=out_dtype)
    out = out.float().cpu().numpy().astype(np.float64)
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), range(w.cfg.batch), scale)
    return max(float(h.normwise_rel_err(out[b], ref[b]).max()) for b in range(w.cfg.batch))


SMALL_NORM_CASES = [
    # (cfg_id, overrides): the streaming kernel at d = 64 (G = 2) and d = 128
    # (G = 8), and the one-role kernel (G = 16; pages of 96 positions)
    (0, dict(length=1500)),
    (1, dict(length=3001)),
    (1, dict(length=2100, n_q_heads=32)),
    (3, dict(batch=2, len_range=(700, 1500), page_tokens=96)),
]


@pytest.mark.parametrize("factor", [1e-2, 1e-3, 30.0])
@pytest.mark.parametrize("cfg_id,kw", SMALL_NORM_CASES,
                         ids=[f"cfg{c}-" + "-".join(f"{k}{v}" for k, v in kw.items()) for c, kw in SMALL_NORM_CASES])
def test_decode_accuracy_does_not_depend_on_the_value_scale(cfg_id, kw, factor):
    """Value norms 100x and 1000x smaller (and 30x larger) than the
    generator's: the value-weight operands must stay in the fp16 normal range,
    so the error stays within the bar."""
    h = H()
    w = _scaled_values(generate(cfg_id, **kw), factor)
    _say(f"value scale x{factor}: cfg{cfg_id} {kw}")
    cfg, params, cache = h.build(w)
    err = _decode_err(w, cfg, params, cache)
    _say(f"worst normwise rel err {err:.3e}")
    assert err <= h.ATTN_TOL


@pytest.mark.parametrize("cfg_id,kw", [(1, dict(length=3001)), (1, dict(length=2100, n_q_heads=32)),
                                       (1, dict(length=1000))],
                         ids=["G8", "G16", "G8-few-partials"])
def test_bf16_output_is_the_fp32_output_rounded(cfg_id, kw):
    """out_dtype = bf16 writes the fp32 result rounded to nearest even, bit for
    bit; against the oracle it is then within the bar plus bf16's own
    rounding (at most 2^-9 of each element, so of the row's largest)."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(cfg_id, **kw)
    cfg, params, cache = h.build(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    o32 = K.kvq_decode_attention(cfg, cache, params, q_rot).cpu().numpy()
    o16 = K.kvq_decode_attention(cfg, cache, params, q_rot, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16
    bits = o16.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, f64_to_bf16_bits(o32.astype(np.float64)))
    assert _decode_err(w, cfg, params, cache, torch.bfloat16) <= h.ATTN_TOL + 2.0 ** -9


def test_captured_decode_replayed_after_the_sessions_outgrow_its_plan():
    """A decode captured at 1,000 positions (four partitions of 256) and
    replayed after appends have taken the session to 20,000 positions: the
    last partition then spans 601 pages of 32 positions, past the 512 page
    entries a partition keeps in LDS, and reads the rest of its page table
    from global memory.  Replays at both lengths match the oracle."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(1, length=20000, page_tokens=32)
    cfg, params, cache = h.build(w, upto=[1000])
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = torch.empty(q_rot.shape, dtype=torch.float32, device=q_rot.device)
    ws = torch.zeros(K.kvq_decode_workspace_bytes(cfg, 1000), dtype=torch.uint8, device=q_rot.device)
    K.kvq_decode_attention(cfg, cache, params, q_rot, scale, out, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            K.kvq_decode_attention(cfg, cache, params, q_rot, scale, out, ws)
    torch.cuda.synchronize()
    q64 = O.as_f64(w.q, w.dtype)
    for n in (1000, 9000, 20000):
        h.append_range(cfg, cache, params, w, 0, int(cache.lengths()[0]), n, chunks=[4096])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, q64, [0], scale)
        err = float(h.normwise_rel_err(got[0], ref[0]).max())
        _say(f"replay at {n} positions: worst normwise rel err {err:.3e}")
        assert err <= h.ATTN_TOL


def test_one_workspace_serves_successive_decodes_of_different_shapes():
    """One workspace reused by decodes of three different configurations
    (twice each) gives bitwise the outputs of fresh workspaces: nothing a
    decode reads from it is left over from an earlier decode."""
    import decode_attention_kvq_amd as K
    h = H()
    shapes = [(2, dict(length=9000)), (3, dict(batch=3, len_range=(700, 2600))), (1, dict(length=2100, n_q_heads=32))]
    built = []
    need = 0
    for cfg_id, kw in shapes:
        w = generate(cfg_id, **kw)
        cfg, params, cache = h.build(w)
        q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
        built.append((cfg, params, cache, q_rot))
        need = max(need, K.kvq_decode_workspace_bytes(cfg, max(cache.lengths())))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")      # stale bytes: a large float pattern
    for rep in range(2):
        for cfg, params, cache, q_rot in built:
            ref = K.kvq_decode_attention(cfg, cache, params, q_rot)
            got = K.kvq_decode_attention(cfg, cache, params, q_rot, workspace=ws)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))


def test_stream_read_probe_reads_every_word():
    """The measurement probe reads every 16-byte chunk exactly once: the XOR
    of its per-workgroup words equals the XOR of the whole buffer, for several
    grid sizes and a length that is not a multiple of the grid."""
    import decode_attention_kvq_amd as K
    rng = np.random.default_rng(5)
    n = 4 * (3 * 1024 * 1024 + 37)                  # int32 words, 16-byte multiple
    host = rng.integers(-2**31, 2**31 - 1, size=n, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    ref = int(np.bitwise_xor.reduce(host.view(np.uint32)))
    for wgs in (1, 7, 256, 2048):
        sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
        K.kvq_probe_stream_read(buf, sink, wgs)
        torch.cuda.synchronize()
        got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
        assert got == ref, wgs


PLAN_CASES = [
    # (overrides, starting lengths or None): 130 sessions take the uniform
    # plan (one partition count for all); a few very unequal sessions take
    # partition counts of their own (the 20,000-position one gets most)
    (dict(batch=130, len_range=(40, 400), page_tokens=64), None),
    (dict(batch=5, len_range=(20000, 20000)), [0, 31, 19999, 700, 64]),
]


@pytest.mark.parametrize("kw,start", PLAN_CASES, ids=["uniform-130-sessions", "ragged-5-sessions"])
def test_decode_and_step_across_partition_plans(kw, start):
    """The decode and the fused step over both kinds of partition plan:
    against the oracle attending over the GPU's codes (every session), and
    the step against the two calls it stands for (1e-3, see
    tests/test_gpu_step.py)."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(3, **kw)
    B = w.cfg.batch
    upto = [int(x) - 1 for x in w.lengths] if start is None else start
    _say(f"plan case {kw} from {upto if start else 'lengths - 1'}")
    cfg, params, sep = h.build(w, upto=upto)
    _, _, fus = h.build(w, upto=upto)
    scale = h.default_scale(w)
    q = h.query_tensor(w)
    q64 = O.as_f64(w.q, w.dtype)
    # the decode over the starting lengths
    q_rot = K.kvq_rotate_query(cfg, params, q)
    out = K.kvq_decode_attention(cfg, sep, params, q_rot, scale).cpu().numpy().astype(np.float64)
    ref = h.oracle_decode_over_gpu_codes(w, cfg, sep, q64, range(B), scale, threads=16)
    err = max(float(h.normwise_rel_err(out[b], ref[b]).max()) for b in range(B) if upto[b] > 0)
    _say(f"decode worst normwise rel err {err:.3e}")
    assert err <= h.ATTN_TOL
    # one step: append position upto[b] of every session
    k = torch.cat([h._kv_tensor(w.k[b][None, upto[b]:upto[b] + 1], w.dtype) for b in range(B)])
    v = torch.cat([h._kv_tensor(w.v[b][None, upto[b]:upto[b] + 1], w.dtype) for b in range(B)])
    m = torch.from_numpy(np.stack([w.modality[b][upto[b]:upto[b] + 1] for b in range(B)])).cuda()
    q_sep = K.kvq_append_and_rotate(cfg, sep, params, k, v, m, q)
    o_sep = K.kvq_decode_attention(cfg, sep, params, q_sep, scale).cpu().numpy().astype(np.float64)
    o_fus = K.kvq_decode_step(cfg, fus, params, k, v, m, q, scale=scale).cpu().numpy().astype(np.float64)
    twin = max(float(h.normwise_rel_err(o_fus[b], o_sep[b]).max()) for b in range(B))
    _say(f"step: fused vs two calls worst normwise difference {twin:.2e}")
    assert twin <= 1e-3
    a, c = sep.host_arrays(), fus.host_arrays()
    for key in ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "seq_len", "k_tail"):
        np.testing.assert_array_equal(a[key], c[key], err_msg=key)
    ref = h.oracle_decode_over_gpu_codes(w, cfg, fus, q64, range(B), scale, threads=16)
    err = max(float(h.normwise_rel_err(o_fus[b], ref[b]).max()) for b in range(B))
    _say(f"step worst normwise rel err {err:.3e}")
    assert err <= h.ATTN_TOL
