"""GPU parity of the TurboQuant baseline (per-token key codec) through the
same kernels, against the fp64 oracle, through the C ABI.

Bar as for the OmniKVQuant caches: key / value codes and fp16 norms
bit-exact (a code may differ only within 1e-6 of a decision threshold, a
norm only at an fp16 midpoint; fewer than 1e-5 of all elements); decode
outputs within 2e-3 normwise of the oracle attending over the GPU's codes.
The values use either the shared randomized Hadamard (the baseline) or the
per-modality bases (per-token keys with modality rotations: the ablation
between the two codecs).
"""
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


CASES = [
    # (cfg_id, overrides, value bases, append chunks)
    (0, dict(), "hadamard", None),
    (1, dict(length=3001), "hadamard", [1, 31, 100, 7]),
    (2, dict(length=5000), "hadamard", None),
    (2, dict(length=4321), "modality", [513]),
    (3, dict(batch=3, len_range=(700, 2600)), "hadamard", None),
    (4, dict(length=1500), "modality", None),
    (1, dict(length=2000, n_q_heads=8), "hadamard", None),      # G = 4: three modalities in one set
    (3, dict(batch=2, len_range=(700, 1900), page_tokens=32), "hadamard", None),
]


@pytest.mark.parametrize("cfg_id,kw,basis,chunks", CASES,
                         ids=[f"cfg{c}-{b}{'-chunked' if ch else ''}{'-' + str(sorted(kw.items())) if kw else ''}"
                              for c, kw, b, ch in CASES])
def test_per_token_append_and_decode_parity(cfg_id, kw, basis, chunks):
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(cfg_id, **kw)
    rot = h.hadamard_rot(w) if basis == "hadamard" else None
    _say(f"per-token keys cfg{cfg_id} {kw} basis={basis} chunks={chunks} lengths={w.lengths.tolist()}")
    cfg, params, cache = h.build(w, chunks=chunks, key_mode=K.KVQ_KEYS_PER_TOKEN, rot=rot)
    total, mism = h.check_codes(w, cfg, cache, range(w.cfg.batch), rot=rot)
    _say(f"codes: {total} elements, {mism} boundary mismatches")
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale).cpu().numpy()
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), range(w.cfg.batch), scale, rot=rot)
    worst = 0.0
    for b in range(w.cfg.batch):
        worst = max(worst, float(h.normwise_rel_err(out[b].astype(np.float64), ref[b]).max()))
    _say(f"decode worst normwise rel err {worst:.3e}")
    assert worst <= h.ATTN_TOL


def test_per_token_decode_over_sparse_pages():
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(1, length=4000, page_tokens=64)
    rot = h.hadamard_rot(w)
    _say("per-token keys, every other page unmapped")
    cfg, params, cache = h.build(w, key_mode=K.KVQ_KEYS_PER_TOKEN, rot=rot)
    cache.page_table[:, 1::2] = -1
    scale = h.default_scale(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    out = K.kvq_decode_attention(cfg, cache, params, q_rot, scale).cpu().numpy()
    ref = h.oracle_decode_over_gpu_codes(w, cfg, cache, O.as_f64(w.q, w.dtype), [0], scale, rot=rot)
    err = float(h.normwise_rel_err(out[0].astype(np.float64), ref[0]).max())
    _say(f"decode normwise rel err {err:.3e}")
    assert err <= h.ATTN_TOL


def test_per_token_keys_need_the_streaming_kernel():
    """G > 8 has no per-token decode: the call fails on the host, launching nothing."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(1, length=300, n_q_heads=32)
    _say("per-token keys with G = 16: unsupported")
    cfg, params, cache = h.build(w, key_mode=K.KVQ_KEYS_PER_TOKEN, rot=h.hadamard_rot(w))
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    with pytest.raises(K.KvqError) as e:
        K.kvq_decode_attention(cfg, cache, params, q_rot)
    assert e.value.status == 2


def test_key_grouping_harness_on_gpu_codes():
    """The key-grouping comparison (Sec. 3, "Key Adaptation" bullet) run
    through the kernels: for each grouping order the permuted stream is
    appended with kvq_quantize_append, and the relative error of the rotated
    keys rebuilt from the GPU's codes and statistics equals the oracle's
    harness number; the per-token (TurboQuant) key codec likewise."""
    import dataclasses

    import decode_attention_kvq_amd as K
    from decode_attention_kvq_amd.layout import session_view
    h = H()
    w = generate(2, length=16384)
    n = int(w.lengths[0])
    k64 = O.as_f64(w.k[0], w.dtype)
    for order in O.GROUP_ORDERS:
        perm = O.grouping_order(w.modality[0], order)
        wp = dataclasses.replace(w, k=[w.k[0][perm]], v=[w.v[0][perm]], modality=[w.modality[0][perm]])
        cfg, params, cache = h.build(wp)
        host = cache.host_arrays()
        for hh in range(w.cfg.n_kv_heads):
            g = session_view(host, cfg, 0, n, hh)
            y = O.randomized_hadamard(k64[perm, hh], w.signs[hh])
            y_hat = O.dequantize_keys(g["k_codes"], g["lo"], g["hi"], w.codebook)
            got = float(((y - y_hat) ** 2).sum() / (y ** 2).sum())
            ref = O.key_grouping_error(k64[:, hh], w.modality[0], w.signs[hh], w.codebook, order)
            _say(f"{order:18s} head {hh}: GPU codes {got:.6f}, oracle {ref:.6f}")
            assert abs(got - ref) <= 1e-6 * ref
    cfg, params, cache = h.build(w, key_mode=K.KVQ_KEYS_PER_TOKEN, rot=h.hadamard_rot(w))
    host = cache.host_arrays()
    for hh in range(w.cfg.n_kv_heads):
        g = session_view(host, cfg, 0, n, hh)
        y = O.randomized_hadamard(k64[:, hh], w.signs[hh])
        y_hat = O.dequantize_keys_per_token(g["k_codes"], g["k_norms"], w.codebook)
        got = float(((y - y_hat) ** 2).sum() / (y ** 2).sum())
        ref = O.per_token_key_error(k64[:, hh], w.signs[hh], w.codebook)
        _say(f"per-token keys     head {hh}: GPU codes {got:.6f}, oracle {ref:.6f}")
        assert abs(got - ref) <= 1e-6 * ref
