"""GPU parity of 3- and 4-bit caches (8- and 16-level Lloyd-Max codebooks,
b-bit lane-major blocks) against the fp64 oracle, through the C ABI.

Bar as for 2 bits: codes and fp16 statistics / norms bit-exact (a code may
differ only within 1e-6 of a decision threshold, fewer than 1e-5 of all
elements); decode outputs within 2e-3 normwise of the oracle attending over
the GPU's own codes.  Ragged append chunks make the append re-read earlier
codes that straddle word boundaries (3 bits).
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
    # (bits, cfg_id, overrides, append chunks, key mode)
    (3, 0, dict(), None, 0),
    (4, 0, dict(), [1, 5, 64], 0),
    (3, 1, dict(length=3001), [1, 31, 100, 7], 0),
    (4, 1, dict(length=3001), [1, 31, 100, 7], 0),
    (3, 2, dict(length=5000), None, 0),
    (4, 2, dict(length=5000), [513], 0),
    (3, 3, dict(batch=3, len_range=(700, 2600)), None, 0),
    (4, 3, dict(batch=2, len_range=(700, 1900), page_tokens=32), None, 0),
    (3, 1, dict(length=2000, n_q_heads=8), [3, 29], 0),      # G = 4: one accumulator set
    (4, 4, dict(length=1500), None, 1),                        # per-token keys at 4 bits
    (3, 2, dict(length=2100), [77], 1),
    # the 80K workload at its full size (the widest codebook has the least
    # fp16 headroom in its levels)
    (4, 2, dict(), None, 0),
    (4, 2, dict(), None, 1),
    (3, 2, dict(), None, 0),
]


@pytest.mark.parametrize("bits,cfg_id,kw,chunks,key_mode", CASES,
                         ids=[f"b{b}-cfg{c}{'-chunked' if ch else ''}{'-tq' if km else ''}-{i}"
                              for i, (b, c, kw, ch, km) in enumerate(CASES)])
def test_wide_code_append_and_decode_parity(bits, cfg_id, kw, chunks, key_mode):
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(cfg_id, bits=bits, **kw)
    rot = h.hadamard_rot(w) if key_mode else None
    _say(f"{bits}-bit cfg{cfg_id} {kw} chunks={chunks} key_mode={key_mode} lengths={w.lengths.tolist()}")
    cfg, params, cache = h.build(w, chunks=chunks, key_mode=key_mode, rot=rot)
    assert cfg.bits == bits
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


def test_wide_codes_need_the_streaming_kernel():
    """G > 8 has no 3- / 4-bit decode: the call fails on the host."""
    import decode_attention_kvq_amd as K
    h = H()
    w = generate(1, length=300, n_q_heads=32, bits=4)
    _say("4-bit codes with G = 16: unsupported")
    cfg, params, cache = h.build(w)
    h.check_codes(w, cfg, cache, [0])                # the append itself supports every shape
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    with pytest.raises(K.KvqError) as e:
        K.kvq_decode_attention(cfg, cache, params, q_rot)
    assert e.value.status == 2
