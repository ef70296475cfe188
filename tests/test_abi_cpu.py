"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import decode_attention_kvq_amd._lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return L, L.load()


def _declared():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:kvq_status|size_t|const char\*)\s+(kvq_\w+)\s*\(", src, re.M)))


def test_header_declares_the_three_entry_points():
    names = _declared()
    for n in ("kvq_quantize_append", "kvq_rotate_query", "kvq_decode_attention"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L, lib = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(L.EXPORTED) == set(_declared())


def _cfg(L, **kw):
    base = dict(head_dim=128, n_q_heads=16, n_kv_heads=2, batch=2, page_tokens=256, max_pages=4,
                num_pages=8, kv_dtype=L.KVQ_BF16, key_mode=L.KVQ_KEYS_GROUP_MINMAX, bits=2)
    base.update(kw)
    return L.KvqConfig(*[base[f] for f, _ in L.KvqConfig._fields_])


def _fake_params(L, codebook=(-1.5104, -0.4528, 0.4528, 1.5104)):
    return L.KvqParams(0x1000, 0x2000, (ctypes.c_float * 16)(*codebook, *([0.0] * (16 - len(codebook)))))


def _fake_cache(L, lengths):
    arr = (ctypes.c_int32 * len(lengths))(*lengths)
    c = L.KvqCache(*([0x1000] * 9), arr)
    return c, arr


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2), (dict(head_dim=256), 2), (dict(n_q_heads=15), 1),
    (dict(n_q_heads=34, n_kv_heads=2), 2), (dict(page_tokens=100), 1), (dict(batch=0), 1),
    (dict(kv_dtype=7), 2), (dict(max_pages=0), 1), (dict(key_mode=2), 1), (dict(key_mode=-1), 1),
    (dict(bits=1), 2), (dict(bits=5), 2), (dict(bits=8), 2),
])
def test_config_validation(kw, status):
    L, lib = _lib()
    out = (ctypes.c_size_t * 6)()
    assert lib.kvq_cache_buffer_bytes(ctypes.byref(_cfg(L, **kw)), out) == status


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_buffer_sizes(bits):
    L, lib = _lib()
    out = (ctypes.c_size_t * 6)()
    assert lib.kvq_cache_buffer_bytes(ctypes.byref(_cfg(L, bits=bits)), out) == 0
    groups = 8 * 2 * 8
    code = groups * 4 * bits * 128                       # 4 b d bytes per group block
    assert list(out) == [code, groups * 512, code, 8 * 2 * 256 * 2, 8 * 256, 2 * 2 * 32 * 128 * 2]


def test_codebook_must_increase_over_its_2_to_the_bits_levels():
    L, lib = _lib()
    c, lens = _fake_cache(L, [0, 0])
    ok8 = _fake_params(L, tuple(float(x) for x in range(-4, 4)))
    bad8 = _fake_params(L, (-3.0, -2.0, -1.0, 0.0, 0.5, 0.4, 2.0, 3.0))
    short = _fake_params(L)                                         # 4 levels, then zeros
    for p, st in [(ok8, 0), (bad8, 1), (short, 1)]:
        cfg = _cfg(L, bits=3)
        # an empty append validates every argument and launches nothing
        assert lib.kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(p), 0, 2, 0,
                                       ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8), None) == st


def test_append_rejects_bad_arguments_without_launching():
    L, lib = _lib()
    cfg = _cfg(L)
    p = _fake_params(L)
    c, lens = _fake_cache(L, [0, 1000])
    args = lambda b0, nb, n: (ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(p), b0, nb, n,
                              ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8), None)
    assert lib.kvq_quantize_append(*args(0, 3, 1)) == L.KVQ_ERR_INVALID          # sessions out of range
    assert lib.kvq_quantize_append(*args(-1, 1, 1)) == L.KVQ_ERR_INVALID
    assert lib.kvq_quantize_append(*args(0, 1, -5)) == L.KVQ_ERR_INVALID
    assert lib.kvq_quantize_append(*args(1, 1, 25)) == L.KVQ_ERR_CAPACITY        # 1000 + 25 > 4 * 256
    assert list(lens) == [0, 1000]                                                # no state change
    assert lib.kvq_quantize_append(*args(0, 2, 0)) == L.KVQ_OK                    # empty append: no-op
    bad = _fake_params(L, (-1.0, 0.5, 0.2, 1.0))
    assert lib.kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(bad), 0, 1, 1,
                                   ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8), None) == 1
    assert lib.kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(p), 0, 1, 4,
                                   None, ctypes.c_void_p(8), ctypes.c_void_p(8), None) == 1
    nulls = L.KvqCache(0, *([0x1000] * 8), lens)
    assert lib.kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(nulls), ctypes.byref(p), 0, 1, 1,
                                   ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8), None) == 1
    no_tickets = L.KvqCache(*([0x1000] * 8), 0, lens)
    assert lib.kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(no_tickets), ctypes.byref(p), 0, 1, 1,
                                   ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8), None) == 1


def test_decode_and_rotate_reject_bad_arguments():
    L, lib = _lib()
    cfg = _cfg(L)
    p = _fake_params(L)
    c, lens = _fake_cache(L, [10, 1000])
    need = lib.kvq_decode_workspace_bytes(ctypes.byref(cfg), 1000)
    assert need > 0
    dec = lambda ws, nbytes, scale=0.1, od=L.KVQ_F32: lib.kvq_decode_attention(
        ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(p), ctypes.c_void_p(8), ctypes.c_float(scale),
        ctypes.c_void_p(8), od, ws, nbytes, None)
    assert dec(None, need) == L.KVQ_ERR_WORKSPACE
    assert dec(ctypes.c_void_p(8), need, od=7) == L.KVQ_ERR_UNSUPPORTED          # output dtype
    assert dec(ctypes.c_void_p(8), 64) == L.KVQ_ERR_WORKSPACE                    # below any plan's partials
    assert dec(ctypes.c_void_p(8), need, float("nan")) == L.KVQ_ERR_INVALID
    lens[1] = 5000                                                                # beyond capacity
    assert dec(ctypes.c_void_p(8), 1 << 30) == L.KVQ_ERR_INVALID
    assert lib.kvq_rotate_query(ctypes.byref(cfg), ctypes.byref(p), 0, ctypes.c_void_p(8), 0,
                                ctypes.c_void_p(8), None) == L.KVQ_ERR_INVALID
    assert lib.kvq_rotate_query(ctypes.byref(cfg), ctypes.byref(p), 1, ctypes.c_void_p(8), 9,
                                ctypes.c_void_p(8), None) == L.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_rotate_query(ctypes.byref(cfg), None, 1, ctypes.c_void_p(8), 0,
                                ctypes.c_void_p(8), None) == L.KVQ_ERR_INVALID
    for s in range(6):
        assert lib.kvq_status_string(s)


def test_noalloc_decode_rejects_before_launch():
    """The no-allocation decode checks its arguments, then the size of the
    partials against the static scratch, on the host: a plan needing more
    than KVQ_NOALLOC_SCRATCH_BYTES returns KVQ_ERR_SCRATCH with no launch and
    no device call (this host has no GPU)."""
    L, lib = _lib()
    p = _fake_params(L)
    V = ctypes.c_void_p
    call = lambda cfg, c, od=L.KVQ_F32: lib.kvq_decode_attention_noalloc(
        ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(p), V(8), ctypes.c_float(0.1), V(8), od, None)
    big = _cfg(L, batch=128, n_q_heads=128, n_kv_heads=8, max_pages=256, num_pages=128 * 256)
    c, lens = _fake_cache(L, [65536] * 128)
    # 128 sessions x 128 query heads x 1 partition x (8 + 3 * 128) floats = 25.7 MB > 16 MiB
    assert call(big, c) == L.KVQ_ERR_SCRATCH
    assert call(big, c, od=9) == L.KVQ_ERR_UNSUPPORTED
    lens[3] = -1
    assert call(big, c) == L.KVQ_ERR_INVALID
    assert lib.kvq_status_string(L.KVQ_ERR_SCRATCH)


def test_append_and_rotate_rejects_bad_arguments_before_launch():
    """The fused call checks both halves on the host; a failure in either
    launches nothing and leaves the length mirror untouched."""
    L, lib = _lib()
    cfg = _cfg(L)
    p = _fake_params(L)
    c, lens = _fake_cache(L, [10, 20])
    V = ctypes.c_void_p

    def call(b0=0, nb=1, n_new=1, k=V(8), v=V(8), m=V(8), batch=2, q=V(8), qd=0, qr=V(8), params=p):
        return lib.kvq_append_and_rotate(ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(params) if params else None,
                                         b0, nb, n_new, k, v, m, batch, q, qd, qr, None)
    assert call(k=None) == L.KVQ_ERR_INVALID                 # append half
    assert call(b0=1, nb=2) == L.KVQ_ERR_INVALID
    assert call(n_new=-1) == L.KVQ_ERR_INVALID
    assert call(n_new=4 * 256) == L.KVQ_ERR_CAPACITY
    assert call(q=None) == L.KVQ_ERR_INVALID                 # rotation half
    assert call(qr=None) == L.KVQ_ERR_INVALID
    assert call(batch=0) == L.KVQ_ERR_INVALID
    assert call(qd=7) == L.KVQ_ERR_UNSUPPORTED
    assert call(params=None) == L.KVQ_ERR_INVALID
    assert list(lens) == [10, 20]


def test_decode_step_rejects_bad_arguments_before_launch():
    """The fused decode step checks the append, the rotation and the decode on
    the host; a failure launches nothing and leaves the length mirror as it
    was.  Its workspace covers the partials, the open group's included, and
    a workspace sized for a length serves every shorter one."""
    L, lib = _lib()
    cfg = _cfg(L)                                   # G = 8, 256-position pages, bf16: the two-launch path
    p = _fake_params(L)
    c, lens = _fake_cache(L, [10, 700])
    V = ctypes.c_void_p
    need = lib.kvq_decode_step_workspace_bytes(ctypes.byref(cfg), 701)
    # per (session, query head): the partials of at least one partition and
    # the open group's
    assert need >= 2 * 16 * 2 * (8 + 3 * 128) * 4
    assert all(lib.kvq_decode_step_workspace_bytes(ctypes.byref(cfg), n) <= need for n in (0, 1, 33, 256, 700))

    def call(k=V(8), v=V(8), m=V(8), q=V(8), qd=L.KVQ_BF16, qr=V(8), scale=0.1, out=V(8), od=L.KVQ_F32,
             ws=V(8), nbytes=need, params=p):
        return lib.kvq_decode_step(ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(params) if params else None,
                                   k, v, m, q, qd, qr, ctypes.c_float(scale), out, od, ws, nbytes, None)
    assert call(ws=None) == L.KVQ_ERR_WORKSPACE
    assert call(nbytes=64) == L.KVQ_ERR_WORKSPACE
    assert call(k=None) == L.KVQ_ERR_INVALID
    assert call(m=None) == L.KVQ_ERR_INVALID
    assert call(q=None) == L.KVQ_ERR_INVALID
    assert call(qr=None) == L.KVQ_ERR_INVALID
    assert call(out=None) == L.KVQ_ERR_INVALID
    assert call(scale=float("inf")) == L.KVQ_ERR_INVALID
    assert call(qd=7) == L.KVQ_ERR_UNSUPPORTED
    assert call(od=7) == L.KVQ_ERR_UNSUPPORTED
    assert call(params=None) == L.KVQ_ERR_INVALID
    lens[1] = 4 * 256                               # a full session: no room for the step's position
    assert call() == L.KVQ_ERR_CAPACITY
    lens[1] = 700
    assert list(lens) == [10, 700]


def test_binding_refuses_cpu_tensors():
    import torch
    import decode_attention_kvq_amd as K
    _lib()
    cfg = K.Config(64, 2, 1, 1, 256, 8, 8, torch.float32)
    with pytest.raises(TypeError):
        K.Params(torch.ones(1, 64, dtype=torch.int8), torch.zeros(1, 3, 64, 64), [-1.5, -0.5, 0.5, 1.5])


def test_calibration_rejects_bad_arguments_without_launching():
    L, lib = _lib()
    V = ctypes.c_void_p

    def shape(**kw):
        f = dict(head_dim=128, n_q_heads=16, n_kv_heads=2, n_tokens=1000, n_queries=4)
        f.update(kw)
        return L.KvqCalibShape(*[f[name] for name, _ in L.KvqCalibShape._fields_])
    good = shape()
    need = lib.kvq_calib_workspace_bytes(ctypes.byref(good))
    # the Jacobi rotation log, (c, s) per (sweep, round, pair); then, each region 256-byte aligned, the
    # round counts, the eigenvalues and V^T of the 6 matrices
    eig_need = 6 * 50 * 127 * 64 * 16 + 256 + 6 * 128 * 8 + 6 * 128 * 128 * 8
    assert need >= lib.kvq_calib_eigenbasis_workspace_bytes(6, 128) == eig_need
    assert lib.kvq_calib_workspace_bytes(ctypes.byref(shape(head_dim=96))) == 0
    assert lib.kvq_calib_eigenbasis_workspace_bytes(-1, 128) == 0
    for kw, status in [(dict(head_dim=96), 2), (dict(n_q_heads=15), 1), (dict(n_tokens=-1), 1),
                       (dict(n_queries=0), 1), (dict(n_kv_heads=0), 1)]:
        s_ = shape(**kw)
        assert lib.kvq_calib_contribution(ctypes.byref(s_), V(8), 1, V(8), 1, 0.1, V(8), V(8), need, None) == status
        assert lib.kvq_calib_covariance(ctypes.byref(s_), V(8), 1, V(8), V(8), V(8), V(8), V(8), need, None) == status
    con = lambda **kw: lib.kvq_calib_contribution(
        ctypes.byref(kw.pop("shape", good)), kw.pop("k", V(8)), kw.pop("kd", 1), kw.pop("q", V(8)), kw.pop("qd", 1),
        kw.pop("scale", 0.1), kw.pop("w", V(8)), kw.pop("ws", V(8)), kw.pop("nbytes", need), None)
    assert con(kd=5) == L.KVQ_ERR_UNSUPPORTED
    assert con(scale=0.0) == L.KVQ_ERR_INVALID
    assert con(scale=float("inf")) == L.KVQ_ERR_INVALID
    assert con(q=None) == L.KVQ_ERR_INVALID
    assert con(ws=None) == L.KVQ_ERR_WORKSPACE
    assert con(nbytes=16) == L.KVQ_ERR_WORKSPACE
    assert con(shape=shape(n_tokens=0), k=None, q=None, w=None) == L.KVQ_OK      # nothing to do
    cov = lambda **kw: lib.kvq_calib_covariance(
        ctypes.byref(good), kw.pop("v", V(16)), kw.pop("vd", 0), kw.pop("m", V(8)), kw.pop("w", V(8)),
        kw.pop("c", V(8)), kw.pop("s", V(8)), kw.pop("ws", V(8)), kw.pop("nbytes", need), None)
    assert cov(vd=3) == L.KVQ_ERR_UNSUPPORTED
    assert cov(m=None) == L.KVQ_ERR_INVALID and cov(c=None) == L.KVQ_ERR_INVALID and cov(s=None) == L.KVQ_ERR_INVALID
    assert cov(nbytes=1) == L.KVQ_ERR_WORKSPACE
    assert cov(v=V(24)) == L.KVQ_ERR_INVALID                                      # v read in 16-byte pieces
    eig = lambda count=6, d=128, c=V(8), r=V(8), e=V(8), ws=V(16), nbytes=need: lib.kvq_calib_eigenbasis(
        count, d, c, r, e, ws, nbytes, None)
    assert eig(count=-1) == L.KVQ_ERR_INVALID
    assert eig(d=32) == L.KVQ_ERR_UNSUPPORTED
    assert eig(r=None) == L.KVQ_ERR_INVALID
    assert eig(nbytes=eig_need - 1) == L.KVQ_ERR_WORKSPACE
    assert eig(ws=V(24)) == L.KVQ_ERR_INVALID                                     # (c, s) read in 16-byte pieces
    assert eig(count=0, c=None, r=None, e=None) == L.KVQ_OK                       # nothing to do
