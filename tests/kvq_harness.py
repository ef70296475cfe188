"""Shared plumbing of the GPU parity tests: run a seeded workload through the
HIP library and through the fp64 oracle, and compare them."""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

from omnistream import Workload


class _LazyOracle:
    """The fp64 oracle, imported on first use: the cache-building helpers
    here (used by the benchmark's GPU legs too) never load it."""

    def __getattr__(self, name):
        from oracle import kvq_oracle
        return getattr(kvq_oracle, name)


O = _LazyOracle()

ATTN_TOL = 2e-3          # max normwise relative error per (session, query head)
BOUNDARY_EPS = 1e-6      # |z - threshold| below which a code may differ
BOUNDARY_FRAC = 1e-5     # allowed fraction of such elements


def _kv_tensor(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def build(w: Workload, page_table: Optional[np.ndarray] = None, chunks: Optional[Sequence[int]] = None,
          upto: Optional[Sequence[int]] = None, num_pages: Optional[int] = None, device="cuda",
          key_mode: int = 0, rot: Optional[np.ndarray] = None):
    """Create cfg/params/cache for workload w and append every session's stream
    (split into `chunks` sized appends if given) up to `upto[b]` positions.
    The pool holds `num_pages` physical pages (default: the largest mapped one + 1).
    key_mode 1 builds a per-token-key (TurboQuant) cache; rot overrides the
    value bases [Hkv, 3, d, d]."""
    import decode_attention_kvq_amd as K
    c = w.cfg
    kv_dtype = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    pt = w.page_table if page_table is None else page_table
    num_pages = int(pt.max()) + 1 if num_pages is None else int(num_pages)
    bits = int(len(w.codebook)).bit_length() - 1          # 4, 8 or 16 levels
    cfg = K.Config(c.head_dim, c.n_q_heads, c.n_kv_heads, c.batch, w.page_tokens, pt.shape[1],
                   num_pages, kv_dtype, key_mode, bits)
    rot = w.rot if rot is None else np.ascontiguousarray(rot, dtype=np.float32)
    params = K.Params(torch.from_numpy(w.signs).to(device), torch.from_numpy(rot).to(device),
                      w.codebook.tolist())
    cache = K.Cache(cfg, torch.from_numpy(pt), device=device)
    for b in range(c.batch):
        n = int(w.lengths[b] if upto is None else upto[b])
        append_range(cfg, cache, params, w, b, 0, n, chunks)
    return cfg, params, cache


def append_range(cfg, cache, params, w: Workload, b: int, start: int, stop: int,
                 chunks: Optional[Sequence[int]] = None):
    import decode_attention_kvq_amd as K
    pos = start
    ci = 0
    while pos < stop:
        n = stop - pos if not chunks else min(int(chunks[ci % len(chunks)]), stop - pos)
        ci += 1
        k = _kv_tensor(w.k[b][None, pos:pos + n], w.dtype)
        v = _kv_tensor(w.v[b][None, pos:pos + n], w.dtype)
        m = torch.from_numpy(np.ascontiguousarray(w.modality[b][None, pos:pos + n])).to(k.device)
        K.kvq_quantize_append(cfg, cache, params, k, v, m, b0=b)
        pos += n


def query_tensor(w: Workload, device="cuda") -> torch.Tensor:
    return _kv_tensor(w.q, w.dtype, device)


def hadamard_rot(w: Workload) -> np.ndarray:
    """The TurboQuant value basis: every modality of KV head h uses the
    randomized Hadamard of h, [Hkv, 3, d, d] fp32 (an input, built by the
    stream generator)."""
    from omnistream import hadamard_value_bases
    return hadamard_value_bases(w)


def oracle_session(w: Workload, b: int, length: Optional[int] = None, key_mode: int = 0,
                   rot: Optional[np.ndarray] = None) -> list:
    n = int(w.lengths[b] if length is None else length)
    k = O.as_f64(w.k[b][:n], w.dtype)
    v = O.as_f64(w.v[b][:n], w.dtype)
    rot = w.rot if rot is None else rot
    if key_mode == 0:
        return O.quantize_session(k, v, w.modality[b][:n], w.signs, rot, w.codebook)
    out = []
    for h in range(w.cfg.n_kv_heads):
        kc, kn = O.quantize_keys_per_token(k[:, h], w.signs[h], w.codebook)
        vc, vn = O.quantize_values(v[:, h], w.modality[b][:n], rot[h], w.codebook)
        out.append(dict(k_codes=kc, k_norms=kn, v_codes=vc, norms=vn, modality=w.modality[b][:n]))
    return out


def _boundary_ok(z: np.ndarray, mism: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    dist = np.min(np.abs(z[mism][:, None] - thresholds[None, :]), axis=1)
    return dist < BOUNDARY_EPS


def _norms_mismatch(gpu_n: np.ndarray, ora_n: np.ndarray, x: np.ndarray, what: str) -> int:
    """fp16 norms may differ only where the exact norm sits on an fp16 midpoint."""
    nm = gpu_n.view(np.uint16) != ora_n.view(np.uint16)
    if nm.any():
        n64 = np.sqrt(np.sum(x * x, axis=1))[nm]
        lo_ = np.minimum(gpu_n[nm], ora_n[nm]).astype(np.float64)
        hi_ = np.maximum(gpu_n[nm], ora_n[nm]).astype(np.float64)
        mid = (lo_ + hi_) / 2
        assert np.all(np.abs(n64 - mid) <= 1e-12 * n64), f"{what} differ away from an fp16 midpoint"
    return int(nm.sum())


def compare_session_codes(w: Workload, b: int, gpu: dict, ora: list, h: int, length: int,
                          key_mode: int = 0, rot: Optional[np.ndarray] = None) -> dict:
    """Bit-exact comparison of one (session, KV head); returns counts."""
    o = ora[h]
    rot = w.rot if rot is None else rot
    stats = {}
    np.testing.assert_array_equal(gpu["modality"], w.modality[b][:length])
    thr = O.decision_thresholds(w.codebook)
    k = O.as_f64(w.k[b][:length, h], w.dtype)
    v = O.as_f64(w.v[b][:length, h], w.dtype)
    km = gpu["k_codes"] != o["k_codes"]
    knm = 0
    if key_mode == 0:
        np.testing.assert_array_equal(gpu["lo"].view(np.uint16), o["lo"].view(np.uint16), err_msg=f"LO b={b} h={h}")
        np.testing.assert_array_equal(gpu["hi"].view(np.uint16), o["hi"].view(np.uint16), err_msg=f"HI b={b} h={h}")
        if km.any():
            z = O.key_normalized_values(k, w.signs[h], o["lo"], o["hi"], w.codebook)
            ok = _boundary_ok(z, km, thr)
            assert ok.all(), f"key codes differ away from a threshold: b={b} h={h} n={int((~ok).sum())}"
    else:
        knm = _norms_mismatch(gpu["k_norms"], o["k_norms"], k, f"key norms b={b} h={h}")
        if km.any():
            z = O.key_per_token_normalized_values(k, w.signs[h])
            ok = _boundary_ok(z, km, thr)
            assert ok.all(), f"key codes differ away from a threshold: b={b} h={h} n={int((~ok).sum())}"
    vm = gpu["v_codes"] != o["v_codes"]
    if vm.any():
        z = O.value_normalized_values(v, w.modality[b][:length], rot[h])
        ok = _boundary_ok(z, vm, thr)
        assert ok.all(), f"value codes differ away from a threshold: b={b} h={h} n={int((~ok).sum())}"
    nm = _norms_mismatch(gpu["norms"], o["norms"], v, f"value norms b={b} h={h}")
    stats["elements"] = 2 * k.size
    stats["boundary_mismatches"] = int(km.sum() + vm.sum() + nm + knm)
    return stats


def _map_sessions(fn, sessions, threads: int):
    """fn over the sessions, on a pool of host threads when threads > 1 (the
    oracle's heavy steps are NumPy calls that release the interpreter lock;
    no thread touches the GPU)."""
    sessions = list(sessions)
    if threads <= 1 or len(sessions) <= 1:
        return [fn(b) for b in sessions]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, sessions))


def check_codes(w: Workload, cfg, cache, sessions: Sequence[int], lengths: Optional[Sequence[int]] = None,
                rot: Optional[np.ndarray] = None, threads: int = 1):
    from decode_attention_kvq_amd.layout import session_view
    host = cache.host_arrays()
    key_mode = getattr(cfg, "key_mode", 0)

    def one(b):
        n = int(w.lengths[b] if lengths is None else lengths[b])
        assert int(host["seq_len"][b]) == n
        ora = oracle_session(w, b, n, key_mode, rot)
        tot = mis = 0
        for h in range(w.cfg.n_kv_heads):
            gpu = session_view(host, cfg, b, n, h)
            s = compare_session_codes(w, b, gpu, ora, h, n, key_mode, rot)
            tot += s["elements"]
            mis += s["boundary_mismatches"]
        return tot, mis

    res = _map_sessions(one, sessions, threads)
    total = sum(r[0] for r in res)
    mism = sum(r[1] for r in res)
    assert mism <= BOUNDARY_FRAC * max(total, 1), f"{mism} boundary mismatches of {total}"
    return total, mism


def oracle_decode_over_gpu_codes(w: Workload, cfg, cache, q: np.ndarray, sessions: Sequence[int],
                                 scale: float, rot: Optional[np.ndarray] = None, threads: int = 1) -> dict:
    """The oracle attending over the GPU's own packed cache (codes read back),
    over the positions of the pages the page table maps (a negative entry
    marks a page that is not retained)."""
    from decode_attention_kvq_amd.layout import session_view
    host = cache.host_arrays()
    out = {}

    def one(b):
        n = int(host["seq_len"][b])
        caches = [session_view(host, cfg, b, n, h) for h in range(w.cfg.n_kv_heads)]
        keep = caches[0]["retained"] if caches else None
        q_rot = O.rotate_query(q[b], w.signs, w.cfg.n_kv_heads)
        r = w.rot if rot is None else rot
        ret = None if keep is None or keep.all() else keep
        if getattr(cfg, "key_mode", 0) == 0:
            return O.decode_attention(q_rot, caches, r, w.codebook, scale, retained=ret)
        g = w.cfg.n_q_heads // w.cfg.n_kv_heads
        return np.stack([O.decode_attention_head_per_token_keys(
            q_rot[i], caches[i // g]["k_codes"], caches[i // g]["k_norms"], caches[i // g]["v_codes"],
            caches[i // g]["norms"], caches[i // g]["modality"], r[i // g], w.codebook, scale, ret)
            for i in range(w.cfg.n_q_heads)])

    sessions = list(sessions)
    for b, o in zip(sessions, _map_sessions(one, sessions, threads)):
        out[b] = o
    return out


def normwise_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row: max_j |got - ref| / max_j |ref|."""
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return np.abs(got - ref).max(axis=-1) / den


def default_scale(w: Workload) -> float:
    return 1.0 / math.sqrt(w.cfg.head_dim)
