"""Host-side readers of the packed cache layout documented in include/kvq.h.

They turn the lane-major 2-bit group blocks, the paged statistics, norms and
modality bytes of one session back into logical per-position arrays
(codes [L, d], lo/hi [ceil(L/32), d] fp16, norms [L] fp16, modality [L]).
Pure index bookkeeping: no quantization arithmetic.
"""
from __future__ import annotations

from functools import lru_cache

import numpy as np

GROUP = 32


@lru_cache(maxsize=None)
def _key_index(d: int):
    w = d // 8
    t = np.arange(GROUP)[:, None]
    c = np.arange(d)[None, :]
    lane = ((c % 32) // 8) * 16 + t % 16
    byte = lane * w + (t // 16) * (d // 16) + (c // 32) * 2 + (c % 8) // 4
    return byte, 2 * (c % 4) + 0 * t


@lru_cache(maxsize=None)
def _value_index(d: int):
    w = d // 8
    t = np.arange(GROUP)[:, None]
    c = np.arange(d)[None, :]
    lane = ((t % 16) // 4) * 16 + c % 16
    byte = lane * w + (c // 16) * 2 + t // 16
    return byte, 2 * (t % 4) + 0 * c


def unpack_key_blocks(blocks: np.ndarray, d: int) -> np.ndarray:
    """blocks [..., 8d] uint8 -> codes [..., 32, d]."""
    byte, shift = _key_index(d)
    return ((blocks[..., byte] >> shift) & 3).astype(np.uint8)


def unpack_value_blocks(blocks: np.ndarray, d: int) -> np.ndarray:
    byte, shift = _value_index(d)
    return ((blocks[..., byte] >> shift) & 3).astype(np.uint8)


def pack_key_codes(codes: np.ndarray, d: int) -> np.ndarray:
    """codes [..., 32, d] -> blocks [..., 8d] (inverse of unpack_key_blocks)."""
    byte, shift = _key_index(d)
    out = np.zeros(codes.shape[:-2] + (8 * d,), np.uint8)
    flat = out.reshape(-1, 8 * d)
    cf = codes.reshape(-1, GROUP, d).astype(np.uint32)
    for i in range(flat.shape[0]):
        np.bitwise_or.at(flat[i], byte.ravel(), (cf[i] << shift).ravel().astype(np.uint8))
    return out


def session_view(host: dict, cfg, b: int, length: int, h: int) -> dict:
    """Logical arrays of session b, KV head h, from Cache.host_arrays().

    A logical page whose page-table entry is negative is not retained: its
    positions read as physical page 0 here and are False in `retained`."""
    d, hkv, pt = cfg.head_dim, cfg.n_kv_heads, cfg.page_tokens
    gp = pt // GROUP
    npg = -(-length // pt)
    mapped = host["page_table"][b, :npg].astype(np.int64)
    pages = np.maximum(mapped, 0)
    kb = host["k_codes"].reshape(-1, hkv, gp, 8 * d)[pages, h]          # [npg, gp, 8d]
    vb = host["v_codes"].reshape(-1, hkv, gp, 8 * d)[pages, h]
    st = host["k_stats"].reshape(-1, hkv, gp, 2, d)[pages, h]           # [npg, gp, 2, d]
    nr = host["v_norms"].reshape(-1, hkv, pt)[pages, h]                 # [npg, pt]
    md = host["modality"].reshape(-1, pt)[pages]
    ng = -(-length // GROUP)
    kc = unpack_key_blocks(kb, d).reshape(-1, d)[:length]
    vc = unpack_value_blocks(vb, d).reshape(-1, d)[:length]
    st = st.reshape(-1, 2, d)[:ng]
    # per-token key mode: the group's key norms are the first 32 entries of row 0
    k_norms = st[:, 0, :GROUP].reshape(-1)[:length].copy().view(np.float16)
    return dict(k_codes=kc, v_codes=vc, k_norms=k_norms,
                lo=st[:, 0].copy().view(np.float16), hi=st[:, 1].copy().view(np.float16),
                norms=nr.reshape(-1)[:length].copy().view(np.float16),
                modality=md.reshape(-1)[:length].copy(),
                retained=np.repeat(mapped >= 0, pt)[:length])
