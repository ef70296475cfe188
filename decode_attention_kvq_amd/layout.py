"""Host-side readers of the packed cache layout documented in include/kvq.h.

They turn the lane-major 2-, 3- or 4-bit group blocks, the paged statistics, norms and
modality bytes of one session back into logical per-position arrays
(codes [L, d], lo/hi [ceil(L/32), d] fp16, norms [L] fp16, modality [L]).
Pure index bookkeeping: no quantization arithmetic.
"""
from __future__ import annotations

from functools import lru_cache

import numpy as np

GROUP = 32


# Lane-major code blocks of b bits (b = 2, 3, 4): a 32-position group block
# is 4 b d bytes, b d / 16 bytes per lane (64 lanes), each lane's bytes a
# little-endian bit stream of operand units of 8 codes (8 b bits), code k of
# unit u at bit 8 b u + b k.
#   key   (position t, channel c): lane ((c % 32) / 8) * 16 + t % 16,
#         unit (t / 16) (d / 32) + c / 32, k = c % 8
#   value (position t, channel c): lane ((t % 16) / 4) * 16 + c % 16,
#         unit c / 16, k = (t / 16) 4 + t % 4
@lru_cache(maxsize=None)
def _key_bits(d: int, bits: int):
    t = np.arange(GROUP)[:, None]
    c = np.arange(d)[None, :]
    lane = ((c % 32) // 8) * 16 + t % 16
    unit = (t // 16) * (d // 32) + c // 32
    return lane * (bits * d // 16) * 8 + 8 * bits * unit + bits * (c % 8)


@lru_cache(maxsize=None)
def _value_bits(d: int, bits: int):
    t = np.arange(GROUP)[:, None]
    c = np.arange(d)[None, :]
    lane = ((t % 16) // 4) * 16 + c % 16
    unit = c // 16
    return lane * (bits * d // 16) * 8 + 8 * bits * unit + bits * ((t // 16) * 4 + t % 4)


def _unpack(blocks: np.ndarray, pos: np.ndarray, bits: int) -> np.ndarray:
    b = blocks.astype(np.uint32)
    byte, shift = pos // 8, pos % 8
    nxt = np.minimum(byte + 1, blocks.shape[-1] - 1)
    word = b[..., byte] | (b[..., nxt] << 8)
    return ((word >> shift) & ((1 << bits) - 1)).astype(np.uint8)


def _pack(codes: np.ndarray, pos: np.ndarray, d: int, bits: int) -> np.ndarray:
    nbytes = 4 * bits * d
    out = np.zeros(codes.shape[:-2] + (nbytes,), np.uint8)
    flat = out.reshape(-1, nbytes)
    cf = codes.reshape(-1, GROUP, d).astype(np.uint32)
    byte, shift = (pos // 8).ravel(), (pos % 8).ravel()
    for i in range(flat.shape[0]):
        v = cf[i].ravel() << shift
        np.bitwise_or.at(flat[i], byte, (v & 0xFF).astype(np.uint8))
        hi = v >> 8
        m = hi > 0
        np.bitwise_or.at(flat[i], byte[m] + 1, hi[m].astype(np.uint8))
    return out


def unpack_key_blocks(blocks: np.ndarray, d: int, bits: int = 2) -> np.ndarray:
    """blocks [..., 4 b d] uint8 -> codes [..., 32, d]."""
    return _unpack(blocks, _key_bits(d, bits), bits)


def unpack_value_blocks(blocks: np.ndarray, d: int, bits: int = 2) -> np.ndarray:
    return _unpack(blocks, _value_bits(d, bits), bits)


def pack_key_codes(codes: np.ndarray, d: int, bits: int = 2) -> np.ndarray:
    """codes [..., 32, d] -> blocks [..., 4 b d] (inverse of unpack_key_blocks)."""
    return _pack(codes, _key_bits(d, bits), d, bits)


def pack_value_codes(codes: np.ndarray, d: int, bits: int = 2) -> np.ndarray:
    return _pack(codes, _value_bits(d, bits), d, bits)


def session_view(host: dict, cfg, b: int, length: int, h: int) -> dict:
    """Logical arrays of session b, KV head h, from Cache.host_arrays().

    A logical page whose page-table entry is negative is not retained: its
    positions read as physical page 0 here and are False in `retained`."""
    d, hkv, pt = cfg.head_dim, cfg.n_kv_heads, cfg.page_tokens
    bits = getattr(cfg, "bits", 2)
    gp = pt // GROUP
    npg = -(-length // pt)
    mapped = host["page_table"][b, :npg].astype(np.int64)
    pages = np.maximum(mapped, 0)
    kb = host["k_codes"].reshape(-1, hkv, gp, 4 * bits * d)[pages, h]   # [npg, gp, 4 b d]
    vb = host["v_codes"].reshape(-1, hkv, gp, 4 * bits * d)[pages, h]
    st = host["k_stats"].reshape(-1, hkv, gp, 2, d)[pages, h]           # [npg, gp, 2, d]
    nr = host["v_norms"].reshape(-1, hkv, pt)[pages, h]                 # [npg, pt]
    md = host["modality"].reshape(-1, pt)[pages]
    ng = -(-length // GROUP)
    kc = unpack_key_blocks(kb, d, bits).reshape(-1, d)[:length]
    vc = unpack_value_blocks(vb, d, bits).reshape(-1, d)[:length]
    st = st.reshape(-1, 2, d)[:ng]
    # per-token key mode: the group's key norms are the first 32 entries of row 0
    k_norms = st[:, 0, :GROUP].reshape(-1)[:length].copy().view(np.float16)
    return dict(k_codes=kc, v_codes=vc, k_norms=k_norms,
                lo=st[:, 0].copy().view(np.float16), hi=st[:, 1].copy().view(np.float16),
                norms=nr.reshape(-1)[:length].copy().view(np.float16),
                modality=md.reshape(-1)[:length].copy(),
                retained=np.repeat(mapped >= 0, pt)[:length])
