"""Python binding of libkvq: rotation-based 2-bit KV-cache quantization with
fused decode attention on MI355X (gfx950).

The functions here only marshal arguments into the C ABI of include/kvq.h;
every step runs in the library's HIP kernels.  PyTorch supplies device memory
and the current stream.  There is no fallback: if libkvq.so is missing or a
tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import (KVQ_BF16, KVQ_F32, KVQ_KEYS_GROUP_MINMAX, KVQ_KEYS_PER_TOKEN, KvqCache,  # noqa: F401
                   KvqCalibShape, KvqConfig, KvqError, KvqParams)

__all__ = ["Config", "Params", "Cache", "kvq_quantize_append", "kvq_rotate_query", "kvq_append_and_rotate",
           "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_decode_attention_noalloc",
           "kvq_decode_step_workspace_bytes", "kvq_decode_step",
           "kvq_calib_workspace_bytes", "kvq_probe_stream_read",
           "kvq_calib_eigenbasis_workspace_bytes", "kvq_calib_contribution", "kvq_calib_covariance",
           "kvq_calib_eigenbasis", "KvqError"]

_DTYPES = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class Config:
    """Shapes of one packed cache (mirrors kvq_config).  key_mode selects the
    key codec: KVQ_KEYS_GROUP_MINMAX (OmniKVQuant) or KVQ_KEYS_PER_TOKEN (the
    TurboQuant baseline)."""

    def __init__(self, head_dim: int, n_q_heads: int, n_kv_heads: int, batch: int,
                 page_tokens: int, max_pages: int, num_pages: int, kv_dtype: torch.dtype,
                 key_mode: int = KVQ_KEYS_GROUP_MINMAX, bits: int = 2):
        self.head_dim, self.n_q_heads, self.n_kv_heads = head_dim, n_q_heads, n_kv_heads
        self.batch, self.page_tokens, self.max_pages, self.num_pages = batch, page_tokens, max_pages, num_pages
        self.kv_dtype, self.key_mode, self.bits = kv_dtype, int(key_mode), int(bits)
        self.struct = KvqConfig(head_dim, n_q_heads, n_kv_heads, batch, page_tokens, max_pages,
                                num_pages, _DTYPES[kv_dtype], self.key_mode, self.bits)

    def buffer_bytes(self) -> list:
        out = (ctypes.c_size_t * 6)()
        _lib.check("kvq_cache_buffer_bytes", _lib.load().kvq_cache_buffer_bytes(ctypes.byref(self.struct), out))
        return list(out)


class Params:
    """Hadamard signs [Hkv, d] int8, value bases [Hkv, 3, d, d] fp32, and the
    2^bits codebook levels (at most 16)."""

    def __init__(self, signs: torch.Tensor, rot: torch.Tensor, codebook: Sequence[float]):
        self.signs, self.rot = signs, rot
        self.codebook = [float(c) for c in codebook]
        if not 1 <= len(self.codebook) <= 16:
            raise ValueError("the codebook holds 4, 8 or 16 levels")
        padded = self.codebook + [0.0] * (16 - len(self.codebook))
        self.struct = KvqParams(_dev(signs, "signs", torch.int8), _dev(rot, "rot", torch.float32),
                                (ctypes.c_float * 16)(*padded))


class Cache:
    """Caller-owned packed cache buffers (allocated with torch) + length mirror."""

    def __init__(self, cfg: Config, page_table: torch.Tensor, device="cuda"):
        nbytes = cfg.buffer_bytes()
        u8 = lambda n: torch.zeros(n, dtype=torch.uint8, device=device)
        self.cfg = cfg
        self.k_codes = u8(nbytes[0])
        self.k_stats = torch.zeros(nbytes[1] // 2, dtype=torch.int16, device=device)
        self.v_codes = u8(nbytes[2])
        self.v_norms = torch.zeros(nbytes[3] // 2, dtype=torch.int16, device=device)
        self.modality = u8(nbytes[4])
        self.k_tail = u8(nbytes[5])
        if tuple(page_table.shape) != (cfg.batch, cfg.max_pages):
            raise ValueError("page_table must be [batch, max_pages]")
        self.page_table = page_table.to(device=device, dtype=torch.int32).contiguous()
        self.seq_len = torch.zeros(cfg.batch, dtype=torch.int32, device=device)
        self.append_tickets = torch.zeros(cfg.batch, dtype=torch.int32, device=device)
        self.seq_len_host = (ctypes.c_int32 * cfg.batch)()
        self.struct = KvqCache(self.k_codes.data_ptr(), self.k_stats.data_ptr(), self.v_codes.data_ptr(),
                               self.v_norms.data_ptr(), self.modality.data_ptr(),
                               self.page_table.data_ptr(), self.seq_len.data_ptr(),
                               self.k_tail.data_ptr(), self.append_tickets.data_ptr(), self.seq_len_host)

    def lengths(self) -> list:
        return list(self.seq_len_host)

    def set_lengths(self, lengths: Sequence[int]) -> None:
        """Rewind (or restore) session lengths on both the device and the host mirror."""
        for b, n in enumerate(lengths):
            self.seq_len_host[b] = int(n)
        self.seq_len.copy_(torch.tensor(list(lengths), dtype=torch.int32))

    def host_arrays(self) -> dict:
        """numpy copies of every buffer (for inspection and tests)."""
        torch.cuda.synchronize()
        return dict(k_codes=self.k_codes.cpu().numpy(), k_stats=self.k_stats.cpu().numpy().view("uint16"),
                    v_codes=self.v_codes.cpu().numpy(), v_norms=self.v_norms.cpu().numpy().view("uint16"),
                    modality=self.modality.cpu().numpy(), page_table=self.page_table.cpu().numpy(),
                    seq_len=self.seq_len.cpu().numpy(), k_tail=self.k_tail.cpu().numpy())


def kvq_quantize_append(cfg: Config, cache: Cache, params: Params, k_new: torch.Tensor,
                        v_new: torch.Tensor, modality_new: torch.Tensor, b0: int = 0, stream=None) -> None:
    """k_new, v_new: [nb, n_new, Hkv, d] in cfg.kv_dtype; modality_new: [nb, n_new] uint8."""
    nb, n_new = int(k_new.shape[0]), int(k_new.shape[1])
    if tuple(k_new.shape) != (nb, n_new, cfg.n_kv_heads, cfg.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [nb, n_new, Hkv, d]")
    if tuple(modality_new.shape) != (nb, n_new):
        raise ValueError("modality_new must be [nb, n_new]")
    st = _lib.load().kvq_quantize_append(
        ctypes.byref(cfg.struct), ctypes.byref(cache.struct), ctypes.byref(params.struct), b0, nb, n_new,
        _dev(k_new, "k_new", cfg.kv_dtype), _dev(v_new, "v_new", cfg.kv_dtype),
        _dev(modality_new, "modality_new", torch.uint8), _stream(stream))
    _lib.check("kvq_quantize_append", st)


def kvq_append_and_rotate(cfg: Config, cache: Cache, params: Params, k_new: torch.Tensor,
                          v_new: torch.Tensor, modality_new: torch.Tensor, q: torch.Tensor,
                          q_rot: Optional[torch.Tensor] = None, b0: int = 0, stream=None) -> torch.Tensor:
    """kvq_quantize_append(k_new, v_new, modality_new) and kvq_rotate_query(q) in
    one launch, with identical results; returns q_rot [B, Hq, d] fp32."""
    nb, n_new = int(k_new.shape[0]), int(k_new.shape[1])
    if tuple(k_new.shape) != (nb, n_new, cfg.n_kv_heads, cfg.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [nb, n_new, Hkv, d]")
    if tuple(modality_new.shape) != (nb, n_new):
        raise ValueError("modality_new must be [nb, n_new]")
    B = int(q.shape[0])
    if tuple(q.shape) != (B, cfg.n_q_heads, cfg.head_dim):
        raise ValueError("q must be [B, Hq, d]")
    if q.dtype not in _DTYPES:
        raise TypeError("q must be float32 or bfloat16")
    if q_rot is None:
        q_rot = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    st = _lib.load().kvq_append_and_rotate(
        ctypes.byref(cfg.struct), ctypes.byref(cache.struct), ctypes.byref(params.struct), b0, nb, n_new,
        _dev(k_new, "k_new", cfg.kv_dtype), _dev(v_new, "v_new", cfg.kv_dtype),
        _dev(modality_new, "modality_new", torch.uint8), B, _dev(q, "q"), _DTYPES[q.dtype],
        _dev(q_rot, "q_rot", torch.float32), _stream(stream))
    _lib.check("kvq_append_and_rotate", st)
    return q_rot


def kvq_rotate_query(cfg: Config, params: Params, q: torch.Tensor, q_rot: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """q: [B, Hq, d] fp32 or bf16 -> q_rot [B, Hq, d] fp32."""
    B = int(q.shape[0])
    if tuple(q.shape) != (B, cfg.n_q_heads, cfg.head_dim):
        raise ValueError("q must be [B, Hq, d]")
    if q.dtype not in _DTYPES:
        raise TypeError("q must be float32 or bfloat16")
    if q_rot is None:
        q_rot = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    st = _lib.load().kvq_rotate_query(ctypes.byref(cfg.struct), ctypes.byref(params.struct), B,
                                      _dev(q, "q"), _DTYPES[q.dtype], _dev(q_rot, "q_rot", torch.float32),
                                      _stream(stream))
    _lib.check("kvq_rotate_query", st)
    return q_rot


def kvq_decode_workspace_bytes(cfg: Config, max_len: int) -> int:
    return int(_lib.load().kvq_decode_workspace_bytes(ctypes.byref(cfg.struct), int(max_len)))


def kvq_decode_attention(cfg: Config, cache: Cache, params: Params, q_rot: torch.Tensor,
                         scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None,
                         out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """q_rot: [batch, Hq, d] fp32 -> out [batch, Hq, d] in out_dtype (fp32 or
    bf16; an `out` tensor given sets the dtype)."""
    if tuple(q_rot.shape) != (cfg.batch, cfg.n_q_heads, cfg.head_dim):
        raise ValueError("q_rot must be [batch, Hq, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(cfg.head_dim)
    if out is None:
        out = torch.empty(q_rot.shape, dtype=out_dtype, device=q_rot.device)
    if out.dtype not in _DTYPES or tuple(out.shape) != tuple(q_rot.shape):
        raise ValueError("out must be [batch, Hq, d] float32 or bfloat16")
    need = kvq_decode_workspace_bytes(cfg, max(cache.lengths()))
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q_rot.device)
    st = _lib.load().kvq_decode_attention(
        ctypes.byref(cfg.struct), ctypes.byref(cache.struct), ctypes.byref(params.struct),
        _dev(q_rot, "q_rot", torch.float32), float(scale), _dev(out, "out"), _DTYPES[out.dtype],
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("kvq_decode_attention", st)
    return out


def kvq_decode_attention_noalloc(cfg: Config, cache: Cache, params: Params, q_rot: torch.Tensor,
                                 out: torch.Tensor, scale: Optional[float] = None, stream=None) -> torch.Tensor:
    """kvq_decode_attention with the partials in the library's static device
    scratch: nothing is allocated, by the library or here (the caller passes
    `out`, [batch, Hq, d] fp32 or bf16)."""
    if tuple(q_rot.shape) != (cfg.batch, cfg.n_q_heads, cfg.head_dim):
        raise ValueError("q_rot must be [batch, Hq, d]")
    if out.dtype not in _DTYPES or tuple(out.shape) != tuple(q_rot.shape):
        raise ValueError("out must be [batch, Hq, d] float32 or bfloat16")
    if scale is None:
        scale = 1.0 / math.sqrt(cfg.head_dim)
    st = _lib.load().kvq_decode_attention_noalloc(
        ctypes.byref(cfg.struct), ctypes.byref(cache.struct), ctypes.byref(params.struct),
        _dev(q_rot, "q_rot", torch.float32), float(scale), _dev(out, "out"), _DTYPES[out.dtype], _stream(stream))
    _lib.check("kvq_decode_attention_noalloc", st)
    return out


def kvq_decode_step_workspace_bytes(cfg: Config, max_len: int) -> int:
    return int(_lib.load().kvq_decode_step_workspace_bytes(ctypes.byref(cfg.struct), int(max_len)))


def kvq_decode_step(cfg: Config, cache: Cache, params: Params, k_new: torch.Tensor, v_new: torch.Tensor,
                    modality_new: torch.Tensor, q: torch.Tensor, q_rot: Optional[torch.Tensor] = None,
                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """One decode step of every session: append k_new / v_new / modality_new
    ([batch, 1, Hkv, d] in cfg.kv_dtype; [batch, 1] uint8), rotate q ([batch,
    Hq, d] fp32 or bf16) into q_rot, and attend every position including the
    new one; returns out [batch, Hq, d] in out_dtype (an `out` tensor given
    sets the dtype)."""
    B = cfg.batch
    if tuple(k_new.shape) != (B, 1, cfg.n_kv_heads, cfg.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [batch, 1, Hkv, d]")
    if tuple(modality_new.shape) != (B, 1):
        raise ValueError("modality_new must be [batch, 1]")
    if tuple(q.shape) != (B, cfg.n_q_heads, cfg.head_dim):
        raise ValueError("q must be [batch, Hq, d]")
    if q.dtype not in _DTYPES:
        raise TypeError("q must be float32 or bfloat16")
    if q_rot is None:
        q_rot = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(cfg.head_dim)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if out.dtype not in _DTYPES or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be [batch, Hq, d] float32 or bfloat16")
    if workspace is None:
        need = kvq_decode_step_workspace_bytes(cfg, max(cache.lengths()) + 1)
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    st = _lib.load().kvq_decode_step(
        ctypes.byref(cfg.struct), ctypes.byref(cache.struct), ctypes.byref(params.struct),
        _dev(k_new, "k_new", cfg.kv_dtype), _dev(v_new, "v_new", cfg.kv_dtype),
        _dev(modality_new, "modality_new", torch.uint8), _dev(q, "q"), _DTYPES[q.dtype],
        _dev(q_rot, "q_rot", torch.float32), float(scale), _dev(out, "out"), _DTYPES[out.dtype],
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("kvq_decode_step", st)
    return out


def kvq_probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int, stream=None) -> None:
    """Measurement aid: one launch reading every byte of `buf` once (see
    include/kvq.h); sink: int32 tensor of at least `workgroups` words."""
    if sink.numel() < workgroups:
        raise ValueError("sink needs one word per workgroup")
    st = _lib.load().kvq_probe_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                           _dev(sink, "sink", torch.int32), int(workgroups), _stream(stream))
    _lib.check("kvq_probe_stream_read", st)


# ------------------------------------------------------ value-basis calibration

def _calib_shape(head_dim: int, n_q_heads: int, n_kv_heads: int, n_tokens: int, n_queries: int) -> KvqCalibShape:
    return KvqCalibShape(int(head_dim), int(n_q_heads), int(n_kv_heads), int(n_tokens), int(n_queries))


def kvq_calib_workspace_bytes(head_dim: int, n_q_heads: int, n_kv_heads: int, n_tokens: int,
                              n_queries: int) -> int:
    shape = _calib_shape(head_dim, n_q_heads, n_kv_heads, n_tokens, n_queries)
    return int(_lib.load().kvq_calib_workspace_bytes(ctypes.byref(shape)))


def kvq_calib_eigenbasis_workspace_bytes(count: int, head_dim: int) -> int:
    return int(_lib.load().kvq_calib_eigenbasis_workspace_bytes(int(count), int(head_dim)))


def _workspace(need: int, workspace, device) -> torch.Tensor:
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def kvq_calib_contribution(k: torch.Tensor, q: torch.Tensor, scale: Optional[float] = None,
                           weights: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """k: [n, Hkv, d], q: [nq, Hq, d] (fp32 or bf16) -> weights [Hkv, n] fp64."""
    if k.dim() != 3 or q.dim() != 3 or k.shape[2] != q.shape[2]:
        raise ValueError("k must be [n, Hkv, d] and q [nq, Hq, d]")
    if k.dtype not in _DTYPES or q.dtype not in _DTYPES:
        raise TypeError("k and q must be float32 or bfloat16")
    n, hkv, d = (int(x) for x in k.shape)
    nq, hq = int(q.shape[0]), int(q.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    shape = _calib_shape(d, hq, hkv, n, nq)
    if weights is None:
        weights = torch.empty((hkv, n), dtype=torch.float64, device=k.device)
    workspace = _workspace(kvq_calib_workspace_bytes(d, hq, hkv, n, nq), workspace, k.device)
    st = _lib.load().kvq_calib_contribution(
        ctypes.byref(shape), _dev(k, "k"), _DTYPES[k.dtype], _dev(q, "q"), _DTYPES[q.dtype], float(scale),
        _dev(weights, "weights", torch.float64), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("kvq_calib_contribution", st)
    return weights


def kvq_calib_covariance(v: torch.Tensor, modality: torch.Tensor, weights: torch.Tensor,
                         cov: Optional[torch.Tensor] = None, weight_sum: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """v: [n, Hkv, d] (fp32 or bf16), modality: [n] uint8, weights: [Hkv, n] fp64
    -> (cov [Hkv, 3, d, d] fp64, weight_sum [Hkv, 3] fp64)."""
    if v.dim() != 3 or v.dtype not in _DTYPES:
        raise ValueError("v must be [n, Hkv, d] float32 or bfloat16")
    n, hkv, d = (int(x) for x in v.shape)
    if tuple(modality.shape) != (n,) or tuple(weights.shape) != (hkv, n):
        raise ValueError("modality must be [n] and weights [Hkv, n]")
    shape = _calib_shape(d, hkv, hkv, n, 1)
    if cov is None:
        cov = torch.empty((hkv, 3, d, d), dtype=torch.float64, device=v.device)
    if weight_sum is None:
        weight_sum = torch.empty((hkv, 3), dtype=torch.float64, device=v.device)
    workspace = _workspace(kvq_calib_workspace_bytes(d, hkv, hkv, n, 1), workspace, v.device)
    st = _lib.load().kvq_calib_covariance(
        ctypes.byref(shape), _dev(v, "v"), _DTYPES[v.dtype], _dev(modality, "modality", torch.uint8),
        _dev(weights, "weights", torch.float64), _dev(cov, "cov", torch.float64),
        _dev(weight_sum, "weight_sum", torch.float64), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("kvq_calib_covariance", st)
    return cov, weight_sum


def kvq_calib_eigenbasis(cov: torch.Tensor, rot: Optional[torch.Tensor] = None,
                         eigenvalues: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None):
    """cov: [..., d, d] fp64 symmetric -> (rot [..., d, d] fp32 with eigenvector
    columns in decreasing eigenvalue order, eigenvalues [..., d] fp64)."""
    if cov.dim() < 2 or cov.shape[-1] != cov.shape[-2]:
        raise ValueError("cov must be [..., d, d]")
    d = int(cov.shape[-1])
    count = int(cov.numel() // (d * d))
    if rot is None:
        rot = torch.empty(cov.shape, dtype=torch.float32, device=cov.device)
    if eigenvalues is None:
        eigenvalues = torch.empty(cov.shape[:-1], dtype=torch.float64, device=cov.device)
    workspace = _workspace(kvq_calib_eigenbasis_workspace_bytes(count, d), workspace, cov.device)
    st = _lib.load().kvq_calib_eigenbasis(
        count, d, _dev(cov, "cov", torch.float64), _dev(rot, "rot", torch.float32),
        _dev(eigenvalues, "eigenvalues", torch.float64), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check("kvq_calib_eigenbasis", st)
    return rot, eigenvalues
