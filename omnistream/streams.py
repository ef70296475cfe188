"""Seeded synthetic omni-modal key/value streams.

The OmniKVQuant pages evaluate on real Omni-LLM caches (Qwen2.5-Omni,
Qwen3-Omni) over audio-visual benchmarks and calibrate on VGGSound; none of
that is available here.  These generators stand in for them with the shapes
of the pages' omni workloads: interleaved video / audio / text tokens in
temporal chunks (OmniTide, Sec. 2.1 and Table 1: a few hundred to ~2,300
video tokens per frame, 10-25 audio tokens per second) and an ~80K-token
context (OmniTide, Sec. 1 / Fig. 2 profile).

Everything here is input generation: random numbers, modality labels,
page tables.  Nothing in this module quantizes, rotates for quantization,
or attends.  The value bases R_m handed to the method are the generating
eigenbases of each modality's value covariance, i.e. what the
attention-weighted per-modality calibration (OmniKVQuant, Sec. 2, values
bullet) would ideally recover.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

MOD_VIDEO, MOD_AUDIO, MOD_TEXT = 0, 1, 2

# The four fp32 reconstruction levels of the 2-bit Lloyd-Max quantizer for a
# standard normal source (the "shared fixed codebook").
_CODEBOOK_2BIT = (-1.5104, -0.4528, 0.4528, 1.5104)


def lloyd_max_codebook_2bit() -> np.ndarray:
    return np.array(_CODEBOOK_2BIT, dtype=np.float32)


def _normal_pdf(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _normal_cdf(x: float) -> float:
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def lloyd_max_codebook(bits: int) -> np.ndarray:
    """The fixed codebook for `bits`-bit codes: the 2^bits reconstruction
    levels of the Lloyd-Max quantizer for a standard normal source, as fp32
    (2 bits: the four levels above; 3 and 4 bits: Lloyd's iteration, each
    level the conditional mean of its cell, (pdf(a) - pdf(b)) / (cdf(b) -
    cdf(a)), cells split at the midpoints, run to convergence in fp64)."""
    if bits == 2:
        return lloyd_max_codebook_2bit()
    if bits not in (3, 4):
        raise ValueError("bits must be 2, 3 or 4")
    n = 1 << bits
    c = [-3.0 + 6.0 * (k + 0.5) / n for k in range(n)]
    for _ in range(100000):
        b = [(c[k] + c[k + 1]) / 2.0 for k in range(n - 1)]
        new = []
        for k in range(n):
            pa = _normal_pdf(b[k - 1]) if k > 0 else 0.0
            pb = _normal_pdf(b[k]) if k < n - 1 else 0.0
            fa = _normal_cdf(b[k - 1]) if k > 0 else 0.0
            fb = _normal_cdf(b[k]) if k < n - 1 else 1.0
            new.append((pa - pb) / (fb - fa))
        done = max(abs(x - y) for x, y in zip(new, c)) < 1e-15
        c = new
        if done:
            break
    return np.array(c, dtype=np.float32)


@dataclass(frozen=True)
class StreamConfig:
    cfg_id: int
    name: str
    head_dim: int
    n_q_heads: int
    n_kv_heads: int
    batch: int
    dtype: str                 # "f32" or "bf16" (K, V and q)
    recipe: str                # "block84", "chunk_fixed", "chunk_var"
    length: int = 0            # context length for fixed-length configs
    len_range: tuple = ()      # (lo, hi) inclusive, per-session uniform
    page_tokens: int = 256
    paged_random: bool = False
    append_tokens: int = 0     # tokens appended (and timed) after the prefix
    audio_k_scale: float = 1.0

    @property
    def group_size(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS = {
    0: StreamConfig(0, "tiny d64 2k fp32", 64, 2, 1, 1, "f32", "block84", length=2048),
    1: StreamConfig(1, "gqa16/2 d128 16k bf16", 128, 16, 2, 1, "bf16", "chunk_fixed",
                    length=16384, audio_k_scale=1.5),
    2: StreamConfig(2, "gqa28/4 d128 80k bf16", 128, 28, 4, 1, "bf16", "chunk_var",
                    length=81920, audio_k_scale=1.5),
    3: StreamConfig(3, "32 sessions paged gqa16/2 d128 8k-64k bf16", 128, 16, 2, 32, "bf16",
                    "chunk_fixed", len_range=(8192, 65536), paged_random=True,
                    audio_k_scale=1.5),
    4: StreamConfig(4, "stream loop gqa32/8 d128 128k+1k bf16", 128, 32, 8, 1, "bf16",
                    "chunk_fixed", length=131072, append_tokens=1024, audio_k_scale=1.5),
}


@dataclass
class Workload:
    cfg: StreamConfig
    signs: np.ndarray               # [Hkv, d] int8, +-1
    codebook: np.ndarray            # [4] float32
    rot: np.ndarray                 # [Hkv, 3, d, d] float32, R[h, m] (columns = basis)
    k: List[np.ndarray]             # per session [L_b, Hkv, d]  (float32, or uint16 bf16 bits)
    v: List[np.ndarray]             # per session [L_b, Hkv, d]
    modality: List[np.ndarray]      # per session [L_b] uint8
    q: np.ndarray                   # [B, Hq, d] (float32, or uint16 bf16 bits)
    lengths: np.ndarray             # [B] int64 total tokens per session (prefix + append)
    prefix_lengths: np.ndarray      # [B] tokens present before the timed append
    page_tokens: int
    max_pages: int                  # page-table row length
    num_pages: int                  # physical pages in the pool
    page_table: np.ndarray          # [B, max_pages] int32, -1 = unused
    meta: dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.cfg.dtype


# ---------------------------------------------------------------- bf16 helpers

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (via float32, round-to-nearest-even) and return the raw bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x.astype(np.float32))
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    raise ValueError(dtype)


# ------------------------------------------------------------ modality streams

def _modality_block84(n: int) -> np.ndarray:
    block = np.array([MOD_VIDEO] * 64 + [MOD_AUDIO] * 16 + [MOD_TEXT] * 4, np.uint8)
    reps = -(-n // block.size)
    return np.tile(block, reps)[:n].copy()


def _modality_chunks(rng: np.random.Generator, n: int, variable_frames: bool) -> np.ndarray:
    """1-s chunks: one video frame, its audio, then sparse text (p = 0.1, 1..16 tokens)."""
    parts = []
    total = 0
    while total < n:
        nv = int(rng.integers(640, 2305)) if variable_frames else 640
        na = int(rng.integers(10, 26)) if variable_frames else 25
        parts.append(np.full(nv, MOD_VIDEO, np.uint8))
        parts.append(np.full(na, MOD_AUDIO, np.uint8))
        total += nv + na
        if rng.random() < 0.1:
            nt = int(rng.integers(1, 17))
            parts.append(np.full(nt, MOD_TEXT, np.uint8))
            total += nt
    return np.concatenate(parts)[:n].copy()


def _append_chunk_modality(n_video=640, n_audio=25, n_text=359) -> np.ndarray:
    return np.concatenate([np.full(n_video, MOD_VIDEO, np.uint8),
                           np.full(n_audio, MOD_AUDIO, np.uint8),
                           np.full(n_text, MOD_TEXT, np.uint8)])


# ------------------------------------------------------------------ K/V draws

def _haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def _draw_keys(rng, modality, n_kv, d, audio_scale, outliers):
    """N(0,1) (audio part scaled) + per-channel random-walk mean (std-0.05 step per
    64 tokens) + two x8 outlier channels per KV head."""
    n = modality.size
    k = rng.standard_normal((n, n_kv, d))
    if audio_scale != 1.0:
        k[modality == MOD_AUDIO] *= audio_scale
    nblk = -(-n // 64)
    mu = np.cumsum(rng.normal(0.0, 0.05, size=(nblk, n_kv, d)), axis=0)
    k += mu[np.arange(n) // 64]
    for h in range(n_kv):
        k[:, h, outliers[h]] *= 8.0
    return k


def _draw_values(rng, modality, basis, lam):
    """v ~ N(0, Q_m diag(lam_m) Q_m^T) per KV head and modality."""
    n = modality.size
    n_kv, _, d, _ = basis.shape
    xi = rng.standard_normal((n, n_kv, d))
    v = np.empty_like(xi)
    for h in range(n_kv):
        for m in range(3):
            idx = modality == m
            if idx.any():
                v[idx, h] = (xi[idx, h] * np.sqrt(lam[h, m])[None, :]) @ basis[h, m].T
    return v


# ------------------------------------------------------------------- generate

def generate(cfg_id: int, length: Optional[int] = None, batch: Optional[int] = None,
             len_range: Optional[tuple] = None, append_tokens: Optional[int] = None,
             page_tokens: Optional[int] = None, n_q_heads: Optional[int] = None,
             bits: int = 2) -> Workload:
    """Build the seeded workload of one configuration.

    Overrides shrink a configuration for fast tests while keeping its recipe,
    KV heads and dtypes (n_q_heads changes only the number of queries, i.e.
    the GQA group size; bits picks the fixed codebook, 2, 3 or 4 bits).  Seeds: SeedSequence(cfg_id) spawned in the fixed
    order signs, bases, keys, values, chunking, queries, lengths/pages.
    """
    base = CONFIGS[cfg_id]
    cfg = StreamConfig(
        base.cfg_id, base.name, base.head_dim, base.n_q_heads if n_q_heads is None else n_q_heads, base.n_kv_heads,
        base.batch if batch is None else batch, base.dtype, base.recipe,
        length=base.length if length is None else length,
        len_range=base.len_range if len_range is None else len_range,
        page_tokens=base.page_tokens if page_tokens is None else page_tokens,
        paged_random=base.paged_random,
        append_tokens=base.append_tokens if append_tokens is None else append_tokens,
        audio_k_scale=base.audio_k_scale)
    d, n_kv, n_q, B = cfg.head_dim, cfg.n_kv_heads, cfg.n_q_heads, cfg.batch
    s_signs, s_rot, s_k, s_v, s_chunk, s_q, s_len = np.random.SeedSequence(cfg_id).spawn(7)

    rng = np.random.default_rng(s_signs)
    signs = np.where(rng.random((n_kv, d)) < 0.5, -1, 1).astype(np.int8)
    outliers = [np.sort(rng.choice(d, size=2, replace=False)) for _ in range(n_kv)]

    rng = np.random.default_rng(s_rot)
    basis = np.stack([np.stack([_haar_orthogonal(rng, d) for _ in range(3)]) for _ in range(n_kv)])
    lam = 10.0 ** rng.uniform(-2.0, 1.0, size=(n_kv, 3, d))
    rot = basis.astype(np.float32)

    rng = np.random.default_rng(s_len)
    if cfg.len_range:
        lo, hi = cfg.len_range
        prefix = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    else:
        prefix = np.full(B, cfg.length, np.int64)
    total = prefix + cfg.append_tokens

    k_list, v_list, m_list = [], [], []
    kss, vss, css = s_k.spawn(B), s_v.spawn(B), s_chunk.spawn(B)
    for b in range(B):
        crng = np.random.default_rng(css[b])
        n0 = int(prefix[b])
        if cfg.recipe == "block84":
            mod = _modality_block84(n0)
        else:
            mod = _modality_chunks(crng, n0, variable_frames=(cfg.recipe == "chunk_var"))
        if cfg.append_tokens:
            extra = _append_chunk_modality()
            if cfg.append_tokens != extra.size:
                extra = _modality_chunks(crng, cfg.append_tokens, False)
            mod = np.concatenate([mod, extra])
        k = _draw_keys(np.random.default_rng(kss[b]), mod, n_kv, d, cfg.audio_k_scale, outliers)
        v = _draw_values(np.random.default_rng(vss[b]), mod, basis, lam)
        k_list.append(_to_dtype(k, cfg.dtype))
        v_list.append(_to_dtype(v, cfg.dtype))
        m_list.append(mod)

    rng = np.random.default_rng(s_q)
    q = _to_dtype(rng.standard_normal((B, n_q, d)), cfg.dtype)

    # Page table: 256-token pages; a contiguous cache is the identity table.
    pt = cfg.page_tokens
    npages = [-(-int(t) // pt) for t in total]
    max_pages = max(npages)
    num_pages = int(sum(npages))
    table = np.full((B, max_pages), -1, np.int32)
    rng = np.random.default_rng(s_len.spawn(1)[0])
    pool = rng.permutation(num_pages) if cfg.paged_random else np.arange(num_pages)
    off = 0
    for b in range(B):
        table[b, :npages[b]] = pool[off:off + npages[b]]
        off += npages[b]

    return Workload(cfg=cfg, signs=signs, codebook=lloyd_max_codebook(bits), rot=rot,
                    k=k_list, v=v_list, modality=m_list, q=q, lengths=total,
                    prefix_lengths=prefix, page_tokens=pt, max_pages=max_pages,
                    num_pages=num_pages, page_table=table,
                    meta={"outlier_channels": [o.tolist() for o in outliers],
                          "value_spectrum": lam})


def sylvester_hadamard(d: int) -> np.ndarray:
    """The d x d Sylvester Hadamard matrix (entries +-1, natural order), by the
    doubling construction H_1 = [1], H_2n = [[H, H], [H, -H]] (np.kron)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1), np.int64)
    while H.shape[0] < d:
        H = np.kron(np.array([[1, 1], [1, -1]], np.int64), H)
    return H


def hadamard_value_bases(w: Workload) -> np.ndarray:
    """Value bases of the shared-rotation (TurboQuant) baseline as an input
    array [Hkv, 3, d, d] float32: every modality of KV head h gets
    R = diag(s_h) H_d / sqrt(d), so that the forward map R^T v is the
    randomized Hadamard H_d (s_h * v) / sqrt(d) of the keys.  Entries are
    +-1/sqrt(d), exact in fp32 for d = 64 and rounded once for d = 128."""
    d = w.cfg.head_dim
    H = sylvester_hadamard(d).astype(np.float64)
    out = np.empty((w.cfg.n_kv_heads, 3, d, d), np.float32)
    for h in range(w.cfg.n_kv_heads):
        R = (w.signs[h].astype(np.float64)[:, None] * H) / np.sqrt(d)
        out[h] = R.astype(np.float32)[None]
    return out


def calibration_queries(w: Workload, n_queries: int) -> np.ndarray:
    """n_queries seeded N(0, 1) query vectors per query head, [n_queries, Hq, d]
    in the workload's dtype: the queries a value-basis calibration attends
    with.  Seeded apart from the workload's own draws (entropy (cfg_id, 7))."""
    rng = np.random.default_rng(np.random.SeedSequence([w.cfg.cfg_id, 7]))
    return _to_dtype(rng.standard_normal((n_queries, w.cfg.n_q_heads, w.cfg.head_dim)), w.cfg.dtype)


def workload_digest(w: Workload) -> str:
    h = hashlib.sha256()
    for a in [w.signs, w.codebook, w.rot, w.q, w.page_table, *w.k, *w.v, *w.modality]:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
