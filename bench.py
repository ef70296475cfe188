"""Benchmark: fused 2-bit decode attention on the packed KV cache at 80K context.

One step = one decode step of one attention layer on the seeded synthetic
omni stream (81,920 cached positions, 28 query / 4 KV heads, d = 128, bf16
input): quantize-append the step's new key/value, rotate the query, and run
the fused decode over the packed cache.  Steps cycle over R layer replicas
(R x 27.8 MB > the 256 MB Infinity Cache) so that the cache is read from HBM.

Prints one JSON line (rank 0).  `value` = KV positions attended per second
(context length / time per step, inputs resident in HBM).  `roofline` is for
the decode launch (partition + merge kernels), timed with HIP events on the
stream it runs on.  `cpu_baseline` is the fp64 oracle decoding the same
packed cache on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes of one decode launch (partition + merge kernels) at this workload,
# from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), each scaled by
# what the counter reads for a plain 256 MiB device copy (FETCH_SIZE x 1.9997,
# WRITE_SIZE x 1.0); see profiles/decode_80k_hbm_bytes.md.  Valid only for
# the decode source the counters were taken on (SHA-256 of kvq_decode.hip).
DECODE_TRAFFIC = {"kvq_decode_sha256": "fb0af28a8adb44a0e86a5f4c2ab31b6e1b4d06614c0c3e0999a7add4728270a1",
                  "bytes": 34910618}


def decode_traffic_bytes():
    import hashlib
    path = os.path.join(ROOT, "decode_attention_kvq_amd", "csrc", "kvq_decode.hip")
    try:
        digest = hashlib.sha256(open(path, "rb").read()).hexdigest()
    except OSError:
        return None
    return DECODE_TRAFFIC["bytes"] if digest == DECODE_TRAFFIC["kvq_decode_sha256"] else None


def algorithmic_decode_bytes(L: int, d: int, hq: int, hkv: int) -> int:
    """Bytes one decode must move: per (position, KV head) the key codes
    (d/4), value codes (d/4), key group statistics (2 d fp16 per 32
    positions) and the value norm (fp16); one modality byte per position;
    the value bases (3 d^2 fp32 per KV head); the rotated query and output."""
    per_pos_head = d // 4 + d // 4 + (2 * d * 2) // 32 + 2
    return L * hkv * per_pos_head + L + hkv * 3 * d * d * 4 + 2 * hq * d * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--replicas", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibration-only", action="store_true",
                    help="only time the value-basis calibration on the 80K stream and print its JSON line")
    ap.add_argument("--decode-only", action="store_true",
                    help="only replay the 80K decode graph (partition + merge over the layer replicas) "
                         "--steps times and print its timing (for profiler runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB ten times (reference "
                         "for the HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by KV head with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        x = torch.ones(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(10):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 10}), flush=True)
        return
    import decode_attention_kvq_amd as K
    from omnistream import generate
    from tests import kvq_harness as H

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L0 = 81920
    if args.calibration_only:
        print(json.dumps({"value_calibration": time_calibration(L0)}), flush=True)
        return
    extra = args.steps // args.replicas + args.warmup // args.replicas + 4
    w = generate(2, length=L0 + extra)
    c = w.cfg
    d, hq, hkv = c.head_dim, c.n_q_heads, c.n_kv_heads
    pt = w.page_tokens
    max_pages = -(-(L0 + extra) // pt)
    table = np.arange(max_pages, dtype=np.int32)[None, :]
    cfg, params, cache0 = H.build(w, page_table=table, upto=[L0])
    torch.cuda.synchronize()

    # Layer replicas: identical packed caches in separate buffers.
    caches = [cache0]
    for _ in range(args.replicas - 1):
        cc = K.Cache(cfg, torch.from_numpy(table), device=dev)
        for name in ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "k_tail", "seq_len"):
            getattr(cc, name).copy_(getattr(cache0, name))
        cc.set_lengths(cache0.lengths())
        caches.append(cc)
    torch.cuda.synchronize()

    k_steps = H._kv_tensor(w.k[0][None, L0:L0 + extra], "bf16", dev)     # [1, extra, Hkv, d]
    v_steps = H._kv_tensor(w.v[0][None, L0:L0 + extra], "bf16", dev)
    m_steps = torch.from_numpy(np.ascontiguousarray(w.modality[0][None, L0:L0 + extra])).to(dev)
    q = H.query_tensor(w, dev)
    q_rot = torch.empty(q.shape, dtype=torch.float32, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(K.kvq_decode_workspace_bytes(cfg, L0 + extra), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d)

    def one_step(r, j):
        # append the step's key / value and rotate its query (one launch:
        # kvq_append_and_rotate = kvq_quantize_append + kvq_rotate_query), then decode
        cache = caches[r]
        K.kvq_append_and_rotate(cfg, cache, params, k_steps[:, j:j + 1], v_steps[:, j:j + 1], m_steps[:, j:j + 1],
                                q, q_rot)
        K.kvq_decode_attention(cfg, cache, params, q_rot, scale, out, ws)

    # Eager warm-up (also loads every kernel), then rewind the lengths.
    for r in range(args.replicas):
        one_step(r, 0)
    torch.cuda.synchronize()
    for cc in caches:
        cc.set_lengths([L0])
    torch.cuda.synchronize()

    # One graph = one decode step on each of the R layer replicas.  Replays
    # append the same new token again at the (device-side) current length, so
    # every replay is a full decode step on a cache of L0 + replay positions.
    g_step = torch.cuda.CUDAGraph()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(g_step, stream=s_cap):
            for r in range(args.replicas):
                one_step(r, 0)
    torch.cuda.synchronize()
    for cc in caches:                       # capture advanced the host mirror only
        cc.set_lengths([L0])
    torch.cuda.synchronize()

    g_dec = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(g_dec, stream=s_cap):
            for r in range(args.replicas):
                K.kvq_decode_attention(cfg, caches[r], params, q_rot, scale, out, ws)
    torch.cuda.synchronize()

    n_rep = max(1, args.steps // args.replicas)
    n_warm = max(1, args.warmup // args.replicas)
    stream = torch.cuda.current_stream()
    if args.decode_only:
        for _ in range(n_warm):
            g_dec.replay()
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(n_rep):
            g_dec.replay()
        d1.record(stream)
        torch.cuda.synchronize()
        us = d0.elapsed_time(d1) * 1e3 / (n_rep * args.replicas)
        nb = algorithmic_decode_bytes(L0, d, hq, hkv)
        print(json.dumps({"decode_only": {"context": L0, "launches": n_rep * args.replicas,
                                          "warmup_launches": n_warm * args.replicas, "avg_launch_us": us,
                                          "bytes_per_launch": nb, "GBps": nb / us / 1e3}}), flush=True)
        return
    for _ in range(n_warm):
        g_step.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(n_rep):
        g_step.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steps = n_rep * args.replicas
    ms_step = e0.elapsed_time(e1) / steps
    lens = [int(x) for cc in caches for x in cc.seq_len.cpu().tolist()]
    for cc, n in zip(caches, lens):
        cc.set_lengths([n])
    ctx_mean = float(np.mean(lens)) - (n_rep - 1) / 2.0      # mean context over the timed steps

    # Decode launches alone: R back-to-back decodes per replay, HIP events on the stream.
    for _ in range(2):
        g_dec.replay()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_dec = max(5, (2 * args.steps) // args.replicas)
    d0.record(stream)
    for _ in range(n_dec):
        g_dec.replay()
    d1.record(stream)
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / (n_dec * args.replicas)
    Ld = int(np.mean(lens))
    dec_bytes = algorithmic_decode_bytes(Ld, d, hq, hkv)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9

    # Sparse page set: every other 256-position page unmapped (page-table entry
    # -1) in every replica; the same decode graph, then the full tables again.
    for cc in caches:
        cc.page_table[:, 1::2] = -1
    g_dec.replay()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(n_dec):
        g_dec.replay()
    s1.record(stream)
    torch.cuda.synchronize()
    half_ms = s0.elapsed_time(s1) / (n_dec * args.replicas)
    for cc in caches:
        cc.page_table.copy_(torch.from_numpy(table))
    torch.cuda.synchronize()

    # Warm (Infinity-Cache resident) decode for context: one replica repeatedly.
    g_warm = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(g_warm, stream=s_cap):
            for _ in range(args.replicas):
                K.kvq_decode_attention(cfg, caches[0], params, q_rot, scale, out, ws)
    g_warm.replay()
    ew0, ew1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ew0.record(stream)
    for _ in range(10):
        g_warm.replay()
    ew1.record(stream)
    torch.cuda.synchronize()
    warm_ms = ew0.elapsed_time(ew1) / (10 * args.replicas)

    # Context: a plain device copy (read + write) of the same byte count, one
    # buffer per replica so it runs from HBM, HIP events.
    sbufs = [torch.ones(dec_bytes // 4, dtype=torch.float32, device=dev) for _ in range(args.replicas)]
    cdst = torch.empty_like(sbufs[0])
    for sb in sbufs:
        cdst.copy_(sb)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        for sb in sbufs:
            cdst.copy_(sb)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / (5 * len(sbufs))
    copy_bytes = 2 * cdst.numel() * 4
    del sbufs, cdst

    calib = time_calibration(L0)
    del g_step, g_dec, g_warm
    import decode_attention_kvq_amd as K_
    from omnistream import hadamard_value_bases
    turbo = time_variant_decode(w, table, L0, args.replicas, n_dec, scale, key_mode=K_.KVQ_KEYS_PER_TOKEN,
                                rot=hadamard_value_bases(w))
    turbo["workload"] = "same 80K decode, per-token keys + shared Hadamard values"
    wide = {f"{b}bit": time_variant_decode(w, table, L0, args.replicas, n_dec, scale, bits=b) for b in (3, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, cfg, caches[0], args.cpu_seconds)

    rec = {
        "metric": "fused 2-bit decode attention: KV tokens/s + HBM GB/s (% peak) at 80K ctx",
        "value": ctx_mean / (ms_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": n_warm * args.replicas,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 accumulate over 2-bit codes (bf16 input)",
        "data": "synthetic seeded omni stream (video/audio/text chunks), random bases",
        "config": {"workload": "decode step at 81,920-position context: append 1 token + rotate q + fused decode",
                   "context": int(ctx_mean), "head_dim": d, "q_heads": hq, "kv_heads": hkv,
                   "batch": 1, "layer_replicas": args.replicas, "page_tokens": pt},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": decode_traffic_bytes(),
                     "kernel": "decode (partition + merge)", "bytes_per_launch": dec_bytes,
                     "avg_launch_us": dec_ms * 1e3},
        "cpu_baseline": cpu,
        "extra": {"decode_us_hbm": dec_ms * 1e3, "decode_us_warm": warm_ms * 1e3,
                  "decode_kv_tokens_per_s": Ld / (dec_ms * 1e-3),
                  "decode_us_half_pages_retained": half_ms * 1e3,
                  "copy_read_write_GBps": copy_bytes / (copy_ms * 1e-3) / 1e9,
                  "step_wall_us": wall / steps * 1e6,
                  "value_calibration": calib,
                  "turboquant_baseline": turbo,
                  "wider_codes": wide},
    }
    print(json.dumps(rec), flush=True)


def time_variant_decode(w, table, L0: int, replicas: int, n_dec: int, scale: float, key_mode: int = 0,
                        rot=None, bits: int = 2) -> dict:
    """The same 80K decode for another cache variant through the same
    kernels: per-token keys (key_mode 1) and / or other value bases, or 3- /
    4-bit codes (the stream's own tokens with the wider codebook); `replicas`
    HBM-resident caches, decode launches only, HIP events on the launch
    stream."""
    import dataclasses

    import torch
    import decode_attention_kvq_amd as K
    from omnistream import lloyd_max_codebook
    from tests import kvq_harness as H

    dev = torch.device("cuda", 0)
    wv = dataclasses.replace(w, codebook=lloyd_max_codebook(bits)) if bits != 2 else w
    cfg, params, c0 = H.build(wv, page_table=table, upto=[L0], key_mode=key_mode, rot=rot)
    caches = [c0]
    for _ in range(replicas - 1):
        cc = K.Cache(cfg, torch.from_numpy(table), device=dev)
        for name in ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "k_tail", "seq_len"):
            getattr(cc, name).copy_(getattr(c0, name))
        cc.set_lengths(c0.lengths())
        caches.append(cc)
    q_rot = K.kvq_rotate_query(cfg, params, H.query_tensor(wv, dev))
    out = torch.empty(q_rot.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(K.kvq_decode_workspace_bytes(cfg, L0), dtype=torch.uint8, device=dev)
    for cc in caches:
        K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(g, stream=s_cap):
            for cc in caches:
                K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_dec):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (n_dec * replicas)
    d, hq, hkv = w.cfg.head_dim, w.cfg.n_q_heads, w.cfg.n_kv_heads
    # per (position, KV head): key and value codes (b d / 8 bytes each), the
    # key statistics (2 d fp16 per 32 positions) or a key norm, a value norm
    per = 2 * bits * d // 8 + (4 if key_mode else (2 * d * 2) // 32 + 2)
    nbytes = L0 * hkv * per + L0 + hkv * 3 * d * d * 4 + 2 * hq * d * 4
    del g, caches
    return {"decode_us_hbm": ms * 1e3, "bytes_per_launch": nbytes, "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_8TBps": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def time_calibration(n_tokens: int, n_queries: int = 8, repeats: int = 5) -> dict:
    """Value-basis calibration (contribution weights -> per-modality weighted
    covariances -> eigenbases) over the first n_tokens of the 80K omni stream
    (28 query / 4 KV heads, d = 128, bf16), n_queries calibration queries per
    query head.  Inputs resident on the GPU; HIP events per step on the
    launch stream; the median of `repeats` runs after one warm-up."""
    import torch
    import decode_attention_kvq_amd as K
    from omnistream import calibration_queries, generate
    from tests import kvq_harness as H

    w = generate(2, length=n_tokens)
    dev = torch.device("cuda", 0)
    k = H._kv_tensor(w.k[0], w.dtype, dev)
    v = H._kv_tensor(w.v[0], w.dtype, dev)
    mod = torch.from_numpy(np.ascontiguousarray(w.modality[0])).to(dev)
    q = H._kv_tensor(calibration_queries(w, n_queries), w.dtype, dev)
    c = w.cfg
    ws = torch.empty(K.kvq_calib_workspace_bytes(c.head_dim, c.n_q_heads, c.n_kv_heads, n_tokens, n_queries),
                     dtype=torch.uint8, device=dev)
    wt = torch.empty((c.n_kv_heads, n_tokens), dtype=torch.float64, device=dev)
    cov = torch.empty((c.n_kv_heads, 3, c.head_dim, c.head_dim), dtype=torch.float64, device=dev)
    wsum = torch.empty((c.n_kv_heads, 3), dtype=torch.float64, device=dev)
    rot = torch.empty(cov.shape, dtype=torch.float32, device=dev)
    lam = torch.empty(cov.shape[:-1], dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream()
    times = []
    for rep in range(repeats + 1):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        K.kvq_calib_contribution(k, q, weights=wt, workspace=ws)
        ev[1].record(stream)
        K.kvq_calib_covariance(v, mod, wt, cov=cov, weight_sum=wsum, workspace=ws)
        ev[2].record(stream)
        K.kvq_calib_eigenbasis(cov, rot=rot, eigenvalues=lam, workspace=ws)
        ev[3].record(stream)
        torch.cuda.synchronize()
        if rep:
            times.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
    t = np.median(np.array(times), axis=0)
    # the fp64 oracle's whole calibration on one host thread, for context
    from threadpoolctl import threadpool_limits
    from oracle import kvq_calib_oracle as CO
    from oracle import kvq_oracle as O
    with threadpool_limits(limits=1):
        t_cpu = time.perf_counter()
        CO.calibrate_value_bases(O.as_f64(w.k[0], w.dtype), O.as_f64(w.v[0], w.dtype), w.modality[0],
                                 O.as_f64(calibration_queries(w, n_queries), w.dtype), 1.0 / math.sqrt(c.head_dim))
        t_cpu = time.perf_counter() - t_cpu
    rows = n_queries * c.n_q_heads
    d = c.head_dim
    # fp64 flops: scores twice (max / sum pass, then weights) at 2 per FMA;
    # covariance: one product and one FMA per (token, KV head, entry i <= j)
    contrib_flop = 2.0 * n_tokens * rows * d * 2
    cov_flop = 2.0 * n_tokens * c.n_kv_heads * d * (d + 1) / 2
    return {"workload": f"{n_tokens} tokens, {c.n_q_heads}/{c.n_kv_heads} heads, d={d}, {n_queries} queries/head",
            "ms_total": float(t.sum()), "ms_contribution": float(t[0]), "ms_covariance": float(t[1]),
            "ms_eigenbasis": float(t[2]), "matrices": 3 * c.n_kv_heads,
            "contribution_fp64_TFLOPs": contrib_flop / (t[0] * 1e-3) / 1e12,
            "covariance_fp64_TFLOPs": cov_flop / (t[1] * 1e-3) / 1e12,
            "fp64_peak_TFLOPs": 78.6, "oracle_ms_1thread": t_cpu * 1e3}


def cpu_baseline(w, cfg, cache, budget_s: float) -> dict:
    """The fp64 oracle (as it stands) decoding the same packed cache on the
    host: rotate the queries, dequantize, attend, rotate back.  Sample: whole
    decodes of the 80K-position step, KV head by KV head, repeated until about
    budget_s seconds of CPU work are done (a partial last pass counts its
    heads); the rate is scaled to one full decode."""
    from threadpoolctl import threadpool_limits

    from decode_attention_kvq_amd.layout import session_view
    from oracle import kvq_oracle as O

    host = cache.host_arrays()
    n = int(host["seq_len"][0])
    g = cfg.n_q_heads // cfg.n_kv_heads
    views = [session_view(host, cfg, 0, n, h) for h in range(cfg.n_kv_heads)]
    done_heads = 0
    t_total = 0.0
    with threadpool_limits(limits=1):
        while t_total < budget_s:
            t = time.perf_counter()
            q_rot = O.rotate_query(O.as_f64(w.q, w.dtype)[0], w.signs, cfg.n_kv_heads)
            t_total += time.perf_counter() - t
            for h, view in enumerate(views):
                t = time.perf_counter()
                for i in range(h * g, (h + 1) * g):
                    O.decode_attention_head(q_rot[i], view["k_codes"], view["lo"], view["hi"], view["v_codes"],
                                            view["norms"], view["modality"], w.rot[h], w.codebook,
                                            1.0 / math.sqrt(cfg.head_dim))
                t_total += time.perf_counter() - t
                done_heads += 1
                if t_total >= budget_s:
                    break
    t_step = t_total * cfg.n_kv_heads / done_heads
    return {"value": n / t_step, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"fp64 oracle decode of {done_heads} KV heads ({done_heads / cfg.n_kv_heads:.2f} "
                      f"decodes, {g} query heads each) over {n} positions, scaled to one decode; "
                      f"{t_total:.1f} s on 1 thread"}


if __name__ == "__main__":
    main()
