"""Benchmark: fused 2-bit decode attention on the packed KV cache at 80K context.

One step = one decode step of one attention layer on the seeded synthetic
omni stream (81,920 cached positions, 28 query / 4 KV heads, d = 128, bf16
input): quantize-append the step's new key/value, rotate the query, and run
the fused decode over the packed cache, in one kvq_decode_step call (two
launches; the same step as two calls is reported beside it).  Steps cycle over R layer replicas
(R x 27.8 MB > the 256 MB Infinity Cache) so that the cache is read from HBM.
Exactly --warmup untimed steps, then exactly --steps timed steps.

Prints one JSON line.  `value` = KV positions attended per second (mean
context over the timed steps / time per step, inputs resident in HBM).
`roofline` is for the decode launch (partition + merge kernels), timed with
HIP events on the stream it runs on.  `cpu_baseline` is the fp64 oracle
decoding the same packed cache on the host cores (all of them, and one).
`extra` holds the other workloads' decodes (the 32-session paged batch, the
131K stream loop with its 1,024-position append), the 3- / 4-bit and
per-token-key variants, the value-basis calibration, and context figures
(warm decode, a plain streaming read and copy of the decode's bytes).
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
L80K = 81920

# HBM bytes of one decode launch (partition + merge kernels) at the 80K
# workload, from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), each
# scaled by what the counter reads for a plain 256 MiB device copy
# (FETCH_SIZE x 1.9998, WRITE_SIZE x 1.0); see profiles/decode_80k_hbm_bytes.md.
# Valid only for the decode source the counters were taken on (SHA-256 of
# kvq_decode.hip); otherwise `traffic` is reported as null.
DECODE_TRAFFIC = {"kvq_decode_sha256": "d1b0765908da56527c072c3d9237c7f75f1e9a006eb40feabb38db8ded1b3fcd",
                  "bytes": 32901595}


def decode_traffic_bytes():
    import hashlib
    path = os.path.join(ROOT, "decode_attention_kvq_amd", "csrc", "kvq_decode.hip")
    try:
        digest = hashlib.sha256(open(path, "rb").read()).hexdigest()
    except OSError:
        return None
    return DECODE_TRAFFIC["bytes"] if digest == DECODE_TRAFFIC["kvq_decode_sha256"] else None


def algorithmic_decode_bytes(lengths, d: int, hq: int, hkv: int, bits: int = 2, key_mode: int = 0) -> int:
    """Bytes one decode must move: per (position, KV head) the key and value
    codes (b d / 8 each), the key group statistics (2 d fp16 per 32
    positions; a key norm instead for per-token keys) and the value norm
    (fp16); one modality byte per position; the value bases (3 d^2 fp32 per
    KV head); the rotated queries and the outputs (fp32) of every session."""
    lengths = [int(x) for x in np.atleast_1d(lengths)]
    per_pos_head = 2 * bits * d // 8 + (2 if key_mode else (2 * d * 2) // 32) + 2
    n = sum(lengths)
    return n * hkv * per_pos_head + n + hkv * 3 * d * d * 4 + 2 * len(lengths) * hq * d * 4


def algorithmic_append_bytes(n_new: int, start: int, d: int, hkv: int, in_bytes: int) -> int:
    """Bytes an append of n_new positions at position `start` must move: the
    new keys and values and their modality bytes in; key and value codes,
    value norms and modality bytes out; the statistics of every group the
    append touches (written, and for an open first group its raw keys read
    back from the tail); the value bases and the Hadamard signs."""
    g0, g1 = start // 32, (start + n_new - 1) // 32
    groups = g1 - g0 + 1
    tail = (start % 32) * hkv * d * in_bytes
    return (2 * n_new * hkv * d * in_bytes + n_new                   # K, V, modality in
            + 2 * n_new * hkv * d // 4 + 2 * n_new * hkv + n_new      # codes, norms, modality out
            + groups * hkv * 2 * d * 2 + tail                          # statistics, open-group keys
            + hkv * 3 * d * d * 4 + hkv * d)                           # bases, signs


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _replicas(cfg, cache0, page_table, n, dev):
    """n - 1 copies of cache0 in their own buffers (layer replicas)."""
    import torch
    import decode_attention_kvq_amd as K
    caches = [cache0]
    for _ in range(n - 1):
        cc = K.Cache(cfg, page_table.clone() if isinstance(page_table, torch.Tensor) else torch.from_numpy(page_table),
                     device=dev)
        for name in ("k_codes", "k_stats", "v_codes", "v_norms", "modality", "k_tail", "seq_len", "page_table"):
            getattr(cc, name).copy_(getattr(cache0, name))
        cc.set_lengths(cache0.lengths())
        caches.append(cc)
    torch.cuda.synchronize()
    return caches


def _capture(fns, s_cap):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(g, stream=s_cap):
            for f in fns:
                f()
    return g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--replicas", type=int, default=20)
    ap.add_argument("--context", type=int, default=L80K,
                    help="cached positions before the first step (the workload's is 81,920; other values "
                         "for partition-plan studies with --decode-only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="the 80K step and its decode only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU budget of each oracle timing")
    ap.add_argument("--calibration-only", action="store_true",
                    help="only time the value-basis calibration on the 80K stream and print its JSON line")
    ap.add_argument("--decode-only", action="store_true",
                    help="only replay the 80K decode graph (partition + merge over the layer replicas) "
                         "--steps times and print its timing (for profiler runs)")
    ap.add_argument("--batched-only", action="store_true",
                    help="only time the 32-session paged decode and print its JSON line")
    ap.add_argument("--stream-loop-only", action="store_true",
                    help="only time the 131K stream loop (append, decode, loop) and print its JSON line")
    ap.add_argument("--stream-read", action="store_true",
                    help="only time a plain streaming read of the 80K decode's byte count (one reduction "
                         "kernel per read, layer replicas) --steps times and print its timing")
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
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.stream_read:
        print(json.dumps({"stream_read": time_stream_read(algorithmic_decode_bytes([L80K], 128, 28, 4),
                                                          args.replicas, max(args.steps, 1))}), flush=True)
        return
    if args.calibration_only:
        print(json.dumps({"value_calibration": time_calibration(L80K)}), flush=True)
        return
    if args.batched_only:
        print(json.dumps({"batched_paged_decode": time_batched_paged(max(3, args.replicas // 6))}), flush=True)
        return
    if args.stream_loop_only:
        print(json.dumps({"stream_loop": time_stream_loop(max(4, args.replicas // 5))}), flush=True)
        return

    import decode_attention_kvq_amd as K
    from omnistream import generate
    from tests import kvq_harness as H

    R = args.replicas
    W, S = max(args.warmup, 0), max(args.steps, 1)
    extra_pos = (W + S) // R + 8
    L0 = args.context
    w = generate(2, length=L0 + extra_pos)
    c = w.cfg
    d, hq, hkv = c.head_dim, c.n_q_heads, c.n_kv_heads
    pt = w.page_tokens
    max_pages = -(-(L0 + extra_pos) // pt)
    table = np.arange(max_pages, dtype=np.int32)[None, :]
    cfg, params, cache0 = H.build(w, page_table=table, upto=[L0])
    caches = _replicas(cfg, cache0, table, R, dev)

    k_steps = H._kv_tensor(w.k[0][None, L0:L0 + extra_pos], "bf16", dev)     # [1, extra, Hkv, d]
    v_steps = H._kv_tensor(w.v[0][None, L0:L0 + extra_pos], "bf16", dev)
    m_steps = torch.from_numpy(np.ascontiguousarray(w.modality[0][None, L0:L0 + extra_pos])).to(dev)
    q = H.query_tensor(w, dev)
    q_rot = torch.empty(q.shape, dtype=torch.float32, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kvq_decode_workspace_bytes(cfg, L0 + extra_pos), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d)

    ws_step = torch.zeros(K.kvq_decode_step_workspace_bytes(cfg, L0 + extra_pos), dtype=torch.uint8, device=dev)

    def one_step(r):
        # one decode step, kvq_decode_step: append the step's key / value,
        # rotate its query and attend every position (two launches: the
        # partitions over the closed groups beside the append, then the merge
        # with the open group)
        K.kvq_decode_step(cfg, caches[r], params, k_steps[:, :1], v_steps[:, :1], m_steps[:, :1], q, q_rot,
                          scale, out, ws_step)

    def one_step_two_calls(r):
        # the same step as kvq_append_and_rotate (one launch), then kvq_decode_attention
        cache = caches[r]
        K.kvq_append_and_rotate(cfg, cache, params, k_steps[:, :1], v_steps[:, :1], m_steps[:, :1], q, q_rot)
        K.kvq_decode_attention(cfg, cache, params, q_rot, scale, out, ws)

    # Eager pass over every replica (loads every kernel), then rewind the lengths.
    for r in range(R):
        one_step(r)
        one_step_two_calls(r)
    torch.cuda.synchronize()
    for cc in caches:
        cc.set_lengths([L0])
    torch.cuda.synchronize()

    # Step graphs: one over all R replicas, plus one over the first r replicas
    # for the remainders of --warmup and --steps, so that exactly W and S steps
    # run.  A replay appends the same new position again at the (device-side)
    # current length: every step is a full decode step on a cache of
    # L0 + (steps so far on that replica) + 1 positions.
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    g_step = {R: _capture([lambda r=r: one_step(r) for r in range(R)], s_cap)}
    for rem in {W % R, S % R} - {0}:
        g_step[rem] = _capture([lambda r=r: one_step(r) for r in range(rem)], s_cap)
    torch.cuda.synchronize()
    for cc in caches:                       # capture advanced the host mirror only
        cc.set_lengths([L0])
    torch.cuda.synchronize()

    def run_steps(n):
        for _ in range(n // R):
            g_step[R].replay()
        if n % R:
            g_step[n % R].replay()

    g_dec = _capture([lambda r=r: K.kvq_decode_attention(cfg, caches[r], params, q_rot, scale, out, ws)
                      for r in range(R)], s_cap)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    if args.decode_only:
        for _ in range(max(1, W // R)):
            g_dec.replay()
        torch.cuda.synchronize()
        d0, d1 = _events()
        n_rep = max(1, S // R)
        d0.record(stream)
        for _ in range(n_rep):
            g_dec.replay()
        d1.record(stream)
        torch.cuda.synchronize()
        us = d0.elapsed_time(d1) * 1e3 / (n_rep * R)
        nb = algorithmic_decode_bytes([L0], d, hq, hkv)
        print(json.dumps({"decode_only": {"context": L0, "launches": n_rep * R, "avg_launch_us": us,
                                          "bytes_per_launch": nb, "GBps": nb / us / 1e3}}), flush=True)
        return

    run_steps(W)
    torch.cuda.synchronize()
    len_before = np.array([int(cc.seq_len.cpu()[0]) for cc in caches])
    e0, e1 = _events()
    t0 = time.perf_counter()
    e0.record(stream)
    run_steps(S)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / S
    len_after = np.array([int(cc.seq_len.cpu()[0]) for cc in caches])
    # step j on a replica at length L attends L + 1 positions: the mean over the timed steps
    ctx_sum = sum(int(a - b) * (int(b) + (int(a - b) + 1) / 2.0) for a, b in zip(len_after, len_before))
    ctx_mean = ctx_sum / S
    assert int((len_after - len_before).sum()) == S
    for cc, n in zip(caches, len_after):
        cc.set_lengths([int(n)])

    # Decode launches alone: R back-to-back decodes per replay, HIP events on the stream.
    g_dec.replay()
    n_dec = max(5, (2 * S) // R)
    d0, d1 = _events()
    d0.record(stream)
    for _ in range(n_dec):
        g_dec.replay()
    d1.record(stream)
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / (n_dec * R)
    Ld = int(np.mean(len_after))
    dec_bytes = algorithmic_decode_bytes([Ld], d, hq, hkv)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9

    # The same steps as two calls (append + rotate, then decode: three launches).
    g_two = _capture([lambda r=r: one_step_two_calls(r) for r in range(R)], s_cap)
    for cc, n in zip(caches, len_after):
        cc.set_lengths([int(n)])
    torch.cuda.synchronize()
    g_two.replay()
    n_two = max(5, S // R)
    t0e, t1e = _events()
    t0e.record(stream)
    for _ in range(n_two):
        g_two.replay()
    t1e.record(stream)
    torch.cuda.synchronize()
    two_us = t0e.elapsed_time(t1e) * 1e3 / (n_two * R)
    for cc, n in zip(caches, len_after):
        cc.set_lengths([int(n)])
    torch.cuda.synchronize()
    del g_two

    extra = {"decode_us_hbm": dec_ms * 1e3, "decode_kv_tokens_per_s": Ld / (dec_ms * 1e-3),
             "step_us": ms_step * 1e3, "step_minus_decode_us": ms_step * 1e3 - dec_ms * 1e3,
             "step_two_calls_us": two_us,
             "step_wall_us": wall / S * 1e6, "warmup_steps_run": W, "timed_steps_run": S}
    if not args.no_extra:
        extra.update(extra_80k(K, cfg, params, caches, table, q_rot, out, ws, scale, n_dec, dec_bytes, s_cap, R,
                               dev))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, cfg, caches[0], args.cpu_seconds)
    del g_step, g_dec
    if not args.no_extra:
        from omnistream import hadamard_value_bases
        turbo = time_variant_decode(w, table, L0, R, n_dec, scale, key_mode=K.KVQ_KEYS_PER_TOKEN,
                                    rot=hadamard_value_bases(w))
        turbo["workload"] = "same 80K decode, per-token keys + shared Hadamard values"
        extra["turboquant_baseline"] = turbo
        extra["wider_codes"] = {f"{b}bit": time_variant_decode(w, table, L0, R, n_dec, scale, bits=b)
                                for b in (3, 4)}
        # the same cache attended by 64 query heads (16 per KV head): the
        # decode takes its wider-group partition kernel there
        import dataclasses
        w16 = dataclasses.replace(w, cfg=dataclasses.replace(w.cfg, n_q_heads=64),
                                  q=np.ascontiguousarray(np.concatenate([w.q] * 3, axis=1)[:, :64]))
        g16 = time_variant_decode(w16, table, L0, R, n_dec, scale)
        g16["workload"] = "same 80K cache, 64 query heads (16 per KV head, the wider-group partition kernel)"
        extra["gqa16_decode"] = g16
        del caches
        torch.cuda.empty_cache()
        extra["batched_paged_decode"] = time_batched_paged(max(3, R // 6))
        torch.cuda.empty_cache()
        extra["stream_loop"] = time_stream_loop(max(4, R // 5))
        torch.cuda.empty_cache()
        extra["value_calibration"] = time_calibration(L0, with_oracle=not args.no_cpu_baseline)

    rec = {
        "metric": "fused 2-bit decode attention: KV tokens/s + HBM GB/s (% peak) at 80K ctx",
        "value": ctx_mean / (ms_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1, "steps": S, "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 accumulate over 2-bit codes (bf16 input)",
        "data": "synthetic seeded omni stream (video/audio/text chunks), random bases",
        "config": {"workload": "decode step at 81,920-position context (kvq_decode_step: append 1 token + rotate q "
                               "+ fused decode, two launches)",
                   "context": round(ctx_mean, 1), "head_dim": d, "q_heads": hq, "kv_heads": hkv,
                   "batch": 1, "layer_replicas": R, "page_tokens": pt},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": decode_traffic_bytes(),
                     "kernel": "decode (partition + merge)", "bytes_per_launch": dec_bytes,
                     "avg_launch_us": dec_ms * 1e3},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(rec), flush=True)


def extra_80k(K, cfg, params, caches, table, q_rot, out, ws, scale, n_dec, dec_bytes, s_cap, R, dev) -> dict:
    """Context for the 80K decode: every other page unmapped (sparse page
    set), the warm (Infinity-Cache resident) decode, a plain streaming read
    and a plain copy of the same byte count."""
    import torch
    stream = torch.cuda.current_stream()
    g_dec = _capture([lambda r=r: K.kvq_decode_attention(cfg, caches[r], params, q_rot, scale, out, ws)
                      for r in range(R)], s_cap)
    for cc in caches:
        cc.page_table[:, 1::2] = -1
    g_dec.replay()
    s0, s1 = _events()
    s0.record(stream)
    for _ in range(n_dec):
        g_dec.replay()
    s1.record(stream)
    torch.cuda.synchronize()
    half_ms = s0.elapsed_time(s1) / (n_dec * R)
    for cc in caches:
        cc.page_table.copy_(torch.from_numpy(table))
    torch.cuda.synchronize()

    g_warm = _capture([lambda: K.kvq_decode_attention(cfg, caches[0], params, q_rot, scale, out, ws)] * R, s_cap)
    g_warm.replay()
    w0, w1 = _events()
    w0.record(stream)
    for _ in range(10):
        g_warm.replay()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / (10 * R)

    sbufs = [torch.ones(dec_bytes // 4, dtype=torch.float32, device=dev) for _ in range(R)]
    cdst = torch.empty_like(sbufs[0])
    for sb in sbufs:
        cdst.copy_(sb)
    c0, c1 = _events()
    c0.record(stream)
    for _ in range(5):
        for sb in sbufs:
            cdst.copy_(sb)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / (5 * len(sbufs))
    copy_bytes = 2 * cdst.numel() * 4
    del sbufs, cdst, g_dec, g_warm
    return {"decode_us_half_pages_retained": half_ms * 1e3, "decode_us_warm": warm_ms * 1e3,
            "copy_read_write_GBps": copy_bytes / (copy_ms * 1e-3) / 1e9,
            "stream_read": time_stream_read(dec_bytes, R, 100)}


def time_stream_read(nbytes: int, replicas: int, launches: int) -> dict:
    """The floor for one read-only kernel of nbytes (the decode's algorithmic
    bytes): kvq_probe_stream_read, a plain 16-byte streaming read, over
    `replicas` buffers cycled so the reads come from HBM, launched from a HIP
    graph like the decode, HIP events over about `launches` launches, for
    several grid sizes; the fastest is reported."""
    import torch
    import decode_attention_kvq_amd as K
    nb = (nbytes // 16) * 16
    bufs = [torch.ones(nb // 4, dtype=torch.int32, device="cuda") for _ in range(replicas)]
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(stream)
    n_rep = max(1, launches // replicas)
    shapes = {}
    for wgs in (256, 512, 1024, 2048, 4096):
        # one graph of `replicas` launches (one per buffer), replayed: the
        # launches run back to back like the decode's
        for b in bufs:
            K.kvq_probe_stream_read(b, sink, wgs)
        torch.cuda.synchronize()
        g = _capture([lambda b=b: K.kvq_probe_stream_read(b, sink, wgs) for b in bufs], s_cap)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = _events()
        e0.record(stream)
        for _ in range(n_rep):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        shapes[wgs] = e0.elapsed_time(e1) * 1e3 / (n_rep * replicas)
        del g
    best = min(shapes, key=shapes.get)
    us = shapes[best]
    del bufs
    return {"bytes_per_launch": nb, "avg_launch_us": us, "GBps": nb / us / 1e3,
            "frac_of_8TBps": nb / us / 1e3 / HBM_PEAK_GBS, "workgroups": best,
            "us_by_workgroups": {str(k): round(v, 3) for k, v in shapes.items()},
            "kernel": "kvq_probe_stream_read (256 threads per workgroup)"}


def time_batched_paged(replicas: int, n_rep: int = 10) -> dict:
    """The 32-session batch: 16 query / 2 KV heads, d = 128, session lengths
    U[8,192, 65,536], 256-position pages under a seeded random page table,
    one decode launch for all sessions; `replicas` copies of the packed cache
    (together above the Infinity Cache) cycled, HIP events."""
    import torch
    import decode_attention_kvq_amd as K
    from omnistream import generate
    from tests import kvq_harness as H
    dev = torch.device("cuda", 0)
    w = generate(3)
    c = w.cfg
    cfg, params, c0 = H.build(w, chunks=[16384])
    caches = _replicas(cfg, c0, torch.from_numpy(w.page_table), replicas, dev)
    q_rot = K.kvq_rotate_query(cfg, params, H.query_tensor(w, dev))
    out = torch.empty(q_rot.shape, dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kvq_decode_workspace_bytes(cfg, int(w.lengths.max())), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(c.head_dim)
    for cc in caches:
        K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws)
    torch.cuda.synchronize()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    g = _capture([lambda cc=cc: K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws) for cc in caches],
                 s_cap)
    torch.cuda.synchronize()
    g.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(n_rep):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (n_rep * replicas)
    nb = algorithmic_decode_bytes(w.lengths, c.head_dim, c.n_q_heads, c.n_kv_heads)
    total = int(w.lengths.sum())
    del g, caches
    return {"workload": f"{c.batch} sessions, {total} positions, {c.n_q_heads}/{c.n_kv_heads} heads, d={c.head_dim}, "
                        f"{w.page_tokens}-position pages, random page table",
            "decode_us_hbm": us, "bytes_per_launch": nb, "GBps": nb / us / 1e3,
            "frac_of_8TBps": nb / us / 1e3 / HBM_PEAK_GBS, "kv_tokens_per_s": total / (us * 1e-6),
            "replicas": replicas}


def time_stream_loop(replicas: int, n_rep: int = 10) -> dict:
    """The stream loop: a 131,072-position cache (32 query / 8 KV heads, d =
    128, bf16 input), then one 1,024-position chunk (640 video + 25 audio +
    359 text) quantized and appended in one call, then one decode over the
    132,096 positions.  Timed separately (append alone; decode alone) and end
    to end (append + query rotation in one launch, then the decode), each over
    `replicas` copies of the cache (HBM-resident), HIP events per replay; the
    lengths are rewound to 131,072 between replays, outside the timed region."""
    import torch
    import decode_attention_kvq_amd as K
    from omnistream import generate
    from tests import kvq_harness as H
    dev = torch.device("cuda", 0)
    w = generate(4)
    c = w.cfg
    n0, n1 = int(w.prefix_lengths[0]), int(w.lengths[0])
    cfg, params, c0 = H.build(w, upto=[n0], chunks=[16384])
    caches = _replicas(cfg, c0, torch.from_numpy(w.page_table), replicas, dev)
    kc = H._kv_tensor(w.k[0][None, n0:n1], w.dtype, dev)
    vc = H._kv_tensor(w.v[0][None, n0:n1], w.dtype, dev)
    mc = torch.from_numpy(np.ascontiguousarray(w.modality[0][None, n0:n1])).to(dev)
    q = H.query_tensor(w, dev)
    q_rot = torch.empty(q.shape, dtype=torch.float32, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kvq_decode_workspace_bytes(cfg, n1), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(c.head_dim)
    stream = torch.cuda.current_stream()
    s_cap = torch.cuda.Stream()

    def rewind(n):
        for cc in caches:
            cc.set_lengths([n])
        torch.cuda.synchronize()

    def timed(g, before=None):
        ts = []
        for _ in range(n_rep + 1):
            if before is not None:
                before()
            e0, e1 = _events()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / replicas)
        return float(np.median(ts[1:]))

    # eager pass (kernels loaded), then the three graphs
    for cc in caches:
        K.kvq_append_and_rotate(cfg, cc, params, kc, vc, mc, q, q_rot)
        K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws)
    rewind(n0)
    s_cap.wait_stream(stream)
    g_app = _capture([lambda cc=cc: K.kvq_quantize_append(cfg, cc, params, kc, vc, mc) for cc in caches], s_cap)
    rewind(n0)
    g_loop = _capture([f for cc in caches for f in (
        lambda cc=cc: K.kvq_append_and_rotate(cfg, cc, params, kc, vc, mc, q, q_rot),
        lambda cc=cc: K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws))], s_cap)
    rewind(n1)
    g_dec = _capture([lambda cc=cc: K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws) for cc in caches],
                     s_cap)
    torch.cuda.synchronize()
    app_us = timed(g_app, lambda: rewind(n0))
    loop_us = timed(g_loop, lambda: rewind(n0))
    rewind(n1)
    dec_us = timed(g_dec)
    app_b = algorithmic_append_bytes(n1 - n0, n0, c.head_dim, c.n_kv_heads, 2)
    dec_b = algorithmic_decode_bytes([n1], c.head_dim, c.n_q_heads, c.n_kv_heads)
    del g_app, g_loop, g_dec, caches
    return {"workload": f"{n0}-position cache + {n1 - n0}-position chunk, {c.n_q_heads}/{c.n_kv_heads} heads, "
                        f"d={c.head_dim}, bf16 input",
            "append_us": app_us, "append_tokens_per_s": (n1 - n0) / (app_us * 1e-6),
            "append_bytes": app_b, "append_GBps": app_b / app_us / 1e3,
            "decode_us_hbm": dec_us, "decode_bytes": dec_b, "decode_GBps": dec_b / dec_us / 1e3,
            "decode_frac_of_8TBps": dec_b / dec_us / 1e3 / HBM_PEAK_GBS,
            "decode_kv_tokens_per_s": n1 / (dec_us * 1e-6),
            "loop_us": loop_us, "loop_launches": "append+rotate, decode (partition + merge)",
            "replicas": replicas}


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
    caches = _replicas(cfg, c0, table, replicas, dev)
    q_rot = K.kvq_rotate_query(cfg, params, H.query_tensor(wv, dev))
    out = torch.empty(q_rot.shape, dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kvq_decode_workspace_bytes(cfg, L0), dtype=torch.uint8, device=dev)
    for cc in caches:
        K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws)
    torch.cuda.synchronize()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    g = _capture([lambda cc=cc: K.kvq_decode_attention(cfg, cc, params, q_rot, scale, out, ws) for cc in caches],
                 s_cap)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    g.replay()
    e0, e1 = _events()
    e0.record(stream)
    for _ in range(n_dec):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (n_dec * replicas)
    d, hq, hkv = w.cfg.head_dim, w.cfg.n_q_heads, w.cfg.n_kv_heads
    nbytes = algorithmic_decode_bytes([L0], d, hq, hkv, bits=bits, key_mode=key_mode)
    del g, caches
    return {"decode_us_hbm": ms * 1e3, "bytes_per_launch": nbytes, "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_8TBps": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def time_calibration(n_tokens: int, n_queries: int = 8, repeats: int = 5, with_oracle: bool = True) -> dict:
    """Value-basis calibration (contribution weights -> per-modality weighted
    covariances -> eigenbases) over the first n_tokens of the 80K omni stream
    (28 query / 4 KV heads, d = 128, bf16), n_queries calibration queries per
    query head.  Inputs resident on the GPU; HIP events per step on the
    launch stream; the median of `repeats` runs after one warm-up.  With
    with_oracle, the oracle's whole calibration on one host thread is timed
    beside it (a CPU baseline)."""
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
    rows = n_queries * c.n_q_heads
    d = c.head_dim
    # fp64 flops: scores twice (max / sum pass, then weights) at 2 per FMA;
    # covariance: one product and one FMA per (token, KV head, entry i <= j)
    contrib_flop = 2.0 * n_tokens * rows * d * 2
    cov_flop = 2.0 * n_tokens * c.n_kv_heads * d * (d + 1) / 2
    rec = {"workload": f"{n_tokens} tokens, {c.n_q_heads}/{c.n_kv_heads} heads, d={d}, {n_queries} queries/head",
           "ms_total": float(t.sum()), "ms_contribution": float(t[0]), "ms_covariance": float(t[1]),
           "ms_eigenbasis": float(t[2]), "matrices": 3 * c.n_kv_heads,
           "contribution_fp64_TFLOPs": contrib_flop / (t[0] * 1e-3) / 1e12,
           "covariance_fp64_TFLOPs": cov_flop / (t[1] * 1e-3) / 1e12, "fp64_peak_TFLOPs": 78.6}
    if with_oracle:
        rec["oracle_ms_1thread"] = cpu_baseline_calibration(w, n_queries) * 1e3
    return rec


# ------------------------------------------------------------ CPU baselines

def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_calibration(w, n_queries: int) -> float:
    """Seconds of the fp64 oracle's whole value-basis calibration of the same
    stream on one host thread."""
    from threadpoolctl import threadpool_limits
    from omnistream import calibration_queries
    from oracle import kvq_calib_oracle as CO
    from oracle import kvq_oracle as O
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        CO.calibrate_value_bases(O.as_f64(w.k[0], w.dtype), O.as_f64(w.v[0], w.dtype), w.modality[0],
                                 O.as_f64(calibration_queries(w, n_queries), w.dtype),
                                 1.0 / math.sqrt(w.cfg.head_dim))
        return time.perf_counter() - t


def cpu_baseline(w, cfg, cache, budget_s: float) -> dict:
    """The fp64 oracle (as it stands) decoding the same packed cache on the
    host: rotate the queries, dequantize, attend, rotate back.  Sample: whole
    decodes of the 80K-position step, one task per query head, repeated until
    about budget_s seconds of wall time (a partial last pass counts the heads
    it finished), scaled to one decode.  Run twice: on a pool of host threads,
    one per core up to 16 (NumPy's own threading off, so `cores` is the
    threads used), and on one thread."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from decode_attention_kvq_amd.layout import session_view
    from oracle import kvq_oracle as O

    host = cache.host_arrays()
    n = int(host["seq_len"][0])
    g = cfg.n_q_heads // cfg.n_kv_heads
    views = [session_view(host, cfg, 0, n, h) for h in range(cfg.n_kv_heads)]
    sc = 1.0 / math.sqrt(cfg.head_dim)
    q64 = O.as_f64(w.q, w.dtype)[0]

    def head(i, q_rot):
        v = views[i // g]
        return O.decode_attention_head(q_rot[i], v["k_codes"], v["lo"], v["hi"], v["v_codes"], v["norms"],
                                       v["modality"], w.rot[i // g], w.codebook, sc)

    def run(threads):
        done, t_total = 0, 0.0
        with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=threads) as ex:
            while t_total < budget_s:
                t = time.perf_counter()
                q_rot = O.rotate_query(q64, w.signs, cfg.n_kv_heads)
                list(ex.map(lambda i: head(i, q_rot), range(cfg.n_q_heads)))
                t_total += time.perf_counter() - t
                done += cfg.n_q_heads
        return done, t_total

    nproc = os.cpu_count() or 1
    threads = max(1, min(16, nproc))
    done_n, t_n = run(threads)
    done_1, t_1 = run(1)
    rate_n = n / (t_n * cfg.n_q_heads / done_n)
    rate_1 = n / (t_1 * cfg.n_q_heads / done_1)
    return {"value": rate_n, "unit": "KV tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle decode of the 80K step ({n} positions, {cfg.n_q_heads} query heads as "
                      f"{cfg.n_q_heads} tasks on {threads} threads): {done_n / cfg.n_q_heads:.1f} decodes in "
                      f"{t_n:.1f} s, scaled to one decode",
            "value_1_thread": rate_1,
            "sample_1_thread": f"{done_1 / cfg.n_q_heads:.1f} decodes in {t_1:.1f} s on 1 thread",
            "host_nproc": nproc, "host_cpu": _cpu_model()}


if __name__ == "__main__":
    main()
