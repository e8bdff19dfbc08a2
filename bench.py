#!/usr/bin/env python3
"""Benchmark of the bounded video KV cache hot path on one MI355X.

A step is one steady-state chunk of the 14B-shaped sliding-window workload
(40 heads x 128, 1560-token frames, 6 sink + 12 rolling frames = 28080-token
cache, 3-frame chunks): kvc_append (fused 3D RoPE + ring write, evicting 4680
tokens) followed by kvc_attend (4680 queries over all 28080 cached keys).
Inputs are seeded synthetic N(0,1) bf16 chunks, resident in HBM before timing.

Prints one JSON line.  `value` is attention TFLOP/s over the whole step
(algorithmic 4*H*Lq*Lk*D flop per chunk / step wall time).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def back_to_back_ms(stream, ev, call, n=10):
    """Median event-timed duration of `call` over n calls queued back to back on `stream` with one
    synchronize at the end: the protocol of the chunk loop, used by every matrix-core leg."""
    import numpy as np
    import torch
    evs = [(ev(), ev()) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-context", action="store_true", help="skip the vendor-library reference timings")
    p.add_argument("--no-configs", action="store_true", help="skip the per-config chunk streams")
    p.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic_attend_c3.json"))
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (heads would shard across GPUs "
              "with no exchange on the attention path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from workloads import WORKLOADS, chunk_inputs

    w = WORKLOADS["c3"]
    S, H, D = w.frame_seqlen, w.heads, w.head_dim
    F = 3
    N = F * S
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---- inputs: a pool of chunks resident in HBM
    pool = []
    for c in range(4):
        q, k, v = chunk_inputs(w, c)
        pool.append(tuple(torch.from_numpy(x).to(dev, torch.bfloat16) for x in (q, k, v)))
    cache = kvc.KVCache(w.sink_frames, w.window_frames, S, H, D, w.grid_w, torch.bfloat16)
    out = torch.empty_like(pool[0][0])

    # fill the cache to capacity (6 chunks = 28080 tokens)
    t_frame = 0
    for c in range(6):
        q, k, v = pool[c % 4]
        cache.append(k, v, t_frame)
        t_frame += F
    torch.cuda.synchronize()
    Lk = cache.info()["n_valid"]
    assert Lk == w.capacity == 28080

    ev = lambda: torch.cuda.Event(enable_timing=True)
    flop = 4.0 * H * N * Lk * D

    def step(i, rec=None):
        nonlocal t_frame
        q, k, v = pool[i % 4]
        if rec:
            rec[0].record(stream)
        cache.append(k, v, t_frame)
        if rec:
            rec[1].record(stream)
        cache.attend(q, t_frame, out=out)
        if rec:
            rec[2].record(stream)
        t_frame += F

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    recs = [(ev(), ev(), ev()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, recs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    app_ms = [a.elapsed_time(b) for a, b, _ in recs]
    att_ms = [b.elapsed_time(c) for _, b, c in recs]
    att_avg = float(np.mean(att_ms))
    app_avg = float(np.mean(app_ms))
    assert cache.info()["n_valid"] == 28080

    # ---- retime over the whole cache (time band only), MALL flushed between samples by reading
    # 1 GiB of unrelated data (a read leaves no dirty lines to write back inside the timed kernel)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    ret_ms = []
    for i in range(12):
        flush.sum()
        a, b = ev(), ev()
        a.record(stream)
        cache.retime(1 if i % 2 == 0 else -1)
        b.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            ret_ms.append(a.elapsed_time(b))
    ret_avg = float(np.mean(ret_ms))
    # append with the MALL flushed as well (the step loop above runs warm)
    app_cold = []
    for i in range(8):
        flush.sum()
        a, b = ev(), ev()
        q, k, v = pool[i % 4]
        a.record(stream)
        cache.append(k, v, t_frame)
        b.record(stream)
        t_frame += F
        torch.cuda.synchronize()
        if i >= 2:
            app_cold.append(a.elapsed_time(b))
    dt_band = D - 4 * (D // 6)
    ceil_app_us, ceil_ret_us = same_size_ceilings(dev, stream, ev, flush, N * H * D * 2 * 2, Lk * H * dt_band * 2)
    # attention-mass scores of this chunk's queries over the whole cache (the Deep-Forcing scoring pass)
    qwin = pool[0][0]
    sc_out = cache.score(qwin, [t_frame - 3, t_frame - 2, t_frame - 1])
    torch.cuda.synchronize()
    score_ms = back_to_back_ms(stream, ev, lambda: cache.score(qwin, [t_frame - 3, t_frame - 2, t_frame - 1],
                                                              out=sc_out), n=6)
    # the same scores from the attention's row statistics (Deep Forcing scores the queries the previous
    # chunk attended with, over the cache that attention saw): the attend keeps each row's normaliser
    # (kvc_attend_stats) and the scoring runs only its columns pass (kvc_score_with_stats)
    row_stats = torch.empty(H * N, dtype=torch.float32, device=dev)
    att_stats_ms = back_to_back_ms(stream, ev, lambda: cache.attend(qwin, t_frame - 3, out=out, row_stats=row_stats),
                                   n=6)
    att_plain_ms = back_to_back_ms(stream, ev, lambda: cache.attend(qwin, t_frame - 3, out=out), n=6)
    cache.attend(qwin, t_frame - 3, out=out, row_stats=row_stats)
    sc_stats = cache.score(qwin, [t_frame - 3, t_frame - 2, t_frame - 1], row_stats=row_stats)
    torch.cuda.synchronize()
    score_stats_diff = float((sc_stats - sc_out).abs().max() / sc_out.abs().max())
    score_stats_ms = back_to_back_ms(stream, ev, lambda: cache.score(qwin, [t_frame - 3, t_frame - 2, t_frame - 1],
                                                                    out=sc_stats, row_stats=row_stats), n=6)
    extras = ceilings(dev, stream, ev)
    extras.update(sink_push_and_compact(dev, stream, flush, ev))
    extras.update(per_gpu_share(dev, stream, ev, w))
    extras.update(head_dim_64(dev, stream, ev, w))
    extras.update(block_causal_clip(dev, stream, ev, WORKLOADS["c2"]))
    extras.update(raw_keys_ab(dev, stream, ev, flush, w))
    extras.update(memrope_chunk(dev, stream, ev, flush, WORKLOADS["c6"]))
    extras.update(layer_group(dev, stream, ev, flush, WORKLOADS["c5a"]))
    # plain device copy of 1 GiB (twice the MALL): the achievable HBM rate on this board
    cx = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cy = torch.empty_like(cx)
    cy.copy_(cx)
    cp_ms = []
    for i in range(5):
        a, b = ev(), ev()
        a.record(stream)
        cy.copy_(cx)
        b.record(stream)
        torch.cuda.synchronize()
        cp_ms.append(a.elapsed_time(b))
    copy_gbps = 2.0 * (1 << 30) / (float(np.median(cp_ms)) * 1e-3) / 1e9
    del flush, cx, cy
    context = None if args.no_context else vendor_context(dev, stream, H, N, Lk, D)
    configs = {} if args.no_configs else config_streams(dev, stream, ev, cpu=not args.no_cpu_baseline)

    dt = D - 4 * (D // 6)
    app_bytes = 4.0 * N * H * D * 2
    ret_bytes = 2.0 * Lk * H * dt * 2
    att_tflops = flop / (att_avg * 1e-3) / 1e12
    value = flop / (ms_step * 1e-3) / 1e12

    traffic = None
    if os.path.exists(args.traffic):
        # counters taken on an older version of the kernel source do not count
        import hashlib
        h = hashlib.sha256()
        for name in ("kvc_attend.hip", "kvc_tiles.hpp"):     # the attention kernels' sources
            h.update(open(os.path.join(ROOT, "rolling_kv_cache_amd", "csrc", name), "rb").read())
        digest = h.hexdigest()
        try:
            rec = json.load(open(args.traffic))
            if rec.get("kernel_source_sha256") == digest:
                traffic = rec.get("bytes_per_launch")
        except Exception:
            traffic = None

    res = {
        "metric": "kvc_attend TFLOP/s (% bf16 MFMA peak) + ms per 3-frame chunk at 28080-token cache",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c3 14B-shaped sliding window + sink: 40 heads x 128, 1560-token frames (30x52), "
                               "3-frame chunks (4680 queries), 6 sink + 12 rolling frames = 28080-token cache",
                   "heads": H, "head_dim": D, "cache_tokens": Lk, "chunk_tokens": N, "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": round(att_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "kernels": {
            "attend_ms": round(att_avg, 4),
            "attend_tflops": round(att_tflops, 2),
            "attend_ms_p10_median_p90": [round(float(x), 4) for x in np.percentile(att_ms, [10, 50, 90])],
            "append_us_warm": round(app_avg * 1e3, 2),
            "append_us_warm_p10_median_p90": [round(float(x) * 1e3, 2) for x in np.percentile(app_ms, [10, 50, 90])],
            "append_GBps_warm": round(app_bytes / (app_avg * 1e-3) / 1e9, 1),
            "append_us_cold": round(float(np.mean(app_cold)) * 1e3, 2),
            "append_GBps_cold": round(app_bytes / (float(np.mean(app_cold)) * 1e-3) / 1e9, 1),
            "retime_us_cold": round(ret_avg * 1e3, 2),
            "retime_GBps_cold": round(ret_bytes / (ret_avg * 1e-3) / 1e9, 1),
            "append_hbm_frac_cold": round(app_bytes / (float(np.mean(app_cold)) * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "retime_hbm_frac_cold": round(ret_bytes / (ret_avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "append_same_size_copy_ceiling_us": round(ceil_app_us, 2),
            "append_frac_of_copy_ceiling": round(ceil_app_us / (float(np.mean(app_cold)) * 1e3), 4),
            "retime_same_size_inplace_ceiling_us": round(ceil_ret_us, 2),
            "retime_frac_of_inplace_ceiling": round(ceil_ret_us / (ret_avg * 1e3), 4),
            "hbm_copy_torch_GBps_measured": round(copy_gbps, 1),
            "score_ms": round(score_ms, 4),
            "score_tflops": round(flop / (score_ms * 1e-3) / 1e12, 2),
            "score_with_attention_row_stats_ms": round(score_stats_ms, 4),
            "score_with_row_stats_max_diff_rel_to_max": float("%.3g" % score_stats_diff),
            "attend_with_row_stats_ms": round(att_stats_ms, 4),
            "attend_without_row_stats_ms": round(att_plain_ms, 4),
            **extras,
        },
    }
    if context:
        res["context"] = context
    if configs:
        res["configs"] = configs
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w)
        if "c3" in res.get("configs", {}):
            res["configs"]["c3"]["oracle_s_per_chunk"] = res["cpu_baseline"]["seconds"]
    print(json.dumps(res), flush=True)


# steady-state chunks of each config's stream (the rest warm the cache up, or are the short last chunk)
STREAM_STEADY = {
    "tiny": lambda i, w: i >= 5,                                   # evicting from chunk 5 on
    "c2": lambda i, w: True,                                       # keys grow 4680 -> 32760: every chunk
    "c3": lambda i, w: 6 <= i < w.n_chunks - 1,                    # evicting 4680 per chunk
    "c4": lambda i, w: 7 <= i < w.n_chunks - 1,                    # a sink push every chunk
    "c5a": lambda i, w: 1 <= i < w.n_chunks - 1,                   # a clamped shift every chunk, three cuts
    "c5b": lambda i, w: 7 <= i < w.n_chunks - 1,                   # scores + compaction every 4th chunk
}
# the chunk of each stream the oracle is timed on: a steady one (for c5b one that compacts)
STREAM_ORACLE_CHUNK = {"tiny": 6, "c2": 6, "c4": 8, "c5a": 8, "c5b": 7}


class _TimedCache:
    """A KVCache whose library calls are bracketed by events on the cache's stream (per-operation GPU time)."""
    OPS = ("append", "attend", "retime", "score", "compact", "sink_push", "relax_scores")

    def __init__(self, cache, stream, ev):
        self._c, self._s, self._ev, self.log = cache, stream, ev, []

    def __getattr__(self, name):
        f = getattr(self._c, name)
        if name not in self.OPS:
            return f

        def timed(*a, **kw):
            e0, e1 = self._ev(), self._ev()
            e0.record(self._s)
            r = f(*a, **kw)
            e1.record(self._s)
            self.log.append((name, e0, e1, self._c.info()["n_valid"]))
            return r
        return timed


def config_streams(dev, stream, ev, cpu):
    """Every config's whole chunk stream through the product's policy driver (rolling_kv_cache_amd.policies),
    inputs resident in HBM (four seeded chunks of the config's shape, cycled; the stream's own frame
    counts), each chunk and each library call bracketed by events: ms per chunk over the steady-state chunks
    (mean, p10/p50/p90), attention TFLOP/s over all attends, append and retime GB/s (warm: the stream runs
    back to back, no MALL flush).  With `cpu`, the oracle's time for one steady chunk of the same config on
    this host (its earlier chunks replayed with one query row attended, so that only the timed chunk pays
    the full attention)."""
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from rolling_kv_cache_amd.policies import driver_for
    from workloads import WORKLOADS, chunk_inputs
    res = {}
    for name in STREAM_STEADY:
        w = WORKLOADS[name]
        td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        pools = {}
        for F in sorted(set(w.chunk_frames)):
            pools[F] = [tuple(torch.from_numpy(x).to(dev, td) for x in chunk_inputs(w, c, frames=F))
                        for c in range(4)]
        cache = kvc.KVCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, td,
                            bank_frames=w.bank_frames, compact=name.startswith("c5"))
        tc = _TimedCache(cache, stream, ev)
        drv = driver_for(name)(tc, w)
        chunk_ev, q_prev = [], None
        torch.cuda.synchronize()
        for i in range(w.n_chunks):
            q, k, v = pools[w.chunk_frames[i]][i % 4]
            e0, e1 = ev(), ev()
            n0 = len(tc.log)
            e0.record(stream)
            drv.step(i, q, k, v, q_prev=q_prev)
            e1.record(stream)
            chunk_ev.append((e0, e1, n0, len(tc.log)))
            q_prev = q
        torch.cuda.synchronize()
        S, H, D, esz = w.frame_seqlen, w.heads, w.head_dim, 2 if w.dtype == "bf16" else 4
        dtb = D - 4 * (D // 6)
        steady = [i for i in range(w.n_chunks) if STREAM_STEADY[name](i, w)]
        ms = np.array([a.elapsed_time(b) for a, b, _, _ in chunk_ev])
        att_flop = att_ms = app_b = app_ms = ret_b = ret_ms = 0.0
        op_ms = {}
        for i, (_, _, lo, hi) in enumerate(chunk_ev):
            Lq = w.chunk_frames[i] * S
            for op, a, b, n in tc.log[lo:hi]:
                t = a.elapsed_time(b)
                if i in steady:
                    op_ms[op] = op_ms.get(op, 0.0) + t
                if op == "attend":
                    att_flop += 4.0 * H * Lq * n * D
                    att_ms += t
                elif op == "append":
                    app_b += 4.0 * Lq * H * D * esz
                    app_ms += t
        for op, a, b, n in tc.log:
            if op == "retime" and name == "c5a":    # every valid entry's time band, read and written
                ret_b += 2.0 * n * H * dtb * esz
                ret_ms += a.elapsed_time(b)
        st = ms[steady]
        r = {"chunks": w.n_chunks, "steady_chunks": len(steady),
             "ms_per_chunk_mean": round(float(st.mean()), 4),
             "ms_per_chunk_p10_p50_p90": [round(float(x), 4) for x in np.percentile(st, [10, 50, 90])],
             "stream_total_ms": round(float(ms.sum()), 3),
             "attend_tflops": round(att_flop / (att_ms * 1e-3) / 1e12, 4),
             "attend_frac_bf16_peak": round(att_flop / (att_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
             "append_GBps_warm": round(app_b / (app_ms * 1e-3) / 1e9, 1),
             "steady_op_ms_per_chunk": {op: round(t / len(steady), 4) for op, t in sorted(op_ms.items())}}
        if ret_ms > 0:
            r["retime_GBps_warm"] = round(ret_b / (ret_ms * 1e-3) / 1e9, 1)
        if cpu and name in STREAM_ORACLE_CHUNK:
            r["oracle_s_per_chunk"] = oracle_chunk_seconds(w, STREAM_ORACLE_CHUNK[name])
        res[name] = r
        del tc, drv, cache, pools
        torch.cuda.empty_cache()
    return res


def oracle_chunk_seconds(w, i):
    """Wall time of the oracle (untuned numpy) for chunk i of workload w on this host: chunks 0..i-1 are
    replayed first with one query row attended (their cache operations in full), then chunk i runs in full."""
    import numpy as np
    from oracle import make_run
    from workloads import chunk_inputs
    run = make_run(w)
    q_prev = None
    for c in range(i + 1):
        q, k, v = chunk_inputs(w, c % 4, frames=w.chunk_frames[c])
        kw = {"q_prev": q_prev} if w.name.startswith("c5b") else {}
        if c == i:
            t0 = time.perf_counter()
            run.step(c, q, k, v, **kw)
            return round(time.perf_counter() - t0, 4)
        run.step(c, q, k, v, rows=np.arange(1), **kw)
        q_prev = q


def ceilings(dev, stream, ev):
    """This board's own ceilings beside the published peaks (probe kernels of libkvc_probe.so, not the
    product): the sustained bf16 matrix-core rate of v_mfma_f32_32x32x16_bf16 (four independent chains per
    wave, four waves per SIMD on every CU) with the shader clock it ran at (shader-clock cycles over
    constant-rate wall-clock ticks, per workgroup), and plain streaming kernels over 2 GiB buffers (16-byte
    vectors, four in flight per thread, grid-stride): read, copy, write, and copy with non-temporal stores,
    each the best of a few grid sizes (median of 3 runs per size)."""
    import ctypes
    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "rolling_kv_cache_amd", "libkvc_probe.so"))
    vp = ctypes.c_void_p
    lib.kvc_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.kvc_probe_hbm.argtypes = [ctypes.c_int, vp, vp, ctypes.c_size_t, ctypes.c_int, vp, vp]
    lib.kvc_probe_wall_clock_khz.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    sp = vp(stream.cuda_stream)
    out = {}
    blocks, iters = 4 * 256, 4096
    fo = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    tk = torch.zeros(blocks * 2, dtype=torch.int64, device=dev)
    call = lambda: lib.kvc_probe_mfma(blocks, iters, vp(fo.data_ptr()), vp(tk.data_ptr()), sp)
    assert call() == 0
    torch.cuda.synchronize()
    ms = back_to_back_ms(stream, ev, call, n=5)
    flop = blocks * 4.0 * iters * 4 * 32 * 32 * 16 * 2
    khz = ctypes.c_int()
    lib.kvc_probe_wall_clock_khz(torch.cuda.current_device(), ctypes.byref(khz))
    t = tk.view(blocks, 2).cpu().numpy().astype(np.float64)
    clock_mhz = float(np.mean(t[:, 0] / (t[:, 1] / (khz.value * 1e3)))) / 1e6 if khz.value > 0 else None
    out["mfma_bf16_tflops_measured"] = round(flop / (ms * 1e-3) / 1e12, 1)
    out["mfma_clock_mhz_under_load"] = round(clock_mhz, 0) if clock_mhz else None
    if clock_mhz:
        # the same MFMA stream at the nominal 2.4 GHz clock would reach the published peak
        out["mfma_peak_at_measured_clock_tflops"] = round(PEAK_BF16_TFLOPS * clock_mhz / 2400.0, 1)
    del fo, tk
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b.fill_(2)
    sink = torch.empty(16384 * 256, dtype=torch.int32, device=dev)
    flat = {5: "flat", 6: "flat_nt", 7: "flat_inplace"}
    for name, modes, factor in (("read", (0,), 1), ("write", (2,), 1), ("copy", (1, 3, 4, 5, 6), 2),
                                ("inplace_rmw", (7,), 2)):
        best, how = 0.0, None
        for mode in modes:
            for grid in ((1,) if mode in flat else (512, 1024, 2048, 4096, 16384)):
                f = lambda: lib.kvc_probe_hbm(mode, vp(a.data_ptr()), vp(b.data_ptr()), n, grid, vp(sink.data_ptr()),
                                              sp)
                assert f() == 0
                torch.cuda.synchronize()
                gbps = factor * n / (back_to_back_ms(stream, ev, f, n=3) * 1e-3) / 1e9
                if gbps > best:
                    best, how = gbps, flat.get(mode, f"mode {mode}, {grid} workgroups")
        out[f"hbm_{name}_GBps_probe"] = round(best, 1)
        out[f"hbm_{name}_probe_kernel"] = how
    del a, b, sink
    return out


def same_size_ceilings(dev, stream, ev, flush, nbytes_copy, nbytes_inplace):
    """The plain one-element-per-thread probe kernels on exactly a kernel's own traffic, MALL flushed before
    each sample (median of 8): a copy of nbytes_copy (read once, written once: the append's pattern) and an
    in-place read-modify-write of nbytes_inplace (the retime's pattern).  The time such a kernel needs is the
    ceiling the HBM-bound kernels are set against, beside the 8 TB/s spec."""
    import ctypes
    import numpy as np
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "rolling_kv_cache_amd", "libkvc_probe.so"))
    vp = ctypes.c_void_p
    lib.kvc_probe_hbm.argtypes = [ctypes.c_int, vp, vp, ctypes.c_size_t, ctypes.c_int, vp, vp]
    sp = vp(stream.cuda_stream)
    nc = (int(nbytes_copy) + 15) // 16 * 16
    ni = (int(nbytes_inplace) + 15) // 16 * 16
    a = torch.ones(max(nc, ni), dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)

    def cold(f, k=10):
        ts = []
        for i in range(k):
            flush.sum()
            e0, e1 = ev(), ev()
            e0.record(stream)
            assert f() == 0
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))
    cp = cold(lambda: lib.kvc_probe_hbm(5, vp(a.data_ptr()), vp(b.data_ptr()), nc, 1, None, sp))
    ip = cold(lambda: lib.kvc_probe_hbm(7, None, vp(b.data_ptr()), ni, 1, None, sp))
    del a, b
    return cp, ip



def sink_push_and_compact(dev, stream, flush, ev):
    """The remaining data-movement kernels at their workloads' shapes, MALL flushed before each sample:
    a Rolling-Sink push of one 3-frame bank block (12 heads x 1560-token frames, 15 sink + 6 window frames,
    18-frame bank) and a Deep-Forcing compaction keeping the 3-frame sink plus 9360 of 28080 window entries
    (12 heads, 3 sink + 18 window frames); bytes = read + write of K and V for every moved entry.  Then the
    Relax Forcing frame scores of the full cache of that shape; bytes = the keys read."""
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from workloads import WORKLOADS, chunk_inputs

    def cold(fn, n=8):
        ts = []
        for i in range(n):
            fn(i, False)
            flush.sum()
            a, b = ev(), ev()
            a.record(stream)
            fn(i, True)
            b.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(a.elapsed_time(b))
        return float(np.mean(ts)) * 1e3

    out = {}
    w = WORKLOADS["c4"]
    S, H, D = w.frame_seqlen, w.heads, w.head_dim
    chunks = [tuple(torch.from_numpy(x).to(dev, torch.bfloat16) for x in chunk_inputs(w, c)[1:]) for c in range(7)]
    c4 = kvc.KVCache(w.sink_frames, w.window_frames, S, H, D, w.grid_w, torch.bfloat16, bank_frames=w.bank_frames)
    for c in range(7):
        c4.append(*chunks[c], 3 * c)

    def push(i, timed):
        if timed:
            c4.sink_push(3 * (i % 6), 3, 30 + 3 * i)
    us = cold(push)
    byt = 4.0 * 3 * S * H * D * 2
    out["sink_push_us_cold"] = round(us, 2)
    out["sink_push_GBps_cold"] = round(byt / (us * 1e-6) / 1e9, 1)
    del c4

    w = WORKLOADS["c5b"]
    c5 = kvc.KVCache(w.sink_frames, w.window_frames, S, H, D, w.grid_w, torch.bfloat16, compact=True)
    tf = [0]
    ns = w.sink_frames * S
    keep = np.concatenate([np.arange(ns), ns + np.arange(0, 28080, 3)]).astype(np.int32)   # sink + every 3rd

    def fill():
        while c5.info()["n_valid"] < (w.sink_frames + w.window_frames) * S:
            c5.append(*chunks[tf[0] % 7], tf[0] * 3)
            tf[0] += 1

    def comp(i, timed):
        if not timed:
            fill()
        else:
            c5.compact(keep)
    us = cold(comp)
    byt = 4.0 * (len(keep) - ns) * H * D * 2
    out["compact_us_cold"] = round(us, 2)
    out["compact_GBps_cold"] = round(byt / (us * 1e-6) / 1e9, 1)

    # Relax Forcing scores on the full 3 + 18-frame cache (same shape, c5c): 16 candidate frames and a
    # 2-frame Tail, i.e. the keys of 18 frames read once (frame sums), then the Gram matrix and the scores
    sc = torch.empty(64, dtype=torch.float32, device=dev)

    def relax(i, timed):
        if not timed:
            fill()
        else:
            c5.relax_scores(2, 0.5, out=sc)
    us = cold(relax)
    byt = 18.0 * S * H * D * 2
    out["relax_scores_us_cold"] = round(us, 2)
    out["relax_scores_GBps_cold"] = round(byt / (us * 1e-6) / 1e9, 1)
    return out


def per_gpu_share(dev, stream, ev, w):
    """Attention at one GPU's share of the 40-head layer when heads are split over 8 GPUs: 5 heads, the same
    4680 queries over 28080 keys (19 query blocks x 5 heads = 95 workgroups for 256 CUs): split keys (the
    cache reserves the split buffers), and the unsplit launch for comparison."""
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from workloads import chunk_inputs
    S, D, Hs = w.frame_seqlen, w.head_dim, 5
    c = kvc.KVCache(w.sink_frames, w.window_frames, S, Hs, D, w.grid_w, torch.bfloat16, split_attend=True)
    q = None
    for i in range(6):
        q_, k, v = (torch.from_numpy(x[:, :Hs].copy()).to(dev, torch.bfloat16) for x in chunk_inputs(w, i))
        c.append(k, v, 3 * i)
        q = q_
    flop = 4.0 * Hs * q.shape[0] * c.info()["n_valid"] * D
    res = {}
    for tag, no_split in (("", False), ("_unsplit", True)):
        c.set_paths(no_split=no_split)
        try:
            out = c.attend(q, 15)
            torch.cuda.synchronize()
            ms = back_to_back_ms(stream, ev, lambda: c.attend(q, 15, out=out))
        finally:
            c.set_paths()
        res[f"attend_5head_share{tag}_ms"] = round(ms, 4)
        res[f"attend_5head_share{tag}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
    return res


def head_dim_64(dev, stream, ev, w):
    """The C3 step's attention and a 3-frame score window at head_dim 64 (40 heads, 4680 queries over the
    28080-key cache, bf16): the head_dim-64 matrix-core kernels."""
    import torch
    import rolling_kv_cache_amd as kvc
    from workloads import Workload, chunk_inputs
    w64 = Workload("c3_d64", 230, w.heads, 64, "bf16", w.grid_h, w.grid_w, w.sink_frames, w.window_frames, (3,) * 7)
    S, H, D = w64.frame_seqlen, w64.heads, w64.head_dim
    c = kvc.KVCache(w64.sink_frames, w64.window_frames, S, H, D, w64.grid_w, torch.bfloat16)
    q = None
    for i in range(7):
        q_, k, v = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in chunk_inputs(w64, i % 3))
        c.append(k, v, 3 * i)
        q = q_
    Lk = c.info()["n_valid"]
    flop = 4.0 * H * q.shape[0] * Lk * D
    out = c.attend(q, 18)
    sc = c.score(q, [18, 19, 20])
    torch.cuda.synchronize()
    ms = back_to_back_ms(stream, ev, lambda: c.attend(q, 18, out=out))
    sms = back_to_back_ms(stream, ev, lambda: c.score(q, [18, 19, 20], out=sc), n=6)
    return {"attend_d64_ms": round(ms, 4), "attend_d64_tflops": round(flop / (ms * 1e-3) / 1e12, 1),
            "score_d64_ms": round(sms, 4)}


def block_causal_clip(dev, stream, ev, w, block_frames=3):
    """Block-causal attention of the Wan-1.3B 21-frame clip (32760 query rows, 12 heads) over the cache
    that holds it, in blocks of 3 frames: block b's 4680 rows see (b + 1) * 4680 keys."""
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from workloads import chunk_inputs
    S, D, H, F = w.frame_seqlen, w.head_dim, w.heads, w.total_frames
    c = kvc.KVCache(w.sink_frames, w.window_frames, S, H, D, w.grid_w, torch.bfloat16)
    for i in range(w.n_chunks):
        _, k, v = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in chunk_inputs(w, i))
        c.append(k, v, w.chunk_start_frame(i))
    (q,) = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in chunk_inputs(w, 99, tensors=(0,), frames=F))
    out = c.attend_block_causal(q, 0, block_frames)
    torch.cuda.synchronize()
    ms = back_to_back_ms(stream, ev, lambda: c.attend_block_causal(q, 0, block_frames, out=out), n=8)
    cb = block_frames * S
    n = c.info()["n_valid"]
    vis = sum(min(n, (r // cb + 1) * cb) * min(cb, F * S - r) for r in range(0, F * S, cb))
    flop = 4.0 * H * D * vis
    return {"block_causal_clip_ms": round(ms, 4), "block_causal_clip_tflops": round(flop / (ms * 1e-3) / 1e12, 1)}


def raw_keys_ab(dev, stream, ev, flush, w):
    """The bench chunk on a raw-key cache (same 40-head, 28080-key shape): each attend first places every
    key's time band at its slot's current time in one pass over the time-band plane, then runs the plain
    attention kernels; a retime of the whole cache only rewrites 28080 time indices."""
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from workloads import chunk_inputs
    S, H, D = w.frame_seqlen, w.heads, w.head_dim
    c = kvc.KVCache(w.sink_frames, w.window_frames, S, H, D, w.grid_w, torch.bfloat16, raw_keys=True)
    q = None
    for i in range(6):
        q_, k, v = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in chunk_inputs(w, i % 4))
        c.append(k, v, 3 * i)
        q = q_
    out = c.attend(q, 15)
    torch.cuda.synchronize()
    ms = back_to_back_ms(stream, ev, lambda: c.attend(q, 15, out=out))
    flop = 4.0 * H * q.shape[0] * c.info()["n_valid"] * D
    rt = []
    for i in range(10):
        flush.sum()
        a, b = ev(), ev()
        a.record(stream)
        c.retime(1 if i % 2 == 0 else -1)
        b.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            rt.append(a.elapsed_time(b) * 1e3)
    return {"raw_attend_ms": round(ms, 4), "raw_attend_tflops": round(flop / (ms * 1e-3) / 1e12, 1),
            "raw_retime_us_cold": round(float(np.mean(rt)), 2)}


def memrope_chunk(dev, stream, ev, flush, w):
    """MemRoPE at its workload's shape (12 heads, 3 sink + 18 window frames, raw keys, memories at rates
    0.9 / 0.5), MALL flushed: an append that evicts 3 frames (their fold into both memories, then the write)
    next to the same append on a raw-key cache without memory; and the chunk's attention over sink + 2
    memory frames + window (35880 keys)."""
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from workloads import chunk_inputs
    S, H, D = w.frame_seqlen, w.heads, w.head_dim
    chunks = [tuple(torch.from_numpy(x).to(dev, torch.bfloat16) for x in chunk_inputs(w, c)) for c in range(4)]
    out = {}
    for tag, mem in (("memory", w.memory), ("plain", None)):
        c = kvc.KVCache(w.sink_frames, w.window_frames, S, H, D, w.grid_w, torch.bfloat16, raw_keys=True,
                        memory=mem)
        for i in range(8):
            c.append(chunks[i % 4][1], chunks[i % 4][2], 3 * i)
        ts = []
        for i in range(10):
            flush.sum()
            a, b = ev(), ev()
            a.record(stream)
            c.append(chunks[i % 4][1], chunks[i % 4][2], 24 + 3 * i)
            b.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(a.elapsed_time(b) * 1e3)
        out[f"memrope_append_{tag}_us_cold"] = round(float(np.mean(ts)), 2)
        if mem is not None:
            q = chunks[0][0]
            o = c.attend(q, 54)
            torch.cuda.synchronize()
            ms = back_to_back_ms(stream, ev, lambda: c.attend(q, 54, out=o), n=8)
            nk = c.info()["n_valid"] + 2 * S
            out["memrope_attend_ms"] = round(ms, 4)
            out["memrope_attend_tflops"] = round(4.0 * H * q.shape[0] * nk * D / (ms * 1e-3) / 1e12, 1)
        del c
    return out


def layer_group(dev, stream, ev, flush, w, L=30):
    """A 30-layer group at the Wan-1.3B shape (12 heads, 3 sink + 18 window frames, full: 32760 entries per
    layer, 6 GB in all).  MALL flushed: one Infinity-RoPE shift of every layer (clamped, -3 frames) as one
    launch vs 30 single-layer launches.  Then one chunk of the denoise loop: 4 sampling passes and the commit,
    each pass appending (pass 0) or re-writing the 3-frame chunk and attending, layer after layer."""
    import numpy as np
    import torch
    import rolling_kv_cache_amd as kvc
    from rolling_kv_cache_amd.policies import DenoiseLoop
    from workloads import chunk_inputs
    S, H, D = w.frame_seqlen, w.heads, w.head_dim
    caches = kvc.create_group(L, w.sink_frames, w.window_frames, S, H, D, w.grid_w, torch.bfloat16)
    chunk = [tuple(torch.from_numpy(x).to(dev, torch.bfloat16) for x in chunk_inputs(w, c)) for c in range(2)]
    for i in range(7):
        for c in caches:
            c.append(chunk[i % 2][1], chunk[i % 2][2], 3 * i)
    torch.cuda.synchronize()

    def cold(fn, n=6):
        ts = []
        for i in range(n):
            flush.sum()
            a, b = ev(), ev()
            a.record(stream)
            fn(i)
            b.record(stream)
            torch.cuda.synchronize()
            if i >= 1:
                ts.append(a.elapsed_time(b) * 1e3)
        return float(np.mean(ts))

    batched = cold(lambda i: kvc.retime_layers(caches, -3 if i % 2 == 0 else 3, i % 2 == 0))
    single = cold(lambda i: [c.retime(-3 if i % 2 == 0 else 3, i % 2 == 0) for c in caches])
    loop = DenoiseLoop(caches, w)
    q, k, v = chunk[0]
    for c in caches:
        c.retime(0)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(stream)
    for s in range(5):
        for layer in range(L):
            loop.pass_layer(7, layer, s, q, k, v)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    n = caches[0].info()["n_valid"]
    flop = 5 * L * 4.0 * H * q.shape[0] * n * D
    del caches
    return {"group30_retime_batched_us_cold": round(batched, 1), "group30_retime_per_layer_us_cold": round(single, 1),
            "denoise_chunk_30_layers_ms": round(ms, 2),
            "denoise_chunk_attend_tflops": round(flop / (ms * 1e-3) / 1e12, 1)}


def vendor_context(dev, stream, H, N, Lk, D):
    """Reference points on the same board (not the product path): torch's fused attention at the same
    shape (same flop count, no cache or RoPE), and a plain bf16 GEMM through torch (hipBLASLt)."""
    import numpy as np
    import torch

    def timed(fn, n=10):
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))

    out = {}
    try:
        from torch.nn.attention import sdpa_kernel, SDPBackend
        q = torch.randn(1, H, N, D, device=dev, dtype=torch.bfloat16)
        k = torch.randn(1, H, Lk, D, device=dev, dtype=torch.bfloat16)
        v = torch.randn(1, H, Lk, D, device=dev, dtype=torch.bfloat16)
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            ms = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v))
        out["torch_sdpa_flash_tflops"] = round(4.0 * H * N * Lk * D / (ms * 1e-3) / 1e12, 1)
        del q, k, v
    except Exception as e:  # flash backend not available in this torch
        out["torch_sdpa_flash_error"] = str(e)[:120]
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    ms = timed(lambda: torch.mm(a, b))
    out["torch_gemm_bf16_8192_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    return out


def cpu_baseline(w):
    """The oracle, untuned, on this host: one full steady chunk of the bench workload (chunk 7: the
    append that evicts 4680 entries, then the attention of all 4680 queries x 40 heads over the 28080
    cached keys, fp32 numpy BLAS), after its chunks 0-6 were replayed with one query row attended; reported
    as the chunk's attention flop over its wall time, like the GPU's value."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info() if t.get("user_api") == "blas"] or [1])
    except Exception:
        threads = None
    cores = len(os.sched_getaffinity(0))
    sec = oracle_chunk_seconds(w, 7)
    N = w.chunk_frames[7] * w.frame_seqlen
    flop = 4.0 * w.heads * N * w.capacity * w.head_dim
    return {"value": round(flop / sec / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "blas_threads": threads, "seconds": sec,
            "sample": f"one full steady chunk of the c3 stream (chunk 7: append evicting {N} entries + attention "
                      f"of {N} queries x {w.heads} heads over {w.capacity} keys, incl. the RoPE of keys and "
                      f"queries), fp32 numpy BLAS; chunks 0-6 replayed first with one query row attended"}


if __name__ == "__main__":
    main()
