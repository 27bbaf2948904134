"""Benchmark: FP4-KV chunk attention, latent frames/s per layer, on one GPU.

One step = the whole hot path for one chunk of one attention layer, in
steady state (sink + full window):
    fp4kv_rope_append(Q, K, V) -> fp4kv_attention_chunk
(the queries' rotation and the NVFP4 append in one pass for these bf16
inputs, then attention) on seeded synthetic inputs already resident in
device memory.  The stream keeps going (the ring wraps); inputs rotate over
16 sets (8 seeded draws and their negations, 690 MB for the 1.3B-like
layer, more than the 256 MB Infinity Cache holds).  Before the W warmup
steps the cache is filled by streaming untimed steps for at least FILL_MS,
which outlasts the clock ramp that follows the host-side input draw.

Workload (default): one layer shaped like the 1.3B generator: 12 heads,
head_dim 128, 1560 tokens/frame, chunk 3 frames, sink 3 + window 12 frames,
bf16 inputs ~N(0,1) with 1% outliers x20.  --workload picks another.

Printed: one JSON line.  value = frames/s of one layer = C * K / time of K
steps.  roofline = the attention kernel (the dominant one): algorithmic
FLOP per launch (4*D per (query, key) pair the masks keep) / its mean
duration from HIP events on the launch stream, against the 2.5 PFLOP/s
dense f16/bf16 MFMA peak.  roofline_codec = the step's codec kernel as
timed inside the steps (rotation + append): algorithmic bytes (queries read
and written as float32, kept K and V read once, codes and scales written
once) / their mean duration, against 8 TB/s.  codec = the append alone and
the fused call by the cold protocol (inputs rotating over the sets) and
hot (one set), beside a plain copy of the same K and V bytes.  configs = the
5B-like, multi-shot and long-stream layers at steady state.  cpu_baseline =
the CPU oracle on a bounded sample of the same step.

--kv nvfp4_rot stores keys rotated; the step becomes
    fp4kv_quantize_append_rotated(K, V) -> fp4kv_rope_rel_frames(Q) -> fp4kv_attention_chunk
and roofline_codec covers the first two (the cache update with the
re-encoding of the window keys that survive the window move, and the
rotation).  --kv bf16 is the unquantized baseline cache.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0
METRIC = "FP4-KV chunk attention latent frames/s per layer; HBM GB/s & MFMA % of peak"
# Wall time of the untimed steps that fill the cache before the warmup
# steps (at least the steps that fill the sink and window): past the ~25 ms
# clock ramp that follows the host-side input draw.
FILL_MS = 60.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="l13b")
    ap.add_argument("--kv", default="nvfp4", choices=("nvfp4", "nvfp4_rot", "bf16"),
                    help="cache format: NVFP4 with keys stored before rotation (the path), "
                         "NVFP4 with keys stored rotated (re-rotated when the window "
                         "moves), or the bf16 baseline")
    ap.add_argument("--sink-per-shot", action="store_true",
                    help="per-shot attention sinks (each shot re-anchors the sink)")
    ap.add_argument("--workgroups", type=int, default=0,
                    help="attention workgroups (0: the library's default, one per compute unit "
                         "with at least 4 key tiles each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the codec protocol and the other configurations (profiling runs)")
    ap.add_argument("--traffic-json", default=None,
                    help="per-launch HBM bytes measured with rocprofv3 counters "
                         "(default: profiles/traffic_<workload>.json)")
    ap.add_argument("--codec-sweep", action="store_true",
                    help="only time the append at 3, 6 and 15 frames of the workload next to "
                         "plain device copies of similar sizes, print one JSON line, and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (5 times), to calibrate the "
                         "FETCH_SIZE / WRITE_SIZE counters, and exit")
    return ap.parse_args()


def attention_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("attention.hip", "fp4kv_device.hpp", "internal.hpp"):
        h.update(open(os.path.join(ROOT, "fp4_kv_cache_fp4kv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def copy_calibration(nbytes):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "launches": 5}), flush=True)


def codec_sweep(w):
    """Append bandwidth against size, next to what a plain device copy reaches
    at similar sizes.  A chunk of the step's size takes the one-pass append
    (K and V read once); the larger ones, more than its grid holds, take the
    two kernels (partial maxima, then the encode, which reads K and V a
    second time).  Both are timed with HIP events over 30 calls on the same resident
    inputs, so sizes up to ~100 MB stay in the 256 MB Infinity Cache between
    calls (hot numbers); the benchmark's own step rotates 8 input sets, more
    than the Infinity Cache holds."""
    import torch

    from fp4_kv_cache_fp4kv_amd import api

    def tm(fn, reps=30):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3     # microseconds

    out = {"workload": workload_desc(w), "copy": {}, "append": {}}
    for mb in (37, 74, 184, 512):                   # read mb, write mb
        src = torch.empty(mb * 500_000, dtype=torch.bfloat16, device="cuda:0").normal_()
        dst = torch.empty_like(src)
        us = tm(lambda: dst.copy_(src))
        out["copy"][f"{mb}MB"] = {"us": round(us, 2), "GB/s": round(2 * mb * 1e6 / us / 1e3, 1)}
        del src, dst
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride)
    es = 2 if w.dtype == "bf16" else 4
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    for nf in sorted({w.C, 2 * w.C, w.S + w.W}):
        k = torch.randn(nf * w.T, w.H, w.D, device="cuda:0").to(dt)
        v = torch.randn(nf * w.T, w.H, w.D, device="cuda:0").to(dt)
        us = tm(lambda: api.quantize_append(gc, k, v, 0, nf, [0] * nf))
        kept = 2 * nf * w.Tc * w.H * w.D
        b = kept * es + kept * (0.5 + 1.0 / 16.0)
        out["append"][f"{nf}_frames"] = {"us": round(us, 2), "MB": round(b / 1e6, 1),
                                         "GB/s": round(b / us / 1e3, 1)}
    print(json.dumps(out), flush=True)


def workload_desc(w):
    out = (f"{w.name}: H{w.H} D{w.D} T{w.T} C{w.C} S{w.S} W{w.W}"
           + (f" token_stride {w.token_stride}" if w.token_stride > 1 else "")
           + (f" shots of {w.shot_len} frames" if w.shot_len else "")
           + (f", {w.outlier_p:.0%} outliers x{w.outlier_scale:g}" if w.outlier_p else ""))
    return out


def cpu_baseline(w):
    """The oracle as it stands on all heads of steady-state steps (append of
    the step's K/V chunk plus attention of all its query rows), repeated until
    about 10 s of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from fp4_kv_cache_fp4kv_amd import workloads as wl
    from oracle.stream import OracleCache

    first = -(-(w.S + w.W) // w.C)        # first chunk step with a full window
    one = wl.Workload(w.name + "_sample", H=w.H, D=w.D, T=w.T, C=w.C, S=w.S, W=w.W,
                      n_frames=(first + 3) * w.C, seed=w.seed, dtype=w.dtype,
                      outlier_p=w.outlier_p, outlier_scale=w.outlier_scale,
                      shot_len=w.shot_len, token_stride=w.token_stride)
    oc = OracleCache.for_workload(one)
    for c in range(first):
        f0, n = one.chunk_frames(c)
        (_, _), (k, _), (v, _) = wl.draw_qkv(one, c)
        oc.append(k, v, f0, n, [one.shot_of(f) for f in range(f0, f0 + n)])
    dt, steps = 0.0, 0
    for c in range(first, one.n_chunks):
        f0, n = one.chunk_frames(c)
        (q, _), (k, _), (v, _) = wl.draw_qkv(one, c)
        shots = [one.shot_of(f) for f in range(f0, f0 + n)]
        t0 = time.perf_counter()
        oc.append(k, v, f0, n, shots)
        oc.attention(q, f0, n, shots)
        dt += time.perf_counter() - t0
        steps += 1
        if dt >= 10.0:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(steps * w.C / dt, 4), "unit": "latent frames/s per layer",
            "cores": threads, "kind": "oracle",
            "sample": f"{steps} steady-state step(s), all {w.H} heads (append + attention of "
                      f"{w.C * w.T} query rows over {(w.S + w.W) * w.Tc} keys per head), "
                      f"{dt:.1f} s"}


def visible_pairs(w, f0, per_shot, shot_start):
    """Number of (query frame, key frame) pairs attended at the chunk step
    starting at frame f0 (sink + window, block-causal and shot masks)."""
    f1 = f0 + w.C
    ws = max(w.S, f1 - w.W)
    n = 0
    for qf in range(f0, f1):
        for kf in range(f1):
            if kf // w.C > qf // w.C:
                continue
            same = w.shot_of(kf) == w.shot_of(qf)
            if per_shot:
                rel = kf - shot_start(kf)
                # the sink slot of a frame is taken over by a later shot's
                later = any(g - shot_start(g) == rel for g in range(kf + 1, f1)) if rel < w.S else False
                ok = same and ((rel < w.S and not later) or (rel >= w.S and kf >= ws))
            else:
                ok = (kf < w.S) or (kf >= ws and same)
            n += ok
    return n


def surviving_window_frames(w, f0, per_shot, shot_start):
    """Window frames whose stored rotation moves at the chunk step starting at
    frame f0 (keys stored rotated): frames in window slots that stay in the
    window while its start moves."""
    ws0, ws1 = max(w.S, f0 - w.W), max(w.S, f0 + w.C - w.W)
    if ws1 == ws0:
        return 0
    return sum(1 for f in range(ws1, f0)
               if not (per_shot and f - shot_start(f) < w.S))


def draw_sets(w, n_base, dev):
    """2 * n_base input sets (Q, K, V) of one chunk in device memory: n_base
    seeded draws and their negations (same statistics, other bytes), so
    that a set is cold in the 256 MB Infinity Cache when it comes round."""
    import numpy as np
    import torch

    from fp4_kv_cache_fp4kv_amd import workloads as wl

    def dev_t(vals, bits):
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(vals).to(dev)

    n_tok = w.C * w.T
    sets = [tuple(dev_t(*wl.draw(w, c, tid, n_tokens=n_tok)) for tid in (wl.Q_ID, wl.K_ID, wl.V_ID))
            for c in range(n_base)]
    return sets + [tuple(torch.neg(t) for t in s) for s in sets]


def shot_start_fn(w):
    def shot_start(f):
        s0 = w.shot_of(f)
        while f > 0 and w.shot_of(f - 1) == s0:
            f -= 1
        return f
    return shot_start


def measure(w, steps, warmup, sets, kv="nvfp4", sink_per_shot=False, workgroups=0):
    """Steady-state steps of one layer: the cache update (with the queries'
    rotation when it is fused) and attention, each bracketed by HIP events
    on the launch stream (one event between consecutive kernels); the whole
    K steps bracketed by synchronizations."""
    import torch

    from fp4_kv_cache_fp4kv_amd import api

    dev = torch.device("cuda:0")
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, device="cuda:0",
                        kv_format=kv, sink_per_shot=sink_per_shot)
    shot_start = shot_start_fn(w)
    qrot = torch.empty((w.C * w.T, w.H, w.D), dtype=torch.float32, device=dev)
    out = torch.empty((w.C * w.T, w.H, w.D), dtype=torch.bfloat16, device=dev)
    rot = kv == "nvfp4_rot"
    fused = kv == "nvfp4"   # one rope_append call: rotation fused with the amax pass
    first = -(-(w.S + w.W) // w.C)       # first chunk step with a full window
    # Event chain over the timed steps: b_t | cache update | m_t | attention
    # | b_{t+1}.  Each event ends one kernel's interval and starts the next
    # (they are back to back on the stream); b_0 and b_K are the events that
    # bracket the whole timed region.
    ev = {"b": [], "m": []}

    def step(c, record):
        q, k, v = sets[c % len(sets)]
        f0 = c * w.C
        shots = [w.shot_of(f) for f in range(f0, f0 + w.C)]
        fss = [shot_start(f) for f in range(f0, f0 + w.C)] if sink_per_shot else None
        if fused:   # the queries' rotation and the append in one call (one kernel here)
            api.rope_append(gc, q, k, v, f0, w.C, shots, shot_starts=fss, q_out=qrot)
        elif rot:   # turn the surviving window keys, store the new keys rotated
            api.quantize_append_rotated(gc, k, v, f0, w.C, shots, shot_starts=fss)
        else:
            api.quantize_append(gc, k, v, f0, w.C, shots, shot_starts=fss)
        if not fused:
            api.rope_rel_frames(gc, q, f0, w.C, shot_starts=fss, out=qrot)
        if record:
            ev["m"].append(torch.cuda.Event(enable_timing=True))
            ev["m"][-1].record()
        api.attention_chunk(gc, qrot, f0, w.C, shots, out=out, n_workgroups=workgroups)
        if record and len(ev["m"]) < steps:   # the last step ends at t1
            ev["b"].append(torch.cuda.Event(enable_timing=True))
            ev["b"][-1].record()

    # Fill the sink and window, streaming untimed steps for at least FILL_MS
    # of wall time: the clocks ramp for ~25 ms after the host-side input
    # draw leaves the device idle, and the fill is where that ramp is spent
    # (the W warmup steps and the K timed steps follow as asked).
    import time
    t_fill = time.perf_counter()
    c = 0
    while c < first or time.perf_counter() - t_fill < FILL_MS * 1e-3:
        for _ in range(8):
            step(c, False)
            c += 1
        torch.cuda.synchronize()
    n_fill = c
    for _ in range(warmup):
        step(c, False)
        c += 1
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step(c, True)
        c += 1
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    bounds = [t0] + ev["b"] + [t1]                # b_0 .. b_K
    attn_each = sorted(m.elapsed_time(b) for m, b in zip(ev["m"], bounds[1:]))
    update_ms = sum(b.elapsed_time(m) for b, m in zip(bounds[:-1], ev["m"])) / steps
    f0s = [(c - steps + i) * w.C for i in range(steps)]
    # useful FLOP: only the (query frame, key frame) pairs the masks keep,
    # averaged over the timed steps (equal to 4 H Nq Nk D without shots)
    pairs = [visible_pairs(w, f0, sink_per_shot, shot_start) for f0 in f0s]
    flops = 4.0 * w.H * w.T * w.Tc * w.D * sum(pairs) / len(pairs)
    attn_ms = sum(attn_each) / steps
    es = 2 if w.dtype == "bf16" else 4
    kept = 2 * w.C * w.Tc * w.H * w.D
    update_bytes = kept * es + kept * (2.0 if kv == "bf16" else 0.5 + 1.0 / 16.0)
    q_elems = w.C * w.T * w.H * w.D
    update_bytes += q_elems * (es + 4)      # the queries: read, written as float32
    if rot:
        # the re-encoding of the surviving window keys (their codes and
        # scales read and written once)
        surv = [surviving_window_frames(w, f0, sink_per_shot, shot_start) for f0 in f0s]
        key_frame = w.H * w.Tc * (w.D // 2 + w.D // 16)
        update_bytes += 2.0 * key_frame * sum(surv) / len(surv)
    del gc
    return {"ms_step": ms_step, "attn_ms": attn_ms, "attn_each": attn_each, "fill": n_fill,
            "update_ms": update_ms, "update_bytes": update_bytes, "flops": flops,
            "pairs": sum(pairs) / len(pairs)}


def time_calls(fn, n_calls, reps=3):
    """Mean microseconds per call of fn(i), i = 0 .. n_calls - 1, from HIP
    events on the current stream around the whole loop (best of reps)."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_calls):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n_calls * 1e3
        best = us if best is None else min(best, us)
    return best


def codec_measure(w, sets):
    """The codec at the per-step size by the cold-cache protocol: inputs
    rotate over the sets (cold) or repeat one set (hot); beside them a plain
    device copy of the appended K and V bytes (the practical ceiling), cold
    over as many buffers as the sets and hot."""
    import torch

    from fp4_kv_cache_fp4kv_amd import api

    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, device="cuda:0")
    es = 2 if w.dtype == "bf16" else 4
    kept = 2 * w.C * w.Tc * w.H * w.D
    append_bytes = kept * es + kept * (0.5 + 1.0 / 16.0)
    q_elems = w.C * w.T * w.H * w.D
    prologue_bytes = append_bytes + q_elems * (es + 4)
    qrot = torch.empty((w.C * w.T, w.H, w.D), dtype=torch.float32, device="cuda:0")
    shots = [0] * w.C
    n = len(sets)

    def app(i, cold):
        q, k, v = sets[i % n if cold else 0]
        api.quantize_append(gc, k, v, 0, w.C, shots)

    def pro(i, cold):
        q, k, v = sets[i % n if cold else 0]
        api.rope_append(gc, q, k, v, 0, w.C, shots, q_out=qrot)

    res = {}
    for name, fn, b in (("append", app, append_bytes), ("rope_append", pro, prologue_bytes)):
        cold = time_calls(lambda i: fn(i, True), 4 * n)
        hot = time_calls(lambda i: fn(i, False), 4 * n)
        res[name] = {"bytes": int(b), "cold_us": round(cold, 2), "hot_us": round(hot, 2),
                     "cold_GBs": round(b / cold / 1e3, 1), "hot_GBs": round(b / hot / 1e3, 1),
                     "cold_frac": round(b / cold / 1e3 / HBM_PEAK_GBS, 4),
                     "hot_frac": round(b / hot / 1e3 / HBM_PEAK_GBS, 4)}
    # plain copy of the appended K and V (read and written once each)
    nbytes = kept * es
    srcs = [torch.empty(nbytes // 2, dtype=torch.int16, device="cuda:0").fill_(i) for i in range(n)]
    dsts = [torch.empty_like(srcs[0]) for _ in range(n)]
    cold = time_calls(lambda i: dsts[i % n].copy_(srcs[i % n]), 4 * n)
    hot = time_calls(lambda i: dsts[0].copy_(srcs[0]), 4 * n)
    res["copy"] = {"bytes": int(2 * nbytes), "cold_us": round(cold, 2), "hot_us": round(hot, 2),
                   "cold_GBs": round(2 * nbytes / cold / 1e3, 1),
                   "hot_GBs": round(2 * nbytes / hot / 1e3, 1)}
    res["sets"] = n
    res["set_MB"] = round(sum(t.numel() * t.element_size() for t in sets[0]) / 1e6, 1)
    del gc, srcs, dsts
    torch.cuda.empty_cache()
    return res


def summary(w, m):
    tflops = m["flops"] / (m["attn_ms"] * 1e-3) / 1e12
    return {"workload": workload_desc(w), "ms_per_step": round(m["ms_step"], 4),
            "frames_per_s": round(w.C / (m["ms_step"] * 1e-3), 1),
            "attention_ms": round(m["attn_ms"], 4),
            "attention_only_frames_per_s": round(w.C / (m["attn_ms"] * 1e-3), 1),
            "useful_TFLOPs": round(tflops, 1), "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
            "frame_pairs_per_step": round(m["pairs"], 2),
            "update_ms": round(m["update_ms"], 4),
            "update_frac": round(m["update_bytes"] / (m["update_ms"] * 1e-3) / 1e9
                                 / HBM_PEAK_GBS, 4)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.codec_sweep:
        from fp4_kv_cache_fp4kv_amd import workloads as wl
        codec_sweep(wl.WORKLOADS[args.workload])
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by head or by time, see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    from fp4_kv_cache_fp4kv_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    sets = draw_sets(w, 8, dev)
    m = measure(w, args.steps, args.warmup, sets, args.kv, args.sink_per_shot, args.workgroups)
    pct = lambda v, q: v[min(len(v) - 1, int(q * len(v)))]
    attn_tflops = m["flops"] / (m["attn_ms"] * 1e-3) / 1e12
    update_gbs = m["update_bytes"] / (m["update_ms"] * 1e-3) / 1e9

    # HBM bytes per attention launch from rocprofv3 counters, valid only for
    # the kernel source they were taken on
    traffic = None
    try:
        tj = json.load(open(args.traffic_json or
                            os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")))
        if (tj.get("workload") == w.name and tj.get("source_hash") == attention_source_hash()
                and args.kv == "nvfp4" and not args.sink_per_shot):
            traffic = tj.get("attention_bytes_per_launch")
    except (OSError, ValueError):
        pass

    rot = args.kv == "nvfp4_rot"
    Nq, Nk = w.C * w.T, (w.S + w.W) * w.Tc
    res = {
        "metric": METRIC,
        "value": round(w.C / (m["ms_step"] * 1e-3), 3),
        "unit": "latent frames/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": workload_desc(w), "kv_format": args.kv,
                   "sink": "per_shot" if args.sink_per_shot else "stream", "query_rows": Nq,
                   "workgroups": args.workgroups or "default",
                   "keys": Nk, "input_sets": len(sets), "fill_steps": m["fill"],
                   "frames_per_step": w.C, "attention_ms": round(m["attn_ms"], 4),
                   "attention_only_frames_per_s": round(w.C / (m["attn_ms"] * 1e-3), 1),
                   "attention_ms_p10_p50_p90": [round(pct(m["attn_each"], q), 4)
                                                for q in (0.1, 0.5, 0.9)],
                   ("cache_update_ms" if rot else "rope_append_ms"): round(m["update_ms"], 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic},
        # the step's codec kernels as timed inside the steps: for the NVFP4
        # path the queries' rotation fused with the append (one pass,
        # prologue_kernel, for the bf16 inputs here); bytes = queries read and
        # written as float32, kept K and V read once, codes and scales written
        # once
        "roofline_codec": {"bound": "hbm", "achieved": round(update_gbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(update_gbs / HBM_PEAK_GBS, 4),
                           "bytes": int(m["update_bytes"]),
                           "kernels": {"nvfp4": "prologue_kernel (one pass, bf16 inputs)",
                                       "nvfp4_rot": "amax_kernel + encode_kernel + rope_kernel",
                                       "bf16": "store_bf16_kernel + rope_kernel"}[args.kv]},
    }
    if args.kv == "nvfp4" and not args.no_extra:
        res["codec"] = codec_measure(w, sets)
    del sets
    torch.cuda.empty_cache()
    if args.kv == "nvfp4" and not args.no_extra and args.workload == "l13b":
        # the other full-size configurations, each at steady state
        configs = {}
        for name, per_shot in (("l5b", False), ("l5b_shots", False), ("long", False)):
            wc = wl.WORKLOADS[name]
            sc = draw_sets(wc, 4, dev)
            mc = measure(wc, 20, 3, sc, "nvfp4", per_shot, args.workgroups)
            configs[name] = summary(wc, mc)
            configs[name]["codec"] = codec_measure(wc, sc)
            del sc
            torch.cuda.empty_cache()
        res["configs"] = configs
    if not args.no_cpu_baseline and args.kv == "nvfp4":
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
