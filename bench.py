"""Benchmark: FP4-KV chunk attention, latent frames/s per layer, on one GPU.

One step = the whole hot path for one chunk of one attention layer, in
steady state (sink + full window):
    fp4kv_rope_rel(Q) -> fp4kv_quantize_append(K, V) -> fp4kv_attention_chunk
on seeded synthetic inputs already resident in device memory.  The stream
keeps going (the ring wraps); inputs rotate over 8 pre-drawn chunks.

Workload (default): one layer shaped like the 1.3B generator: 12 heads,
head_dim 128, 1560 tokens/frame, chunk 3 frames, sink 3 + window 12 frames,
bf16 inputs ~N(0,1) with 1% outliers x20.  --workload picks another.

Printed: one JSON line.  value = frames/s of one layer = C * K / time of K
steps.  roofline = the attention kernel (the dominant one): algorithmic
FLOP per launch (4*D per (query, key) pair the masks keep) / its mean
duration from HIP events on the launch stream, against the 2.5 PFLOP/s
dense f16/bf16 MFMA peak.  roofline_codec = the two append kernels:
algorithmic bytes (kept K and V read once, codes and scales written once)
/ their mean duration, against 8 TB/s.  cpu_baseline = the CPU oracle on a
bounded sample of the same step.

--kv nvfp4_rot stores keys rotated; the step becomes
    fp4kv_quantize_append_rotated(K, V) -> fp4kv_rope_rel(Q) -> fp4kv_attention_chunk
and roofline_codec covers the first (the cache update: the append plus the
re-encoding of the window keys that survive the window move).
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
    at similar sizes: the ceiling a two-pass append can approach at a given
    size.  Both are timed with HIP events over 30 calls on the same resident
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

    import numpy as np
    import torch

    from fp4_kv_cache_fp4kv_amd import api
    from fp4_kv_cache_fp4kv_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, device="cuda:0",
                        kv_format=args.kv, sink_per_shot=args.sink_per_shot)

    def shot_start(f):
        s0 = w.shot_of(f)
        while f > 0 and w.shot_of(f - 1) == s0:
            f -= 1
        return f

    def dev_t(vals, bits):
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(vals).to(dev)

    n_sets = 8
    sets = []
    n_tok = w.C * w.T
    for c in range(n_sets):
        sets.append(tuple(dev_t(*wl.draw(w, c, tid, n_tokens=n_tok))
                          for tid in (wl.Q_ID, wl.K_ID, wl.V_ID)))
    qrot = torch.empty((w.C * w.T, w.H, w.D), dtype=torch.float32, device=dev)
    rot = args.kv == "nvfp4_rot"
    out = torch.empty((w.C * w.T, w.H, w.D), dtype=torch.bfloat16, device=dev)
    first = -(-(w.S + w.W) // w.C)       # first chunk step with a full window

    ev = {k: [] for k in ("a0", "a1", "c0", "c1")}

    def step(c, record):
        q, k, v = sets[c % n_sets]
        f0 = c * w.C
        shots = [w.shot_of(f) for f in range(f0, f0 + w.C)]
        fss = [shot_start(f) for f in range(f0, f0 + w.C)] if args.sink_per_shot else None
        def rope(x, y):
            if fss is None:
                api.rope_rel(x, api.cache_positions(w.S, w.W, f0, w.C), w.T, gc.cos_sin, out=y)
            else:   # per-frame positions (a cut inside the chunk breaks the sequence)
                for j in range(w.C):
                    rows = slice(j * w.T, (j + 1) * w.T)
                    api.rope_rel(x[rows], api.frame_position(w.S, w.W, f0 + j, f0 + w.C, fss[j]),
                                 w.T, gc.cos_sin, out=y[rows])

        if record:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
        if rot:   # turn the surviving window keys, store the new keys rotated
            api.quantize_append_rotated(gc, k, v, f0, w.C, shots, shot_starts=fss)
        else:
            api.quantize_append(gc, k, v, f0, w.C, shots, shot_starts=fss)
        if record:
            e[1].record()
        rope(q, qrot)
        if record:
            e[2].record()
        api.attention_chunk(gc, qrot, f0, w.C, shots, out=out, n_workgroups=args.workgroups)
        if record:
            e[3].record()
            ev["c0"].append(e[0]); ev["c1"].append(e[1])
            ev["a0"].append(e[2]); ev["a1"].append(e[3])

    for c in range(first):                # fill the sink and window
        step(c, False)
    c = first
    for _ in range(args.warmup):
        step(c, False)
        c += 1
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step(c, True)
        c += 1
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    attn_each = sorted(a.elapsed_time(b) for a, b in zip(ev["a0"], ev["a1"]))
    attn_ms = sum(attn_each) / args.steps
    codec_ms = sum(a.elapsed_time(b) for a, b in zip(ev["c0"], ev["c1"])) / args.steps
    pct = lambda v, q: v[min(len(v) - 1, int(q * len(v)))]

    Nq, Nk = w.C * w.T, (w.S + w.W) * w.Tc
    # useful FLOP: only the (query frame, key frame) pairs the masks keep,
    # averaged over the timed steps (equal to 4 H Nq Nk D without shots)
    pairs = [visible_pairs(w, (c - args.steps + i) * w.C, args.sink_per_shot, shot_start)
             for i in range(args.steps)]
    flops = 4.0 * w.H * w.T * w.Tc * w.D * sum(pairs) / len(pairs)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    es = 2 if w.dtype == "bf16" else 4
    kept = 2 * w.C * w.Tc * w.H * w.D
    codec_bytes = kept * es + kept * (2.0 if args.kv == "bf16" else 0.5 + 1.0 / 16.0)
    if rot:
        # cache update: the append plus the re-encoding of the surviving
        # window keys (their codes and scales read and written once)
        surv = [surviving_window_frames(w, (c - args.steps + i) * w.C, args.sink_per_shot,
                                        shot_start) for i in range(args.steps)]
        key_frame = w.H * w.Tc * (w.D // 2 + w.D // 16)
        codec_bytes += 2.0 * key_frame * sum(surv) / len(surv)
    codec_gbs = codec_bytes / (codec_ms * 1e-3) / 1e9

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

    res = {
        "metric": METRIC,
        "value": round(w.C / (ms_step * 1e-3), 3),
        "unit": "latent frames/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": workload_desc(w), "kv_format": args.kv,
                   "sink": "per_shot" if args.sink_per_shot else "stream", "query_rows": Nq,
                   "workgroups": args.workgroups or "default",
                   "keys": Nk,
                   "frames_per_step": w.C, "attention_ms": round(attn_ms, 4),
                   "attention_only_frames_per_s": round(w.C / (attn_ms * 1e-3), 1),
                   "attention_ms_p10_p50_p90": [round(pct(attn_each, q), 4)
                                                for q in (0.1, 0.5, 0.9)],
                   ("cache_update_ms" if rot else "append_ms"): round(codec_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic},
        "roofline_codec": {"bound": "hbm", "achieved": round(codec_gbs, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(codec_gbs / HBM_PEAK_GBS, 4),
                           "bytes": int(codec_bytes)},
    }
    if not args.no_cpu_baseline and args.kv == "nvfp4":
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
