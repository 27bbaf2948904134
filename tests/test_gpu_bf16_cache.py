"""GPU parity of the bf16 baseline cache (FP4KV_FORMAT_BF16_V1) against the
oracle's bf16 cache: the stored bf16 values bit-exact, attention within the
same bar as the NVFP4 path (max-abs 1e-2, mean-abs 1e-3 on the float32
output)."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle.stream import OracleCacheBF16
from streams import device_tensor, err_stats, say, shots_of, step_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3


def _bits(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _compare(gc, oc):
    torch.cuda.synchronize()
    v = gc.views()
    bad = []
    if not np.array_equal(v["k_codes"].cpu().numpy().view(np.uint16), _bits(oc.k_vals)):
        bad.append("k")
    if not np.array_equal(v["v_codes"].cpu().numpy().view(np.uint16), _bits(oc.v_vals)):
        bad.append("v")
    for name in ("k_tscale", "v_tscale", "slot_frame", "slot_shot"):
        if not np.array_equal(v[name].cpu().numpy(), getattr(oc, name)):
            bad.append(name)
    return bad


def _run(w, steps, rows=None, heads=None):
    from fp4_kv_cache_fp4kv_amd import api
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, kv_format="bf16")
    oc = OracleCacheBF16.for_workload(w)
    for c in range(max(steps) + 1):
        f0, n = w.chunk_frames(c)
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        shots = shots_of(w, f0, n)
        oc.append(k, v, f0, n, shots)
        say(f"bf16 cache {w.name} step {c}")
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, shots)
        qr = api.rope_rel_frames(gc, device_tensor(q, qb), f0, n)
        o = api.attention_chunk(gc, qr, f0, n, shots, out_dtype=torch.float32)
        torch.cuda.synchronize()
        if c not in steps:
            continue
        assert not _compare(gc, oc), (w.name, c, _compare(gc, oc))
        r = np.arange(n * w.T) if rows is None else np.asarray([x for x in rows if x < n * w.T])
        hs = list(range(w.H)) if heads is None else heads
        ref = oc.attention(q, f0, n, shots, rows=r, heads=hs)
        mx, mn = err_stats(o.cpu().numpy()[r][:, hs], ref)
        say(f"  max-abs {mx:.3e} mean-abs {mn:.3e}")
        assert mx <= MAX_ABS and mn <= MEAN_ABS, (w.name, c, mx, mn)


def test_bf16_cache_tiny_stream():
    _run(wl.TINY, list(range(wl.TINY.n_chunks)))


def test_bf16_cache_multishot_stride2_d64():
    w = wl.Workload("tiny_mix", H=3, D=64, T=24, C=3, S=2, W=6, n_frames=20, seed=21,
                    dtype="bf16", token_stride=2, shot_len=5)
    _run(w, list(range(w.n_chunks)))


def test_bf16_cache_d128_ragged_outliers():
    w = wl.Workload("d128", H=2, D=128, T=100, C=3, S=1, W=6, n_frames=15, seed=22,
                    outlier_p=0.01, outlier_scale=20.0)
    _run(w, [0, 2, 4])


def test_bf16_cache_full_size_sampled():
    w = wl.L13B
    rng = np.random.default_rng(5)
    nq = w.C * w.T
    rows = np.unique(np.concatenate([[0, 255, 256, w.T - 1, w.T, nq - 1],
                                     rng.integers(0, nq, 40)]))
    _run(w, [(w.S + w.W) // w.C - 1], rows=rows, heads=[0, w.H - 1])


def test_bf16_cache_per_shot_sinks_cuts_inside_chunks():
    # the baseline format with per-shot sinks: slots chosen per frame on the
    # host, sink visibility per shot in the kernel's frame list
    from fp4_kv_cache_fp4kv_amd import api
    w = wl.Workload("bf_shots", H=2, D=64, T=24, C=3, S=2, W=6, n_frames=26, seed=71,
                    shot_len=7)
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, kv_format="bf16",
                        sink_per_shot=True)
    oc = OracleCacheBF16.for_workload(w, sink_per_shot=True)

    def shot_start(f):
        s = w.shot_of(f)
        while f > 0 and w.shot_of(f - 1) == s:
            f -= 1
        return f
    qrot = torch.empty((w.C * w.T, w.H, w.D), dtype=torch.float32, device="cuda:0")
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        shots = shots_of(w, f0, n)
        fss = [shot_start(f) for f in range(f0, f0 + n)]
        oc.append(k, v, f0, n, shots, shot_starts=fss)
        say(f"bf16 cache per-shot step {c} shot starts {fss}")
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, shots,
                            shot_starts=fss)
        qd = device_tensor(q, qb)
        api.rope_rel_frames(gc, qd, f0, n, shot_starts=fss, out=qrot[:n * w.T])
        o = api.attention_chunk(gc, qrot[:n * w.T], f0, n, shots, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert not _compare(gc, oc), (c, _compare(gc, oc))
        ref = oc.attention(q, f0, n, shots, q_shot_starts=fss)
        mx, mn = err_stats(o.cpu().numpy(), ref)
        say(f"  max-abs {mx:.3e} mean-abs {mn:.3e}")
        assert mx <= MAX_ABS and mn <= MEAN_ABS, (c, mx, mn)
