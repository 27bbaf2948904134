"""GPU parity of the per-shot sink variant (each shot re-anchors the sink to
its own first S frames) against the oracle's variant: cache bytes bit-exact,
attention within max-abs 1e-2 / mean-abs 1e-3 (float32 output).  The
streams have cuts inside chunks."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle.stream import OracleCache
from streams import compare_cache, device_tensor, err_stats, say, shots_of, step_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3


def _shot_start(w, f):
    s = w.shot_of(f)
    while f > 0 and w.shot_of(f - 1) == s:
        f -= 1
    return f


def _run(w, steps, rows=None, heads=None):
    from fp4_kv_cache_fp4kv_amd import api
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, sink_per_shot=True)
    oc = OracleCache.for_workload(w, sink_per_shot=True)
    qrot = torch.empty((w.C * w.T, w.H, w.D), dtype=torch.float32, device="cuda:0")
    for c in range(max(steps) + 1):
        f0, n = w.chunk_frames(c)
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        shots = shots_of(w, f0, n)
        fss = [_shot_start(w, f) for f in range(f0, f0 + n)]
        oc.append(k, v, f0, n, shots, shot_starts=fss)
        say(f"shot sink {w.name} step {c} frames {f0}..{f0 + n - 1} shot starts {fss}")
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, shots,
                            shot_starts=fss)
        qd = device_tensor(q, qb)
        # positions need not be consecutive across a cut; the library
        # computes each frame's
        api.rope_rel_frames(gc, qd, f0, n, shot_starts=fss, out=qrot[:n * w.T])
        o = api.attention_chunk(gc, qrot[:n * w.T], f0, n, shots, out_dtype=torch.float32)
        torch.cuda.synchronize()
        if c not in steps:
            continue
        assert not compare_cache(gc, oc), (w.name, c)
        r = np.arange(n * w.T) if rows is None else np.asarray([x for x in rows if x < n * w.T])
        hs = list(range(w.H)) if heads is None else heads
        ref = oc.attention(q, f0, n, shots, rows=r, heads=hs, q_shot_starts=fss)
        mx, mn = err_stats(o.cpu().numpy()[r][:, hs], ref)
        say(f"  max-abs {mx:.3e} mean-abs {mn:.3e}")
        assert mx <= MAX_ABS and mn <= MEAN_ABS, (w.name, c, mx, mn)


def test_shot_sink_tiny_stream_cuts_inside_chunks():
    w = wl.Workload("shots5", H=3, D=64, T=24, C=3, S=2, W=6, n_frames=26, seed=41,
                    dtype="bf16", token_stride=2, shot_len=5)
    _run(w, list(range(w.n_chunks)))


def test_shot_sink_d128_outliers():
    w = wl.Workload("shots7", H=2, D=128, T=100, C=3, S=2, W=6, n_frames=24, seed=42,
                    outlier_p=0.01, outlier_scale=20.0, shot_len=7)
    _run(w, [2, 4, 7])


def test_shot_sink_multishot_full_size_sampled():
    w = wl.L5B_SHOTS
    rng = np.random.default_rng(7)
    nq = w.C * w.T
    rows = np.unique(np.concatenate([[0, w.T - 1, w.T, 2 * w.T, nq - 1],
                                     rng.integers(0, nq, 40)]))
    # step 6 holds frames 18..20 (the cut at 20 is inside it); step 7 the new
    # shot's first chunk after its sink
    _run(w, [6, 7], rows=rows, heads=[0, w.H - 1])
