"""GPU parity of the split-KV schedule at every workgroup count class, for
every attention kernel instantiation (head dimension 64 and 128, NVFP4 and
bf16 cache, float32 and bf16 output).

A workgroup count cuts each row block's key tiles into pieces at different
places: one workgroup per row block (no pieces), a few pieces merged inside
the kernel by the workgroup that finishes last (n_wg below 3x the row
blocks), and many pieces combined by the merge pass.  Each launch must meet
the oracle bar (max-abs 1e-2, mean-abs 1e-3 on float32 output, the bf16
output within half a bf16 ulp of the float32 one), and two launches with the same count must
agree bit for bit (the merge order is fixed by workgroup index, not by which
workgroup finishes last)."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle.stream import OracleCache, OracleCacheBF16
from streams import device_tensor, err_stats, say, shots_of, step_inputs

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
# the 2 heads x 300 query rows of a step make 4 row blocks of 256 rows
WORKGROUPS = (1, 3, 4, 5, 8, 11, 12, 16, 24, 64, 256)


@pytest.mark.parametrize("kv_format", ["nvfp4", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_split_every_workgroup_count(kv_format, D):
    from fp4_kv_cache_fp4kv_amd import api
    w = wl.Workload(f"split_d{D}", H=2, D=D, T=100, C=3, S=1, W=6, n_frames=15, seed=31 + D,
                    outlier_p=0.01, outlier_scale=20.0)
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, kv_format=kv_format)
    oc = (OracleCacheBF16 if kv_format == "bf16" else OracleCache).for_workload(w)
    for c in range(5):
        f0, n = w.chunk_frames(c)
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        shots = shots_of(w, f0, n)
        oc.append(k, v, f0, n, shots)
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, shots)
        if c not in (0, 4):   # first step (cache filling) and a full window
            continue
        qr = api.rope_rel_frames(gc, device_tensor(q, qb), f0, n)
        ref = oc.attention(q, f0, n, shots, rows=np.arange(n * w.T), heads=list(range(w.H)))
        for nwg in WORKGROUPS:
            say(f"split {kv_format} D{D} step {c} n_wg {nwg}")
            runs = [api.attention_chunk(gc, qr, f0, n, shots, out_dtype=torch.float32,
                                        n_workgroups=nwg).cpu().numpy() for _ in range(2)]
            assert np.array_equal(runs[0], runs[1]), (kv_format, D, c, nwg, "not repeatable")
            mx, mn = err_stats(runs[0], ref)
            assert mx <= MAX_ABS and mn <= MEAN_ABS, (kv_format, D, c, nwg, mx, mn)
            ob = api.attention_chunk(gc, qr, f0, n, shots, out_dtype=torch.bfloat16,
                                     n_workgroups=nwg).float().cpu().numpy()
            # the bf16 output is the float32 result rounded once
            half_ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ob), 1e-38))) - 8)
            assert np.all(np.abs(ob - runs[0]) <= half_ulp * (1 + 1e-6) + 1e-38), \
                (kv_format, D, c, nwg, "bf16 output")
