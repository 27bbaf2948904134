"""Helpers that drive the same seeded stream through the HIP library and the
CPU oracle.  Inputs come only from the seeded generators; expected values
come only from the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle.stream import OracleCache

CACHE_FIELDS = ("k_codes", "v_codes", "k_scales", "v_scales", "k_tscale", "v_tscale",
                "slot_frame", "slot_shot")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_tensor(vals: np.ndarray, bits, dev="cuda:0") -> torch.Tensor:
    """Seeded input on the device: bf16 from its bit pattern, else float32."""
    if bits is not None:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(vals, np.float32)).to(dev)


def gpu_cache(w: wl.Workload, rot_dim=None):
    from fp4_kv_cache_fp4kv_amd import api
    return api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, rot_dim)


def compare_cache(gc, oc: OracleCache, slots=None):
    """Bit-exact comparison of the device cache with the oracle cache; returns
    a list of mismatching field names."""
    torch.cuda.synchronize()
    v = gc.views()
    bad = []
    for name in CACHE_FIELDS:
        g = v[name].cpu().numpy()
        o = getattr(oc, name)
        if name in ("k_codes", "v_codes", "k_scales", "v_scales") and slots is not None:
            g, o = g[:, slots], o[:, slots]
        elif slots is not None:
            g, o = g[slots], o[slots]
        if g.dtype == np.float32:
            g, o = g.view(np.uint32), np.asarray(o, np.float32).view(np.uint32)
        if not np.array_equal(g, o):
            bad.append(name)
    return bad


def step_inputs(w: wl.Workload, c: int):
    return wl.draw_qkv(w, c)


def shots_of(w, f0, n):
    return [w.shot_of(f) for f in range(f0, f0 + n)]


def err_stats(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    return float(d.max()), float(d.mean())
