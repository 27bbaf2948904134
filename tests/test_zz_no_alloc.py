"""fp4kv_quantize_append_noalloc (the append with the library's own
per-device workspace) against fp4kv_quantize_append with a caller
workspace: the cache bytes of both must be identical, call after call,
including a second call with a smaller input than the first."""
import ctypes

import numpy as np
import pytest
import torch

from fp4_kv_cache_fp4kv_amd import _lib, api
from fp4_kv_cache_fp4kv_amd import workloads as wl
from streams import CACHE_FIELDS, device_tensor, say

pytestmark = pytest.mark.gpu


def _bytes(gc):
    torch.cuda.synchronize()
    v = gc.views()
    return {n: v[n].cpu().numpy().tobytes() for n in CACHE_FIELDS if n in v}


@pytest.mark.parametrize("kv_format", ["nvfp4", "bf16"])
def test_noalloc_append_equals_workspace_append(kv_format):
    # a 1.3B-like layer cut to 4 heads and 1 outlier per 100 elements; the
    # first call appends a 3-frame chunk, the second a 1-frame chunk of a
    # smaller stride-2 cache (fewer kept tokens, other shapes)
    cases = [
        (wl.Workload("na_big", H=4, D=128, T=1560, C=3, S=3, W=12, n_frames=15, seed=41,
                     outlier_p=0.01, outlier_scale=20.0), 0, 3),
        (wl.Workload("na_small", H=2, D=64, T=40, C=2, S=1, W=4, n_frames=9, seed=42,
                     dtype="f32", token_stride=2), 5, 1),
    ]
    for w, f0, n in cases:
        say(f"noalloc append {kv_format} {w.name} frames {f0}..{f0 + n - 1}")
        a = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, kv_format=kv_format)
        b = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, kv_format=kv_format)
        (_, _), (k, kb), (v, vb) = wl.draw_qkv(w, f0 // w.C)
        rows = n * w.T
        kd, vd = device_tensor(k[:rows], None if kb is None else kb[:rows]), \
            device_tensor(v[:rows], None if vb is None else vb[:rows])
        shots = [0] * n
        api.quantize_append(a, kd, vd, f0, n, shots)
        api.quantize_append_noalloc(b, kd, vd, f0, n, shots)
        ba, bb = _bytes(a), _bytes(b)
        for name in ba:
            assert ba[name] == bb[name], (w.name, name)
        # a caller tensor scale goes through the same path
        ts = torch.tensor([0.02, 0.03], dtype=torch.float32, device="cuda:0")
        api.quantize_append(a, kd, vd, f0, n, shots, tscale=ts)
        api.quantize_append_noalloc(b, kd, vd, f0, n, shots, tscale=ts)
        ba, bb = _bytes(a), _bytes(b)
        for name in ba:
            assert ba[name] == bb[name], (w.name, name, "tscale")


def test_noalloc_append_validates_like_the_workspace_append():
    lib = _lib.load()
    w = wl.TINY
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W)
    k = torch.zeros(2 * w.T, w.H, w.D, device="cuda:0")
    shots = (ctypes.c_int32 * 2)(0, 0)
    st = lib.fp4kv_quantize_append_noalloc(ctypes.byref(gc.desc), k.data_ptr(), k.data_ptr(), 0,
                                           0, 0, shots, None, None, None)
    assert st == _lib.FP4KV_EINVAL                      # no frames
    st = lib.fp4kv_quantize_append_noalloc(ctypes.byref(gc.desc), k.data_ptr() + 4,
                                           k.data_ptr(), 0, 0, 2, shots, None, None, None)
    assert st == _lib.FP4KV_EALIGN
    torch.cuda.synchronize()
