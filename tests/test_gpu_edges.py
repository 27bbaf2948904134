"""GPU parity at the edges of the cache descriptor and of one call (same bar
as the other attention tests: cache bytes bit-exact, attention max-abs 1e-2 /
mean-abs 1e-3 against the oracle):

  * no sink frames (S = 0) on a wrapping stream;
  * one token per frame with a one-frame window and one-frame chunks;
  * an odd frame size well below one 64-key tile (T = 33);
  * the largest cache, S + W = 64 slots, through a wrap of the ring;
  * the largest call, 64 frames in one chunk (block-causal inside it);
  * the smallest rotary width, rot_dim = 2;
  * a requested workgroup count far above the key tiles (clamped).
"""
import pytest

from fp4_kv_cache_fp4kv_amd import workloads as wl
from test_gpu_attention import _run_stream

pytestmark = pytest.mark.gpu


def test_no_sink_frames_wrapping():
    w = wl.Workload("s0", H=2, D=64, T=24, C=2, S=0, W=4, n_frames=14, seed=61, dtype="f32")
    _run_stream(w, list(range(w.n_chunks)))


def test_one_token_frames_one_frame_window():
    w = wl.Workload("t1", H=4, D=128, T=1, C=1, S=1, W=1, n_frames=6, seed=62)
    _run_stream(w, list(range(w.n_chunks)))


def test_odd_frame_size_below_one_tile():
    w = wl.Workload("t33", H=2, D=64, T=33, C=3, S=2, W=6, n_frames=15, seed=63, dtype="f32")
    _run_stream(w, list(range(w.n_chunks)))


def test_largest_cache_64_slots_through_a_wrap():
    w = wl.Workload("slots64", H=2, D=64, T=16, C=4, S=4, W=60, n_frames=72, seed=64,
                    dtype="f32")
    _run_stream(w, [0, 7, 15, 16, 17])


def test_largest_call_64_frames_in_one_chunk():
    w = wl.Workload("c64", H=2, D=64, T=4, C=64, S=0, W=64, n_frames=64, seed=65, dtype="f32")
    _run_stream(w, [0])


def test_smallest_rotary_width():
    w = wl.Workload("rd2", H=2, D=128, T=40, C=2, S=1, W=4, n_frames=10, seed=66)
    _run_stream(w, [0, 2, 4], rot_dim=2)


def test_workgroup_request_above_the_key_tiles():
    w = wl.Workload("wg", H=2, D=128, T=100, C=3, S=1, W=6, n_frames=12, seed=67,
                    outlier_p=0.01, outlier_scale=20.0)
    _run_stream(w, [1, 3], n_wg=4096)


def _oracle_attention_check(gc, oc, q, f0, n, shots, rel=0.0):
    import numpy as np
    import torch
    from fp4_kv_cache_fp4kv_amd import api
    from streams import device_tensor, err_stats
    qr = api.rope_rel_frames(gc, device_tensor(q, None), f0, n)
    o = api.attention_chunk(gc, qr, f0, n, shots, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = o.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    ref = oc.attention(q, f0, n, shots)
    excess = np.abs(got - ref) - rel * np.abs(ref)
    assert excess.max() <= 1e-2, excess.max()
    return got, ref


def test_queries_beyond_the_f16_range_saturate():
    """Rotated queries whose rotary pairs exceed the f16 range are scaled to
    norm 65504 and elements past rot_dim clamped to +-65504 (the oracle's
    reading of the f16 operand range); the kernel ends normally and matches."""
    import numpy as np
    from fp4_kv_cache_fp4kv_amd import api
    from oracle.stream import OracleCache
    from streams import device_tensor
    w = wl.Workload("bigq", H=2, D=128, T=40, C=2, S=1, W=4, n_frames=6, seed=68, dtype="f32")
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, rot_dim=96)
    oc = OracleCache.for_workload(w, rot_dim=96)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        (q, _), (k, _), (v, _) = wl.draw_qkv(w, c)
        api.quantize_append(gc, device_tensor(k, None), device_tensor(v, None), f0, n, [0] * n)
        oc.append(k, v, f0, n, [0] * n)
    rng = np.random.default_rng(5)
    q = q.copy()
    q[0, 0, 0], q[0, 0, 1] = 3.0e5, 4.0e5             # a rotary pair of norm 5e5
    q[1, 1, 100] = -2.0e6                              # past rot_dim
    big = rng.random(q.shape) < 0.02
    q[big] *= np.float32(1.0e5)
    _oracle_attention_check(gc, oc, q, f0, n, [0] * n)


def test_bf16_cache_values_beyond_the_f16_range_saturate():
    """A bf16 cache keeps values beyond the f16 range bit for bit; attention
    reads them saturated to +-65504 (the oracle's reading), ends normally and
    matches (outputs of size 65504 compared with a relative term 1e-3 |ref|:
    the weights are f16)."""
    import numpy as np
    from fp4_kv_cache_fp4kv_amd import api
    from oracle.stream import OracleCacheBF16
    from streams import device_tensor
    w = wl.Workload("bigkv", H=2, D=64, T=40, C=2, S=1, W=4, n_frames=6, seed=69, dtype="f32")
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, kv_format="bf16")
    oc = OracleCacheBF16.for_workload(w)
    rng = np.random.default_rng(6)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        (q, _), (k, _), (v, _) = wl.draw_qkv(w, c)
        k, v = k.copy(), v.copy()
        k[rng.random(k.shape) < 0.01] *= np.float32(3.0e5)
        v[rng.random(v.shape) < 0.01] *= np.float32(3.0e5)
        api.quantize_append(gc, device_tensor(k, None), device_tensor(v, None), f0, n, [0] * n)
        oc.append(k, v, f0, n, [0] * n)
    _oracle_attention_check(gc, oc, q, f0, n, [0] * n, rel=1e-3)


@pytest.mark.parametrize("bad", [0.0, -2.0, float("inf"), float("nan")])
def test_invalid_caller_tensor_scale_is_replaced_by_one(bad):
    """A caller tensor scale that is not finite and positive is replaced by 1:
    the cache bytes equal those of an append with scale 1."""
    import torch
    from fp4_kv_cache_fp4kv_amd import api
    from streams import CACHE_FIELDS, device_tensor
    w = wl.TINY
    a, b = (api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W) for _ in range(2))
    (_, _), (k, _), (v, _) = wl.draw_qkv(w, 0)
    kd, vd = device_tensor(k, None), device_tensor(v, None)
    api.quantize_append(a, kd, vd, 0, 2, [0, 0],
                        tscale=torch.tensor([bad, bad], dtype=torch.float32, device="cuda:0"))
    api.quantize_append(b, kd, vd, 0, 2, [0, 0],
                        tscale=torch.tensor([1.0, 1.0], dtype=torch.float32, device="cuda:0"))
    torch.cuda.synchronize()
    va, vb = a.views(), b.views()
    for name in CACHE_FIELDS:
        assert torch.equal(va[name].cpu(), vb[name].cpu()), name
