"""GPU parity of fp4kv_quantize_append with the oracle's NVFP4 encoder.

The bar is bit-exact: every code byte, scale byte, tensor scale and slot
metadata word equals the oracle's, on the same seeded inputs."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle import nvfp4
from oracle.stream import OracleCache
from streams import compare_cache, device_tensor, gpu_cache, say, shots_of, step_inputs

pytestmark = pytest.mark.gpu


def _stream_codec(w, steps, rot_dim=None):
    from fp4_kv_cache_fp4kv_amd import api
    gc, oc = gpu_cache(w, rot_dim), OracleCache.for_workload(w, rot_dim)
    for c in steps:
        f0, n = w.chunk_frames(c)
        say(f"codec {w.name} step {c} frames {f0}..{f0 + n - 1}")
        (_, _), (k, kb), (v, vb) = step_inputs(w, c)
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n,
                            shots_of(w, f0, n))
        oc.append(k, v, f0, n, shots_of(w, f0, n))
        bad = compare_cache(gc, oc)
        assert not bad, (w.name, c, bad)
    return gc, oc


def test_codec_tiny_stream_bit_exact():
    _stream_codec(wl.TINY, range(wl.TINY.n_chunks))


def test_codec_reappend_is_idempotent():
    from fp4_kv_cache_fp4kv_amd import api
    w = wl.TINY
    gc, oc = _stream_codec(w, range(4))
    before = {k: v.clone() for k, v in gc.views().items()}
    f0, n = w.chunk_frames(3)
    (_, _), (k, kb), (v, vb) = step_inputs(w, 3)
    api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, shots_of(w, f0, n))
    torch.cuda.synchronize()
    for name, t in gc.views().items():
        assert torch.equal(t, before[name]), name


def test_codec_partial_chunk_and_stride2():
    w = wl.Workload("tiny_s2", H=3, D=64, T=16, C=3, S=1, W=5, n_frames=11, seed=12,
                    dtype="bf16", token_stride=2, shot_len=4)
    _stream_codec(w, range(w.n_chunks))   # last step has 2 frames


@pytest.mark.parametrize("name", ["l13b", "l5b", "l5b_shots", "long"])
def test_codec_full_size_first_and_wrap_steps(name):
    w = wl.WORKLOADS[name]
    last = min(w.n_chunks - 1, (w.S + w.W) // w.C + 1)   # the ring has wrapped by then
    _stream_codec(w, [0, 1, last])


def _special_values(rng, n_blocks):
    """Blocks that hit the format's corners: ties of E2M1 after scaling,
    subnormal and zero block scales, saturation, signed zeros."""
    blocks = []
    grid = nvfp4.E2M1_VALUES
    for _ in range(n_blocks):
        kind = rng.integers(0, 6)
        scale = np.float32(2.0 ** rng.integers(-40, 40))
        if kind == 0:      # grid points and midpoints times a power of two
            pts = np.concatenate([grid, (grid[:-1] + grid[1:]) / 2, [6.0]])
            x = rng.permutation(pts)[:16] * scale
        elif kind == 1:    # tiny values next to a large one: subnormal/zero scales
            x = rng.standard_normal(16) * scale * 1e-4
        elif kind == 2:    # log-uniform magnitudes over a wide range
            x = np.exp2(rng.uniform(-30, 30, 16)) * np.sign(rng.standard_normal(16))
        elif kind == 3:
            x = np.zeros(16)
            x[rng.integers(0, 16)] = -0.0
            x[rng.integers(0, 16)] = -1e-30
        elif kind == 4:
            x = rng.standard_normal(16) * scale
        else:              # neighbours of ties in float32
            t = np.float32(rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]))
            x = np.array([np.nextafter(t, np.float32(0)), t, np.nextafter(t, np.float32(9)), 6.0]
                         * 4, np.float64) * scale
        blocks.append(np.asarray(x, np.float64))
    return np.concatenate(blocks).astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_codec_special_values_f32(seed):
    from fp4_kv_cache_fp4kv_amd import api
    rng = np.random.default_rng(1000 + seed)
    w = wl.Workload("special", H=4, D=64, T=32, C=2, S=0, W=2, n_frames=2, seed=seed, dtype="f32")
    n_el = 2 * 32 * 4 * 64
    k = _special_values(rng, n_el // 16).reshape(64, 4, 64)
    v = _special_values(rng, n_el // 16).reshape(64, 4, 64)
    if seed == 2:  # one huge element sets g; everything else is tiny
        k[3, 1, 5] = 3e30
    gc, oc = gpu_cache(w), OracleCache.for_workload(w)
    say(f"codec special seed {seed}")
    api.quantize_append(gc, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), 0, 2, [0, 0])
    oc.append(k, v, 0, 2, [0, 0])
    assert not compare_cache(gc, oc)


@pytest.mark.parametrize("g", [1.0 / 2688.0, 2.0 ** -12, 0.37, 5e-6, 300.0])
def test_codec_every_bf16_value_with_caller_scale(g):
    """All 65536 bf16 bit patterns that are finite, arranged in blocks, with a
    caller-supplied tensor scale (which also exercises saturation)."""
    from fp4_kv_cache_fp4kv_amd import api
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    bits = bits[finite]
    rng = np.random.default_rng(7)
    bits = rng.permutation(bits)
    T, H, D = 32, 4, 128
    per = T * H * D
    n_frames = -(-len(bits) // per)
    pad = n_frames * per - len(bits)
    bits = np.concatenate([bits, bits[:pad]])
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    w = wl.Workload("allbf16", H=H, D=D, T=T, C=n_frames, S=0, W=n_frames, n_frames=n_frames,
                    seed=0)
    k = vals.reshape(n_frames * T, H, D)
    v = -k[::-1].copy()
    gc, oc = gpu_cache(w), OracleCache.for_workload(w)
    ts = torch.tensor([g, g * 3.0], dtype=torch.float32, device="cuda:0")
    say(f"codec all-bf16 g={g}")
    api.quantize_append(gc, device_tensor(k, bits.reshape(k.shape)),
                        device_tensor(v, ((v.view(np.uint32)) >> 16).astype(np.uint16)),
                        0, n_frames, [0] * n_frames, tscale=ts)
    oc.append(k, v, 0, n_frames, [0] * n_frames, tscale=[np.float32(g), np.float32(g * 3.0)])
    assert not compare_cache(gc, oc)


def test_codec_zero_tensor_gets_unit_scale():
    from fp4_kv_cache_fp4kv_amd import api
    w = wl.Workload("zeros", H=2, D=128, T=8, C=1, S=1, W=2, n_frames=1, seed=0, dtype="f32")
    gc, oc = gpu_cache(w), OracleCache.for_workload(w)
    z = np.zeros((8, 2, 128), np.float32)
    api.quantize_append(gc, torch.from_numpy(z).cuda(), torch.from_numpy(z).cuda(), 0, 1, [5])
    oc.append(z, z, 0, 1, [5])
    assert not compare_cache(gc, oc)
    assert oc.k_tscale[0] == 1.0 and oc.slot_shot[0] == 5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_workspace_needs_no_initialization(dtype):
    """Garbage in the workspace outside its last 8448 bytes (the one-pass
    kernel's grid barrier, which must start at zero) does not change the
    encoding: float32 inputs take the two-kernel form, bf16 inputs the one
    pass, which leaves the barrier words at zero counts."""
    from fp4_kv_cache_fp4kv_amd import api
    w = wl.Workload("ws", H=3, D=64, T=24, C=2, S=1, W=4, n_frames=12, seed=13, dtype=dtype,
                    outlier_p=0.01, outlier_scale=20.0)
    gc, oc = gpu_cache(w), OracleCache.for_workload(w)
    gc.workspace.fill_(0xA7)
    gc.workspace[-8448:].zero_()
    for c in range(3):
        f0, n = w.chunk_frames(c)
        (_, _), (k, kb), (v, vb) = step_inputs(w, c)
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, [0] * n)
        oc.append(k, v, f0, n, [0] * n)
        assert not compare_cache(gc, oc), c
    bar = gc.workspace.cpu().numpy().view(np.uint32)[-33 * 64:].reshape(33, 64)
    assert not bar[:, 0].any() and bar[32, 32] == 0


def test_bulk_reappend_kv_recache():
    """KV-recache: after the ring has wrapped, the cached frames are
    re-appended in bulk (the sink in one call, the whole window in another,
    each with one tensor scale); the cache stays bit-exact with the oracle
    and attention over it stays within the bar."""
    from fp4_kv_cache_fp4kv_amd import api
    from streams import err_stats, say
    w = wl.Workload("recache", H=2, D=128, T=100, C=3, S=1, W=6, n_frames=12, seed=31,
                    outlier_p=0.01, outlier_scale=20.0)
    gc, oc = gpu_cache(w), OracleCache.for_workload(w)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        (_, _), (k, kb), (v, vb) = step_inputs(w, c)
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, [0] * n)
        oc.append(k, v, f0, n, [0] * n)
    f1 = w.n_frames
    for f0, n in ((0, w.S), (f1 - w.W, w.W)):     # sink frames, then the window
        say(f"recache frames {f0}..{f0 + n - 1}")
        k, kb = wl.draw(w, 100 + f0, wl.K_ID, n_tokens=n * w.T)
        v, vb = wl.draw(w, 100 + f0, wl.V_ID, n_tokens=n * w.T)
        api.quantize_append(gc, device_tensor(k, kb), device_tensor(v, vb), f0, n, [0] * n)
        oc.append(k, v, f0, n, [0] * n)
        assert not compare_cache(gc, oc), (f0, n)
    q, qb = wl.draw(w, w.n_chunks - 1, wl.Q_ID)
    f0 = f1 - w.C
    qr = api.rope_rel_frames(gc, device_tensor(q, qb), f0, w.C)
    o = api.attention_chunk(gc, qr, f0, w.C, [0] * w.C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    mx, mn = err_stats(o.cpu().numpy(), oc.attention(q, f0, w.C, [0] * w.C))
    assert mx <= 1e-2 and mn <= 1e-3, (mx, mn)
