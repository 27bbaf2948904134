"""GPU checks of the library-computed positions and of the fused step
prologue, through the C ABI:

  * fp4kv_rope_rel_frames rotates each frame by the oracle's cache-relative
    position (also across shot cuts with per-shot sinks, where positions are
    not consecutive): bit for bit what fp4kv_rope_rel gives with those
    positions, and within float32 error of the oracle's float64 rotation;
  * fp4kv_rope_append (the queries' rotation and the append: one pass for
    bf16 inputs, two kernels for float32) leaves the same cache bytes and
    rotated queries as the separate calls, step after step, on the small
    streams and on the full-size layers, and leaves its grid barrier's
    workspace words clear.
"""
import numpy as np
import pytest
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle import ring, rope
from streams import CACHE_FIELDS, device_tensor, say, shots_of, step_inputs

pytestmark = pytest.mark.gpu


def _shot_start(w, f):
    s0 = w.shot_of(f)
    while f > 0 and w.shot_of(f - 1) == s0:
        f -= 1
    return f


def _bytes(gc):
    v = gc.views()
    return {n: v[n].cpu().numpy().tobytes() for n in CACHE_FIELDS if n in v}


@pytest.mark.parametrize("per_shot", [False, True])
def test_rope_rel_frames_uses_the_oracle_positions(per_shot):
    from fp4_kv_cache_fp4kv_amd import api
    w = wl.Workload("rf", H=3, D=128, T=24, C=3, S=2, W=6, n_frames=22, seed=71, shot_len=5)
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, rot_dim=96, sink_per_shot=per_shot)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        f1 = f0 + n
        (q, qb), _, _ = step_inputs(w, c)
        fss = [_shot_start(w, f) for f in range(f0, f1)] if per_shot else None
        pos = [ring.pos_shot(f, fss[j], f1, w.S, w.W) if per_shot else ring.rel_pos(f, f1, w.S, w.W)
               for j, f in enumerate(range(f0, f1))]
        say(f"rope_rel_frames step {c} positions {pos}")
        qd = device_tensor(q, qb)
        got = api.rope_rel_frames(gc, qd, f0, n, shot_starts=fss)
        ref = torch.empty_like(got)
        for j in range(n):
            r = slice(j * w.T, (j + 1) * w.T)
            api.rope_rel(qd[r], pos[j], w.T, gc.cos_sin, rot_dim=96, out=ref[r])
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), c
        exact = rope.rotate(q, np.repeat(pos, w.T)[:, None], 96)
        mag = np.abs(q).astype(np.float64)
        assert np.all(np.abs(got.cpu().numpy() - exact) <= 2.0 ** -20 * (mag + np.roll(mag, 1, -1)
                                                                          + np.roll(mag, -1, -1)) + 1e-37)


def _prologue_stream(w, steps, per_shot=False, check=None):
    """Separate calls into cache A, rope_append into cache B; the bytes of
    both caches and both rotated queries must be identical at every step."""
    from fp4_kv_cache_fp4kv_amd import api
    a = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, sink_per_shot=per_shot)
    b = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, sink_per_shot=per_shot)
    for c in range(steps):
        f0, n = w.chunk_frames(c)
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        shots = shots_of(w, f0, n)
        fss = [_shot_start(w, f) for f in range(f0, f0 + n)] if per_shot else None
        say(f"rope_append {w.name} step {c} frames {f0}..{f0 + n - 1}")
        qd, kd, vd = device_tensor(q, qb), device_tensor(k, kb), device_tensor(v, vb)
        api.quantize_append(a, kd, vd, f0, n, shots, shot_starts=fss)
        qa = api.rope_rel_frames(a, qd, f0, n, shot_starts=fss)
        qb_ = api.rope_append(b, qd, kd, vd, f0, n, shots, shot_starts=fss)
        torch.cuda.synchronize()
        if check is None or c in check:
            assert torch.equal(qa.view(torch.int32), qb_.view(torch.int32)), (w.name, c)
            ba, bb = _bytes(a), _bytes(b)
            for name in ba:
                assert ba[name] == bb[name], (w.name, c, name)
    _barrier_words_clear(b)


def _barrier_words_clear(gc):
    """The one-pass prologue's grid barrier (the workspace's last 33 lines of
    64 words: per group an arrival count (word 0) and a phase (word 32), then
    the count of complete groups and the error word) is left with zero counts
    and no error after every call, and all phases agree (each call flips them
    all)."""
    ws = gc.workspace.cpu().numpy().view(np.uint32)
    bar = ws[-33 * 64:].reshape(33, 64)
    assert not bar[:, 0].any(), bar[:, 0]
    assert bar[32, 32] == 0
    assert bar[:32, 32].min() == bar[:32, 32].max() and bar[0, 32] in (0, 1), bar[:32, 32]


def test_rope_append_equals_separate_calls_small():
    _prologue_stream(wl.TINY, wl.TINY.n_chunks)
    w = wl.Workload("tiny_mix", H=3, D=64, T=24, C=3, S=2, W=6, n_frames=20, seed=21,
                    dtype="bf16", token_stride=2, shot_len=5)
    _prologue_stream(w, w.n_chunks)
    _prologue_stream(w, w.n_chunks, per_shot=True)


@pytest.mark.parametrize("name", ["l13b", "long", "l5b_shots"])
def test_rope_append_equals_separate_calls_full_size(name):
    w = wl.WORKLOADS[name]
    steps = 8 if name == "long" else min(w.n_chunks, (w.S + w.W) // w.C + 1)
    _prologue_stream(w, steps, per_shot=name == "l5b_shots", check={0, steps - 1})


def test_rope_append_large_chunk_takes_the_two_kernel_form():
    """A bf16 chunk with more items (4 kept tokens x one 16-element block of
    K or V: 524,288 here) than the one-pass grid has threads on MI355X
    (1024 workgroups of 256) runs the two-kernel form: same bytes as the
    separate calls, and the barrier words untouched."""
    w = wl.Workload("wide", H=32, D=128, T=64, C=64, S=0, W=64, n_frames=64, seed=77,
                    dtype="bf16", outlier_p=0.01, outlier_scale=20.0)
    assert 2 * w.H * w.n_frames * (w.T // 8) * (w.D // 16) * 2 == 524288
    _prologue_stream(w, 1)


def test_one_pass_wait_that_gives_up_keeps_the_bytes(monkeypatch):
    """The one-pass kernel's barrier wait is bounded.  With the limit forced
    to 0 polls from the host (FP4KV_BARRIER_SPINS), workgroups give up their
    wait at once, take the tensor maxima over all of K and V themselves and
    encode: every kernel ends normally, the cache stays bit-exact against the
    oracle step after step, the error word is set, and the barrier counts
    still end at zero."""
    from fp4_kv_cache_fp4kv_amd import api
    from oracle.stream import OracleCache
    from streams import compare_cache
    w = wl.Workload("giveup", H=3, D=128, T=40, C=2, S=1, W=4, n_frames=10, seed=83,
                    dtype="bf16", outlier_p=0.01, outlier_scale=20.0)
    monkeypatch.setenv("FP4KV_BARRIER_SPINS", "0")
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride)
    oc = OracleCache.for_workload(w)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        say(f"rope_append, wait limit 0, step {c}")
        qd, kd, vd = device_tensor(q, qb), device_tensor(k, kb), device_tensor(v, vb)
        got = api.rope_append(gc, qd, kd, vd, f0, n, [0] * n)
        ref = api.rope_rel_frames(gc, qd, f0, n)
        api.quantize_append(gc, kd, vd, f0, n, [0] * n)   # the one-pass append, same limit
        torch.cuda.synchronize()
        oc.append(k, v, f0, n, [0] * n)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), c
        assert not compare_cache(gc, oc), c
    ws = gc.workspace.cpu().numpy().view(np.uint32)
    bar = ws[-33 * 64:].reshape(33, 64)
    assert not bar[:, 0].any()
    assert bar[32, 32] == 1   # at least one wait gave up


def test_concurrent_one_pass_calls_on_two_streams(monkeypatch):
    """Two fp4kv_rope_append calls of full-size 1.3B-like chunks (each grid as
    large as the device holds at once) overlap on two streams, with their
    own caches and workspaces.  Neither grid can then be sure to be resident
    whole; a wait that gives up (its limit lowered from the host to 2000
    polls so that it resolves in milliseconds) takes the maxima itself.
    Every call must end normally with the bytes of the same calls made one
    at a time."""
    from fp4_kv_cache_fp4kv_amd import api
    monkeypatch.setenv("FP4KV_BARRIER_SPINS", "2000")
    w = wl.WORKLOADS["l13b"]
    caches = [api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride) for _ in range(4)]
    inputs = []
    for c in range(2):
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        inputs.append((device_tensor(q, qb), device_tensor(k, kb), device_tensor(v, vb)))
    # one at a time
    ref = []
    for i, (qd, kd, vd) in enumerate(inputs):
        f0 = i * w.C
        ref.append(api.rope_append(caches[i], qd, kd, vd, f0, w.C, [0] * w.C))
    torch.cuda.synchronize()
    # overlapped: the second call's stream does not wait for the first
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = []
    for rep in range(3):
        say(f"two concurrent one-pass calls, round {rep}")
        torch.cuda.synchronize()
        got = []
        for i, (qd, kd, vd) in enumerate(inputs):
            with torch.cuda.stream(streams[i]):
                got.append(api.rope_append(caches[2 + i], qd, kd, vd, i * w.C, w.C, [0] * w.C))
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(got[i].view(torch.int32), ref[i].view(torch.int32)), (rep, i)
            a, b = _bytes(caches[i]), _bytes(caches[2 + i])
            for name in a:
                assert a[name] == b[name], (rep, i, name)
    for i, gc in enumerate(caches):
        bar = gc.workspace.cpu().numpy().view(np.uint32)[-33 * 64:].reshape(33, 64)
        assert not bar[:, 0].any(), bar[:, 0]
        say(f"cache {i}: a wait gave up: {bool(bar[32, 32])}")


@pytest.mark.parametrize("shape", [
    # (H, D, T, C, S, W, n_frames, token_stride): kept tokens per frame Tc = T / stride
    (1, 64, 1, 1, 1, 1, 4, 1),      # one-token frames, one-frame chunks: Tc = 1
    (5, 128, 33, 3, 1, 4, 10, 1),   # Tc = 33: a last 8-token group with one token
    (3, 64, 26, 2, 2, 3, 9, 2),     # Tc = 13: the last group's odd half holds one token
    (7, 128, 12, 1, 0, 3, 5, 1),    # Tc = 12: the last group half full, no sink
    (2, 128, 66, 3, 1, 6, 11, 2),   # Tc = 33 from token stride 2, a 2-frame last chunk
])
def test_one_pass_edge_shapes_against_the_oracle(shape):
    """The one-pass kernel (bf16 inputs) on shapes whose kept tokens end
    inside an 8-token group or inside its 4-token half: cache bytes
    bit-exact against the oracle at every step, through both entry points
    (rope_append, then quantize_append of the same chunk, which must rewrite
    the same bytes), with the rotated queries equal to rope_rel_frames'."""
    from fp4_kv_cache_fp4kv_amd import api
    from oracle.stream import OracleCache
    from streams import compare_cache
    H, D, T, C, S, W, n_frames, stride = shape
    w = wl.Workload(f"edge{H}_{D}_{T}", H=H, D=D, T=T, C=C, S=S, W=W, n_frames=n_frames,
                    seed=97 + H, dtype="bf16", outlier_p=0.01, outlier_scale=20.0,
                    token_stride=stride)
    gc = api.FP4KVCache(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride)
    oc = OracleCache.for_workload(w)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        (q, qb), (k, kb), (v, vb) = step_inputs(w, c)
        say(f"one-pass edge shape {shape} step {c} frames {f0}..{f0 + n - 1}")
        qd, kd, vd = device_tensor(q, qb), device_tensor(k, kb), device_tensor(v, vb)
        got = api.rope_append(gc, qd, kd, vd, f0, n, [0] * n)
        ref = api.rope_rel_frames(gc, qd, f0, n)
        torch.cuda.synchronize()
        oc.append(k, v, f0, n, [0] * n)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), c
        assert not compare_cache(gc, oc), c
        api.quantize_append(gc, kd, vd, f0, n, [0] * n)
        assert not compare_cache(gc, oc), c
    _barrier_words_clear(gc)
