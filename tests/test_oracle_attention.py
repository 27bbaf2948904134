"""Pins for the oracle's attention and the stream that chains it (CPU only).

Against: PyTorch scaled_dot_product_attention in float64 (a library
routine), a scalar triple loop on tiny inputs (brute force), dense
block-causal attention over all frames when nothing is evicted, explicit
filtered key sets for the window, shot and token-keep rules, softmax row sums,
and snapshot/restore.
"""
import numpy as np
import pytest
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle import attention as att
from oracle import nvfp4, ring, rope
from oracle.stream import OracleCache


def _sdpa(q, k, v, mask, scale=None):
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    mt = torch.from_numpy(np.asarray(mask, bool))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    return o[0, 0].numpy()


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((40, 32)), rng.standard_normal((70, 32)), rng.standard_normal((70, 24))
    mask = rng.random((40, 70)) < 0.6
    mask[:, 0] = True
    assert np.allclose(att.attend(q, k, v, mask), _sdpa(q, k, v, mask), atol=1e-12)


def test_softmax_rows_sum_to_one_and_respect_mask():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((30, 50)) * 30
    mask = rng.random((30, 50)) < 0.3
    mask[:, 3] = True
    p = att.softmax_rows(s, mask)
    assert np.allclose(p.sum(1), 1.0, atol=1e-12)
    assert np.all(p[~mask] == 0)


def test_attend_matches_scalar_triple_loop():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((5, 8)), rng.standard_normal((7, 8)), rng.standard_normal((7, 8))
    mask = rng.random((5, 7)) < 0.7
    mask[:, 0] = True
    out = np.zeros((5, 8))
    for i in range(5):
        w = [np.exp(sum(q[i, d] * k[j, d] for d in range(8)) / np.sqrt(8)) if mask[i, j] else 0.0
             for j in range(7)]
        tot = sum(w)
        for d in range(8):
            out[i, d] = sum(w[j] * v[j, d] for j in range(7)) / tot
    assert np.allclose(att.attend(q, k, v, mask), out, atol=1e-12)


def _stream_inputs(w, c):
    (q, _), (k, _), (v, _) = wl.draw_qkv(w, c)
    return q, k, v


def test_full_window_equals_dense_block_causal_attention():
    """With W >= F nothing is evicted: every chunk step's output equals dense
    block-causal attention over all frames with absolute positions, with the
    keys decoded from their own append (torch SDPA in float64)."""
    w = wl.Workload("tiny_full", H=2, D=64, T=16, C=2, S=1, W=12, n_frames=12, seed=0, dtype="f32")
    cache = OracleCache.for_workload(w)
    ks, vs, qs = [], [], []
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        q, k, v = _stream_inputs(w, c)
        gk, gv = cache.append(k, v, f0, n, [0] * n)
        # this chunk's own decode, straight from the codec
        for x, g, lst in ((k, gk, ks), (v, gv, vs)):
            codes, sc = nvfp4.encode_blocks(x, g)
            lst.append(nvfp4.decode_blocks(codes, sc, g))
        qs.append(q)
        out = cache.attention(q, f0, n, [0] * n)
        # dense reference over frames [0, f0+n)
        Kall = np.concatenate(ks)                     # [tokens][H][D]
        Vall = np.concatenate(vs)
        f1 = f0 + n
        kframe = np.repeat(np.arange(f1), w.T)
        qframe = np.repeat(np.arange(f0, f1), w.T)
        mask = (kframe[None, :] // w.C) <= (qframe[:, None] // w.C)
        for h in range(w.H):
            qr = rope.rotate(q[:, h], qframe, w.D)
            kr = rope.rotate(Kall[:, h], kframe, w.D)
            ref = _sdpa(qr, kr, Vall[:, h], mask)
            assert np.allclose(out[:, h], ref, atol=1e-10), (c, h)


def test_all_frames_query_matches_per_chunk_steps():
    """Querying every frame at once (block-causal mask inside one call) equals
    the per-chunk outputs when nothing is evicted."""
    w = wl.Workload("tiny_full", H=1, D=64, T=16, C=2, S=1, W=12, n_frames=8, seed=0, dtype="f32")
    cache = OracleCache.for_workload(w)
    outs, qs = [], []
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        q, k, v = _stream_inputs(w, c)
        cache.append(k, v, f0, n, [0] * n)
        outs.append(None)
        qs.append(q)
    allq = np.concatenate(qs)
    full = cache.attention(allq, 0, w.n_frames, [0] * w.n_frames)
    # the last chunk's rows must equal the last per-chunk step
    f0, n = w.chunk_frames(w.n_chunks - 1)
    last = cache.attention(qs[-1], f0, n, [0] * n)
    assert np.allclose(full[f0 * w.T:], last, atol=1e-12)
    # the first chunk's rows see only chunk 0
    c0 = OracleCache.for_workload(w)
    q, k, v = _stream_inputs(w, 0)
    c0.append(k, v, 0, 2, [0, 0])
    assert np.allclose(full[:2 * w.T], c0.attention(q, 0, 2, [0, 0]), atol=1e-12)


def test_sliding_window_equals_explicit_key_set_with_shifted_sink():
    """With eviction, window keys keep their absolute offsets to the queries;
    only the sink moves: sink frame j acts as if at absolute frame j + ws - S.
    Checked against SDPA over the explicitly gathered key set."""
    w = wl.TINY
    cache = OracleCache.for_workload(w)
    dec = {}
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        q, k, v = _stream_inputs(w, c)
        gk, gv = cache.append(k, v, f0, n, [0] * n)
        ck, sk = nvfp4.encode_blocks(k, gk)
        cv, sv = nvfp4.encode_blocks(v, gv)
        kd = nvfp4.decode_blocks(ck, sk, gk).reshape(n, w.T, w.H, w.D)
        vd = nvfp4.decode_blocks(cv, sv, gv).reshape(n, w.T, w.H, w.D)
        for j in range(n):
            dec[f0 + j] = (kd[j], vd[j])
        out = cache.attention(q, f0, n, [0] * n)
        f1 = f0 + n
        ws = ring.window_start(f1, w.S, w.W)
        frames = [f for f in range(f1) if f < w.S or f >= f1 - w.W]
        K = np.concatenate([dec[f][0] for f in frames])
        V = np.concatenate([dec[f][1] for f in frames])
        kabs = np.concatenate([np.full(w.T, f + (ws - w.S if f < w.S else 0)) for f in frames])
        kfr = np.concatenate([np.full(w.T, f) for f in frames])
        qabs = np.repeat(np.arange(f0, f1), w.T)
        mask = (kfr[None, :] // w.C) <= (qabs[:, None] // w.C)
        for h in range(w.H):
            ref = _sdpa(rope.rotate(q[:, h], qabs, w.D),
                        rope.rotate(K[:, h], kabs, w.D), V[:, h], mask)
            assert np.allclose(out[:, h], ref, atol=1e-10), c


def test_shot_mask_equals_filtered_key_set_and_reduces_to_single_shot():
    w = wl.Workload("tiny_shots", H=1, D=64, T=16, C=3, S=1, W=6, n_frames=14, seed=9,
                    dtype="f32", shot_len=4)
    single = wl.Workload("tiny_1", H=1, D=64, T=16, C=3, S=1, W=6, n_frames=14, seed=9,
                         dtype="f32", shot_len=100)
    plain = wl.Workload("tiny_0", H=1, D=64, T=16, C=3, S=1, W=6, n_frames=14, seed=9,
                        dtype="f32")
    cs, c1 = OracleCache.for_workload(w), OracleCache.for_workload(single)
    c0 = OracleCache.for_workload(plain)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        q, k, v = _stream_inputs(w, c)
        shots = [w.shot_of(f) for f in range(f0, f0 + n)]
        cs.append(k, v, f0, n, shots)
        # one shot that outlasts the stream, labelled 7 on every frame
        long_shot = [single.shot_of(f) + 7 for f in range(f0, f0 + n)]
        c1.append(k, v, f0, n, long_shot)
        c0.append(k, v, f0, n, [plain.shot_of(f) for f in range(f0, f0 + n)])
        out = cs.attention(q, f0, n, shots)
        f1 = f0 + n
        # per query frame: SDPA on a single-shot cache restricted to sink + same shot
        o1 = c1.attention(q, f0, n, long_shot)
        for a, qf in enumerate(range(f0, f1)):
            rows = slice(a * w.T, (a + 1) * w.T)
            same = all(w.shot_of(kf) == w.shot_of(qf) or kf < w.S
                       for kf in ring.visible_frames(f1, w.S, w.W) if kf // w.C <= qf // w.C)
            if same:
                assert np.allclose(out[rows], o1[rows], atol=1e-12)
        # shot_len >= F reduces to single shot: the cache fed one long shot
        # (id 7) attends exactly like the cache of the shot-free workload
        # (id 0), and like SDPA over every visible key with no shot filter
        o_plain = c0.attention(q, f0, n, [0] * n)
        assert np.array_equal(o1, o_plain)
        keys = [(s, kf) for s, kf in c0.visible_slots(f1)]
        K = np.concatenate([c0.decode_slot(s)[0][0] for s, _ in keys])
        V = np.concatenate([c0.decode_slot(s)[1][0] for s, _ in keys])
        kp = np.concatenate([np.full(w.T, ring.rel_pos(kf, f1, w.S, w.W)) for _, kf in keys])
        kchunk = np.concatenate([np.full(w.T, kf // w.C) for _, kf in keys])
        for a, qf in enumerate(range(f0, f1)):
            rows = slice(a * w.T, (a + 1) * w.T)
            mask = np.tile(kchunk <= qf // w.C, (w.T, 1))
            qp = np.full(w.T, ring.rel_pos(qf, f1, w.S, w.W))
            ref = _sdpa(rope.rotate(q[rows, 0], qp, w.D), rope.rotate(K, kp, w.D), V, mask)
            assert np.allclose(o1[rows, 0], ref, atol=1e-12)
    # explicit filter check on the last step
    f0, n = w.chunk_frames(w.n_chunks - 1)
    q, _, _ = _stream_inputs(w, w.n_chunks - 1)
    f1 = f0 + n
    out = cs.attention(q, f0, n, [w.shot_of(f) for f in range(f0, f1)])
    for a, qf in enumerate(range(f0, f1)):
        keep = [(s, kf) for s, kf in cs.visible_slots(f1)
                if kf // w.C <= qf // w.C and (kf < w.S or w.shot_of(kf) == w.shot_of(qf))]
        K = np.concatenate([cs.decode_slot(s)[0][0] for s, _ in keep])
        V = np.concatenate([cs.decode_slot(s)[1][0] for s, _ in keep])
        kp = np.concatenate([np.full(w.T, ring.rel_pos(kf, f1, w.S, w.W)) for _, kf in keep])
        qp = ring.rel_pos(qf, f1, w.S, w.W)
        qq = q[a * w.T:(a + 1) * w.T, 0]
        ref = _sdpa(rope.rotate(qq, np.full(w.T, qp), w.D), rope.rotate(K, kp, w.D),
                    V, np.ones((w.T, len(K)), bool))
        assert np.allclose(out[a * w.T:(a + 1) * w.T, 0], ref, atol=1e-12)


def test_token_keep_equals_cache_of_kept_tokens():
    """Keeping every other cached token gives the same codes as a cache fed
    only those tokens, and attention equals SDPA over the kept keys."""
    w2 = wl.Workload("tiny_s2", H=2, D=64, T=16, C=2, S=1, W=4, n_frames=10, seed=11,
                     dtype="f32", token_stride=2)
    c2 = OracleCache.for_workload(w2)
    ch = OracleCache(2, 64, 8, 2, 1, 4)
    for c in range(w2.n_chunks):
        f0, n = w2.chunk_frames(c)
        q, k, v = _stream_inputs(w2, c)
        c2.append(k, v, f0, n, [0] * n)
        kk = k.reshape(n, 16, 2, 64)[:, ::2].reshape(-1, 2, 64)
        vv = v.reshape(n, 16, 2, 64)[:, ::2].reshape(-1, 2, 64)
        ch.append(kk, vv, f0, n, [0] * n)
        for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_tscale", "v_tscale", "slot_frame"):
            assert np.array_equal(getattr(c2, name), getattr(ch, name)), name
        out = c2.attention(q, f0, n, [0] * n)
        f1 = f0 + n
        for h in range(2):
            keys, vals, kp = [], [], []
            for s, kf in ch.visible_slots(f1):
                kd, vd = ch.decode_slot(s)
                keys.append(kd[h])
                vals.append(vd[h])
                kp.append(np.full(8, ring.rel_pos(kf, f1, 1, 4)))
            K, V, kp = np.concatenate(keys), np.concatenate(vals), np.concatenate(kp)
            qp = np.repeat([ring.rel_pos(f, f1, 1, 4) for f in range(f0, f1)], 16)
            ref = _sdpa(rope.rotate(q[:, h], qp, 64), rope.rotate(K, kp, 64), V,
                        np.ones((len(qp), len(K)), bool))
            assert np.allclose(out[:, h], ref, atol=1e-12)


def test_snapshot_restore_is_bit_identical():
    w = wl.TINY
    a = OracleCache.for_workload(w)
    for c in range(3):
        f0, n = w.chunk_frames(c)
        _, k, v = _stream_inputs(w, c)
        a.append(k, v, f0, n, [0] * n)
    b = a.snapshot()
    for c in range(3, w.n_chunks):
        f0, n = w.chunk_frames(c)
        q, k, v = _stream_inputs(w, c)
        a.append(k, v, f0, n, [0] * n)
        b.append(k, v, f0, n, [0] * n)
        assert np.array_equal(a.attention(q, f0, n, [0] * n), b.attention(q, f0, n, [0] * n))
    for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_tscale", "v_tscale", "slot_frame"):
        assert np.array_equal(getattr(a, name), getattr(b, name))


def test_rows_and_heads_subset_match_full():
    w = wl.TINY
    cache = OracleCache.for_workload(w)
    for c in range(4):
        f0, n = w.chunk_frames(c)
        q, k, v = _stream_inputs(w, c)
        cache.append(k, v, f0, n, [0] * n)
    full = cache.attention(q, f0, n, [0] * n)
    rows = [0, 5, 17, 31]
    sub = cache.attention(q, f0, n, [0] * n, rows=rows, heads=[0])
    assert np.allclose(sub[:, 0], full[rows, 0], atol=1e-13, rtol=0)


def test_reappend_is_idempotent():
    w = wl.TINY
    cache = OracleCache.for_workload(w)
    for c in range(5):
        f0, n = w.chunk_frames(c)
        _, k, v = _stream_inputs(w, c)
        cache.append(k, v, f0, n, [0] * n)
        snap = cache.snapshot()
        cache.append(k, v, f0, n, [0] * n)
        for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_tscale", "slot_frame"):
            assert np.array_equal(getattr(cache, name), getattr(snap, name))


def test_query_saturation_to_the_f16_range():
    """Queries beyond the f16 range: a rotary pair whose norm exceeds 65504
    keeps its direction at norm 65504, an element past rot_dim is clamped,
    and in-range queries are untouched (closed forms)."""
    oc = OracleCache(1, 64, 2, 1, 1, 4, rot_dim=32)
    q = np.zeros((2, 1, 64), np.float32)
    q[0, 0, 0], q[0, 0, 1] = 3.0e5, 4.0e5          # norm 5e5 -> 65504, direction (0.6, 0.8)
    q[0, 0, 40] = -1.0e6                           # past rot_dim: clamped
    q[1, 0, :] = 1.5                               # in range
    y = oc.rope_queries(q, 0, 1)                   # frame 0, position 0: no turn
    assert np.isclose(np.hypot(y[0, 0, 0], y[0, 0, 1]), 65504.0, rtol=1e-12)
    assert np.isclose(y[0, 0, 0] / y[0, 0, 1], 0.75, rtol=1e-12)
    assert y[0, 0, 40] == -65504.0
    assert np.array_equal(y[1, 0], np.full(64, 1.5))
    # a turned pair has the same norm, so saturating before or after the
    # rotation gives the same query
    y3 = oc.rope_queries(q, 3, 1)                  # frame 3 at position 3
    assert np.isclose(np.hypot(y3[0, 0, 0], y3[0, 0, 1]), 65504.0, rtol=1e-12)


def test_caller_scale_guard():
    assert OracleCache.caller_scale(0.5) == np.float32(0.5)
    for bad in (0.0, -1.0, np.inf, np.nan):
        assert OracleCache.caller_scale(bad) == np.float32(1.0)
