"""Pins of the oracle's per-shot sink variant (each shot re-anchors the sink
to its own first S frames): with one shot it is the stream sink exactly, and
on a multi-shot stream (shots of 7 frames, chunks of 3, so cuts fall inside
chunks) every step's attention equals torch SDPA (float64) over the key set
and positions the rule names, gathered by brute force from the whole frame
history."""
import numpy as np
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle import nvfp4, ring, rope
from oracle.stream import OracleCache


def _shot_starts(w, frames):
    out = []
    for f in frames:
        s = w.shot_of(f)
        fs = f
        while fs > 0 and w.shot_of(fs - 1) == s:
            fs -= 1
        out.append(fs)
    return out


def test_single_shot_equals_stream_sink():
    w = wl.Workload("one", H=2, D=64, T=16, C=2, S=2, W=4, n_frames=14, seed=4, dtype="f32")
    a, b = OracleCache.for_workload(w), OracleCache.for_workload(w, sink_per_shot=True)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        (q, _), (k, _), (v, _) = wl.draw_qkv(w, c)
        a.append(k, v, f0, n, [0] * n)
        b.append(k, v, f0, n, [0] * n, shot_starts=[0] * n)
        assert np.array_equal(a.slot_frame, b.slot_frame)
        assert np.array_equal(a.k_codes, b.k_codes) and np.array_equal(a.v_codes, b.v_codes)
        oa = a.attention(q, f0, n, [0] * n)
        ob = b.attention(q, f0, n, [0] * n, q_shot_starts=[0] * n)
        assert np.array_equal(oa, ob), c


def test_multishot_attention_equals_brute_force_key_set():
    w = wl.Workload("ms", H=2, D=64, T=16, C=3, S=2, W=6, n_frames=26, seed=5, dtype="f32",
                    shot_len=7)
    cache = OracleCache.for_workload(w, sink_per_shot=True)
    hist_k, hist_v = {}, {}           # frame -> decoded [T][H][D] (its own append)
    for c in range(w.n_chunks):
        f0, n = w.chunk_frames(c)
        frames = list(range(f0, f0 + n))
        (q, _), (k, _), (v, _) = wl.draw_qkv(w, c)
        shots = [w.shot_of(f) for f in frames]
        fss = _shot_starts(w, frames)
        gk, gv = cache.append(k, v, f0, n, shots, shot_starts=fss)
        for x, g, hist in ((k, gk, hist_k), (v, gv, hist_v)):
            codes, sc = nvfp4.encode_blocks(x, g)
            dec = nvfp4.decode_blocks(codes, sc, g)
            for j, f in enumerate(frames):
                hist[f] = dec[j * w.T:(j + 1) * w.T]
        out = cache.attention(q, f0, n, shots, q_shot_starts=fss)
        f1 = f0 + n
        ws = ring.window_start(f1, w.S, w.W)
        for j, qf in enumerate(frames):
            fsq = fss[j]
            # the rule, by brute force over every frame so far.  A sink frame
            # counts while no later frame (a later shot's sink frame) has
            # taken its sink slot: one cut inside a chunk leaves the earlier
            # shot's frames of that chunk without a sink.
            fs_all = _shot_starts(w, range(f1))

            def sink_present(kf):
                i = kf - fs_all[kf]
                return not any(g - fs_all[g] == i for g in range(kf + 1, f1))
            keys = [kf for kf in range(f1)
                    if w.shot_of(kf) == w.shot_of(qf) and kf // w.C <= qf // w.C
                    and ((kf - fsq < w.S and sink_present(kf)) or
                         (kf - fsq >= w.S and kf >= ws))]
            kpos = [kf - fsq if kf - fsq < w.S else w.S + (kf - ws) for kf in keys]
            qpos = qf - fsq if qf - fsq < w.S else w.S + (qf - ws)
            K = np.concatenate([hist_k[kf] for kf in keys])
            V = np.concatenate([hist_v[kf] for kf in keys])
            kp = np.repeat(kpos, w.T)
            rows = slice(j * w.T, (j + 1) * w.T)
            for h in range(w.H):
                qr = rope.rotate(q[rows, h], np.full(w.T, qpos), w.D)
                kr = rope.rotate(K[:, h], kp, w.D)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(qr)[None, None], torch.from_numpy(kr)[None, None],
                    torch.from_numpy(V[:, h].astype(np.float64))[None, None])[0, 0].numpy()
                assert np.allclose(out[rows, h], ref, atol=1e-10), (c, qf, h)
