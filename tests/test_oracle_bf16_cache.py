"""Pins of the oracle's bf16 baseline cache (the unquantized cache the NVFP4
format is measured against): its rounding equals torch's float32 -> bfloat16
conversion (a library routine), a slot decodes to exactly the rounded kept
inputs, and with nothing evicted the chunk attention equals dense
block-causal attention over the rounded keys and values (torch SDPA in
float64)."""
import numpy as np
import torch

from fp4_kv_cache_fp4kv_amd import workloads as wl
from oracle import ring, rope
from oracle.stream import OracleCacheBF16, bf16_round


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 37.0,
                        np.array([0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                                  65504.0, 1e-30, -3.0e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(bf16_round(x).view(np.uint32), ref.view(np.uint32))


def test_bf16_cache_decodes_the_rounded_inputs():
    w = wl.Workload("bf", H=2, D=64, T=20, C=2, S=1, W=4, n_frames=8, seed=3, token_stride=2)
    c = OracleCacheBF16.for_workload(w)
    rng = np.random.default_rng(2)
    k = rng.standard_normal((2 * w.T, w.H, w.D)).astype(np.float32)
    v = rng.standard_normal((2 * w.T, w.H, w.D)).astype(np.float32)
    c.append(k, v, 2, 2, [0, 0])
    for j in range(2):
        slot = ring.slot_of(2 + j, w.S, w.W)
        kh, vh = c.decode_slot(slot)
        kept = slice(j * w.T, (j + 1) * w.T, w.token_stride)
        assert np.array_equal(kh, bf16_round(k[kept]).transpose(1, 0, 2))
        assert np.array_equal(vh, bf16_round(v[kept]).transpose(1, 0, 2))
        assert not c.v_vals[:, slot, :, w.Tc:].any()     # padding tokens are zero
        assert c.k_tscale[slot] == 1.0 and c.slot_frame[slot] == 2 + j


def test_bf16_cache_full_window_equals_dense_attention():
    w = wl.Workload("bf_full", H=2, D=64, T=16, C=2, S=1, W=12, n_frames=12, seed=0, dtype="f32")
    c = OracleCacheBF16.for_workload(w)
    ks, vs = [], []
    for step in range(w.n_chunks):
        f0, n = w.chunk_frames(step)
        (q, _), (k, _), (v, _) = wl.draw_qkv(w, step)
        c.append(k, v, f0, n, [0] * n)
        ks.append(bf16_round(k))
        vs.append(bf16_round(v))
        out = c.attention(q, f0, n, [0] * n)
        K, V = np.concatenate(ks), np.concatenate(vs)
        f1 = f0 + n
        kframe = np.repeat(np.arange(f1), w.T)
        qframe = np.repeat(np.arange(f0, f1), w.T)
        mask = (kframe[None, :] // w.C) <= (qframe[:, None] // w.C)
        for h in range(w.H):
            qr = torch.from_numpy(rope.rotate(q[:, h], qframe, w.D))[None, None]
            kr = torch.from_numpy(rope.rotate(K[:, h], kframe, w.D))[None, None]
            vt = torch.from_numpy(V[:, h].astype(np.float64))[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qr, kr, vt, attn_mask=torch.from_numpy(mask)[None, None])[0, 0].numpy()
            assert np.allclose(out[:, h], ref, atol=1e-10), (step, h)


def test_operands_saturate_to_the_f16_range():
    """Stored bf16 values beyond the f16 range keep their bits in the cache
    and saturate to +-65504 only where attention reads them."""
    from oracle.stream import OracleCacheBF16
    c = OracleCacheBF16(1, 64, 32, 1, 1, 2)
    k = np.full((32, 1, 64), 1.0e6, np.float32)
    v = np.full((32, 1, 64), -2.0e5, np.float32)
    c.append(k, v, 0, 1, [0])
    kh, vh = c.decode_slot(0)
    assert kh.max() > 65504.0 and vh.min() < -65504.0
    ko, vo = c.operands(kh, vh)
    assert ko.max() == 65504.0 and vo.min() == -65504.0
