"""Pins for the oracle's NVFP4 codec (CPU only).

Each test checks the oracle against something other than itself: PyTorch's
float8_e4m3fn conversion (a library routine), hand-derived values from the
bit layouts (tests/golden/nvfp4_hand.json), brute-force nearest-value search,
closed forms and error bounds of the format.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_hand.json")))


def _h(s):
    return int(s, 16)


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = nvfp4.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])


def test_e4m3_decode_hand_values():
    for code, val in GOLDEN["e4m3_decode"]:
        assert nvfp4.e4m3_decode(_h(code)) == val


def test_e4m3_encode_round_trip_every_finite_code():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = nvfp4.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(nvfp4.e4m3_encode(vals), codes)


def test_e4m3_encode_hand_ties_and_saturation():
    for x, code, _why in GOLDEN["e4m3_encode_rne"]:
        assert nvfp4.e4m3_encode(np.float32(x)) == _h(code), x
    assert nvfp4.e4m3_encode(np.float32(np.inf)) == 0x7E


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    # log-uniform over the whole finite range plus every midpoint +-1 ulp
    x = np.exp2(rng.uniform(-12, np.log2(448.0), 2_000_000)).astype(np.float32)
    vals = nvfp4.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9)), np.float32(vals)])
    x = np.concatenate([x, near.astype(np.float32), np.float32([0.0, 448.0, 460.0])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nvfp4.e4m3_encode(x), ref)


# ------------------------------------------------------------------ E2M1
def _e2m1_brute(y):
    """Nearest of all 8 magnitudes by full distance search; ties -> even code."""
    y = np.asarray(y, dtype=np.float64)
    grid = nvfp4.E2M1_VALUES
    dist = np.abs(y[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer an even code
    even = cand & (np.arange(8) % 2 == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(y > 6.0, 7, pick)
    return pick


def test_e2m1_hand_ties():
    for y, code in GOLDEN["e2m1_encode_rne"]:
        assert nvfp4.e2m1_encode_mag(np.float32(y)) == code, y


def test_e2m1_matches_brute_force_near_every_boundary():
    # every float32 within 2^16 ulps of each grid value and each midpoint
    pts = np.concatenate([nvfp4.E2M1_VALUES,
                          (nvfp4.E2M1_VALUES[:-1] + nvfp4.E2M1_VALUES[1:]) / 2,
                          [8.0, 12.0]]).astype(np.float32)
    ys = []
    for p in pts:
        b = np.float32(p).view(np.int32)
        span = np.arange(-65536, 65537, dtype=np.int64) + int(b)
        span = span[(span >= 0) & (span < 0x7F800000)]
        ys.append(span.astype(np.int32).view(np.float32))
    rng = np.random.default_rng(2)
    ys.append(rng.uniform(0, 16, 4_000_000).astype(np.float32))
    bf = (np.arange(0x8000, dtype=np.uint32) << 16)
    bf = bf[bf < 0x7F800000].view(np.float32)   # every non-negative finite bf16
    ys.append(bf)
    y = np.concatenate(ys)
    assert np.array_equal(nvfp4.e2m1_encode_mag(y), _e2m1_brute(y))
    assert nvfp4.e2m1_encode_mag(np.float32(np.inf)) == 7


def test_e2m1_round_trip_grid_and_decode():
    codes = np.arange(16)
    vals = nvfp4.e2m1_decode(codes)
    assert list(vals[:8]) == [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert list(vals[8:]) == [-0.0, -.5, -1, -1.5, -2, -3, -4, -6]
    assert np.array_equal(nvfp4.e2m1_encode_mag(np.abs(vals).astype(np.float32)), codes & 7)


def test_pack_order():
    p = GOLDEN["pack"]
    packed = nvfp4.pack_nibbles(np.array(p["codes"], np.uint8))
    assert [int(b) for b in packed] == [_h(b) for b in p["bytes"]]
    assert np.array_equal(nvfp4.unpack_nibbles(packed), np.array(p["codes"]))


# ------------------------------------------------------------------ blocks
def test_block_hand_example():
    b = GOLDEN["block"]
    x = np.array(b["x"], np.float32)
    g = nvfp4.tensor_scale(x)
    assert g == np.float32(b["g"])
    codes, scales = nvfp4.encode_blocks(x, g)
    assert list(codes) == b["codes"]
    assert int(scales[0]) == _h(b["scale"])


def test_tensor_scale_closed_form_and_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 3, 32)).astype(np.float32)
    amax = np.float32(np.abs(x).max())
    assert nvfp4.tensor_scale(x) == np.float32(amax / np.float32(2688))
    assert nvfp4.tensor_scale(np.zeros(32, np.float32)) == np.float32(1.0)
    codes, scales = nvfp4.encode_blocks(np.zeros((2, 32), np.float32), np.float32(1.0))
    assert not codes.any() and not scales.any()


@pytest.mark.parametrize("k", [-20, -3, 0, 5])
def test_round_trip_of_every_grid_value_at_power_of_two_scales(k):
    """x = e * sv * 2^k with a block holding 6 at sv = 448 round-trips exactly
    for every E2M1 value e and every normal E4M3 block scale sv."""
    rng = np.random.default_rng(100 + k)
    sv_codes = np.arange(0x08, 0x7F)                     # all normal scales
    n = len(sv_codes) + 1
    mags = np.tile(nvfp4.E2M1_VALUES, 2)                 # 16 per block
    signs = np.where(np.arange(16) >= 8, -1.0, 1.0)
    e = np.empty((n, 16))
    for i in range(n):
        e[i] = rng.permutation(mags * signs)
    e[0] = mags * signs                                   # contains +6
    sv = np.concatenate([[448.0], nvfp4.e4m3_decode(sv_codes)])
    x = (e * sv[:, None] * 2.0 ** k).astype(np.float32).reshape(1, -1)
    g = nvfp4.tensor_scale(x)
    assert g == np.float32(2.0 ** k)
    codes, scales = nvfp4.encode_blocks(x, g)
    back = nvfp4.decode_blocks(codes, scales, g)
    assert np.array_equal(back, x)
    assert np.array_equal(nvfp4.e4m3_decode(scales[0]), sv)


def test_block_amax_maps_to_six_when_scale_is_normal():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4096, 64)) * np.exp2(rng.uniform(-12, 4, (4096, 1)))).astype(np.float32)
    g = nvfp4.tensor_scale(x)
    codes, scales = nvfp4.encode_blocks(x, g)
    xb = np.abs(x).reshape(4096, 4, 16)
    cb = codes.reshape(4096, 4, 16)
    at_max = xb == xb.max(axis=-1, keepdims=True)
    normal = (scales >= 0x08)[..., None] & at_max
    assert normal.sum() > 1000
    assert np.all((cb & 7)[normal] == 7)
    # subnormal block scales are the boundary case: reported, not required
    sub = (scales < 0x08) & (scales > 0)
    assert sub.any()


def test_block_scale_matches_torch_cast():
    """s8 = E4M3(fl(a_b / fl(6 g))) with PyTorch's float8 conversion."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((2048, 128)) * np.exp2(rng.uniform(-6, 6, (2048, 1)))).astype(np.float32)
    g = nvfp4.tensor_scale(x)
    _, scales = nvfp4.encode_blocks(x, g)
    a = np.abs(x).reshape(2048, 8, 16).max(-1)
    s = (a / np.float32(np.float32(6) * g)).astype(np.float32)
    assert s.max() <= 448.0 * (1 + 2 ** -20)
    ref = torch.from_numpy(np.minimum(s, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref)


def test_decoded_value_is_nearest_scaled_grid_point():
    """Every element decodes to the scaled E2M1 point nearest to x within the
    format's bound: |x - x_hat| <= half the local grid gap * S_b (+ rounding)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((512, 64)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 20
    g = nvfp4.tensor_scale(x)
    codes, scales = nvfp4.encode_blocks(x, g)
    xh = nvfp4.decode_blocks(codes, scales, g).astype(np.float64)
    Sb = np.repeat(nvfp4.e4m3_decode(scales) * float(g), 16, axis=-1)
    y = np.abs(x) / Sb
    gap = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    err = np.abs(x - xh)
    # slack: the float32 roundings of S_b and of the decoded product
    bound = np.where(y <= 6, gap / 2 * Sb, np.abs(x) - 6 * Sb) + 2.0 ** -21 * np.abs(x) + 1e-30
    assert np.all(err <= bound)
    # brute force: no other scaled grid point is strictly closer
    cand = np.sign(x)[..., None] * nvfp4.E2M1_VALUES * Sb[..., None]
    assert np.all(np.abs(x[..., None] - cand).min(-1) >= err - 1e-6 * np.abs(x) - 1e-30)


def test_sign_of_zero_and_tiny_negatives():
    x = np.zeros(16, np.float32)
    x[0] = 6.0
    x[1] = -0.0
    x[2] = -1e-6
    codes, _ = nvfp4.encode_blocks(x, nvfp4.tensor_scale(x))
    assert codes[1] == 8 and codes[2] == 8 and codes[3] == 0


def test_caller_tensor_scale_saturates():
    """A caller-supplied g far below amax/2688 saturates scales at 448 and
    elements at 6."""
    x = np.full((1, 16), 1000.0, np.float32)
    codes, scales = nvfp4.encode_blocks(x, np.float32(1e-3))
    assert np.all(scales == 0x7E) and np.all(codes == 7)
