"""Pins for the oracle's ring bookkeeping and rotary rotation (CPU only).

Ring: brute force over the whole stream (every frame ever appended, filtered
by the sink + last-W rule) against what the slot ring actually holds.
RoPE: identities of rotations, a complex-number formulation (numpy complex
multiply), and invariance of scores under a common position shift.
"""
import itertools

import numpy as np
import pytest

from oracle import ring, rope
from oracle.stream import OracleCache


@pytest.mark.parametrize("S,W,C", [(1, 4, 2), (3, 12, 3), (3, 21, 3), (0, 5, 2),
                                   (2, 7, 3), (4, 4, 4), (1, 6, 1)])
def test_ring_holds_exactly_sink_plus_last_window(S, W, C):
    F = 8 * (S + W) + 1
    slots = {}
    for c in range(-(-F // C)):
        f0, f1 = c * C, min(c * C + C, F)
        for f in range(f0, f1):
            slots[ring.slot_of(f, S, W)] = f
        held = {f for f in slots.values()}
        ws = ring.window_start(f1, S, W)
        visible = {f for f in held if f < S or f >= ws}
        # brute force: all frames so far, filtered by the definition
        expect = {f for f in range(f1) if f < S or f >= f1 - W}
        assert visible == expect
        assert set(ring.visible_frames(f1, S, W)) == expect
        assert len(slots) <= S + W


def test_positions_bounded_and_offsets_preserved():
    S, W, C = 3, 12, 3
    for c in range(40):
        f1 = c * C + C
        vis = ring.visible_frames(f1, S, W)
        pos = [ring.rel_pos(f, f1, S, W) for f in vis]
        assert max(pos) < S + W and min(pos) >= 0
        assert len(set(pos)) == len(pos)
        win = [f for f in vis if f >= S]
        for a, b in itertools.combinations(win, 2):
            assert ring.rel_pos(a, f1, S, W) - ring.rel_pos(b, f1, S, W) == a - b
        for f in vis:
            if f < S:
                assert ring.rel_pos(f, f1, S, W) == f
        if f1 <= S + W:   # nothing evicted yet: positions are absolute
            assert pos == vis


def test_key_visible_rules():
    S, W, C = 2, 6, 2
    # block-causal: a later chunk is never visible
    assert not ring.key_visible(5, 3, 6, S, W, C, 0, 0)
    assert ring.key_visible(3, 2, 4, S, W, C, 0, 0)      # same chunk sees both ways
    # evicted frame invisible, sink always visible
    assert not ring.key_visible(2, 10, 11, S, W, C, 0, 0)
    assert ring.key_visible(0, 10, 11, S, W, C, 0, 0)
    # shots: sink ignores shots, window needs the same shot
    assert ring.key_visible(1, 9, 10, S, W, C, 0, 1)
    assert not ring.key_visible(8, 9, 10, S, W, C, 0, 1)
    assert ring.key_visible(8, 9, 10, S, W, C, 1, 1)


# ------------------------------------------------------------------ RoPE
def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 64))
    assert np.array_equal(rope.rotate(x, np.zeros(50), 64), x)
    y = rope.rotate(x, rng.integers(0, 40, 50), 64)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_composes():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((20, 128))
    a = rng.integers(0, 30, 20)
    b = rng.integers(0, 30, 20)
    assert np.allclose(rope.rotate(rope.rotate(x, a, 128), b, 128),
                       rope.rotate(x, a + b, 128), atol=1e-12)
    assert np.allclose(rope.rotate(rope.rotate(x, a, 128), -a, 128), x, atol=1e-12)


def test_rope_matches_complex_multiplication():
    rng = np.random.default_rng(2)
    D, rd = 128, 96
    x = rng.standard_normal((33, D))
    pos = rng.integers(0, 24, 33)
    z = x[:, 0:rd:2] + 1j * x[:, 1:rd:2]
    freq = 10000.0 ** (-np.arange(rd // 2) * 2.0 / rd)
    zr = z * np.exp(1j * pos[:, None] * freq[None, :])
    y = rope.rotate(x, pos, rd)
    assert np.allclose(y[:, 0:rd:2], zr.real, atol=1e-12)
    assert np.allclose(y[:, 1:rd:2], zr.imag, atol=1e-12)
    assert np.array_equal(y[:, rd:], x[:, rd:])


def test_rope_scores_depend_only_on_offsets():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((8, 64))
    k = rng.standard_normal((9, 64))
    pq = rng.integers(0, 15, 8)
    pk = rng.integers(0, 15, 9)
    s0 = rope.rotate(q, pq, 64) @ rope.rotate(k, pk, 64).T
    for delta in (1, 7, 1000):
        s1 = rope.rotate(q, pq + delta, 64) @ rope.rotate(k, pk + delta, 64).T
        assert np.allclose(s0, s1, atol=1e-10)


# ------------------------------------------------------------------ cache
def test_cache_slot_metadata_tracks_ring():
    c = OracleCache(H=1, D=16, T=2, C=2, S=1, W=4)
    rng = np.random.default_rng(4)
    for step in range(7):
        f0 = 2 * step
        k = rng.standard_normal((4, 1, 16)).astype(np.float32)
        c.append(k, k, f0, 2, [0, 0])
        f1 = f0 + 2
        held = sorted(int(f) for f in c.slot_frame if f >= 0)
        vis = sorted(kf for _, kf in c.visible_slots(f1))
        assert vis == ring.visible_frames(f1, 1, 4)
        assert set(vis) <= set(held)
