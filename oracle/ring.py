"""Sink + sliding-window cache bookkeeping: slots, visibility, positions.

TEST INFRASTRUCTURE (CPU oracle); see oracle/__init__.py.

What the pages fix:
  * generation is causal and chunk by chunk, with a KV cache kept across
    steps (hysenlabs.com, "How it differs from a general diffusion
    pipeline");
  * attention sinks keep the first frames so a streaming generator does not
    drift (heatdrop.ai, "What it does"; hysenlabs.com, "NVFP4, sequence
    parallel and the async decode path");
  * positions are relative to the KV cache so appended chunks do not drift
    and the stream can run without bound (refft.com, relative RoPE and
    TriAttention question; aiany.app, "What Sets It Apart");
  * multi-shot masking lets a new shot use relevant past context without
    bleeding across cuts (evermx.com, "Multi-Shot Generation").

Readings (the pages give no formula):
  * frames are numbered from 0; chunk step c holds frames
    [c*C, min(c*C + C, F));
  * the sink is frames [0, S) and is never evicted; the window holds the
    last W frames including the current chunk, so the cache has S + W slots;
    frame f lives in slot f if f < S, else S + ((f - S) mod W);
  * with f1 the end of the current query frames, the window starts at
    ws = max(S, f1 - W) and the visible key frames are
    [0, min(S, f1)) U [ws, f1);
  * cache-relative position: pos(f) = f for f < S, else S + (f - ws), for
    keys and queries alike (bounded by S + W);
  * key frame kf is visible to query frame qf iff kf is visible at this step,
    chunk(kf) <= chunk(qf) (block-causal: frames of one chunk see each
    other), and kf is a sink frame or shot(kf) == shot(qf).
"""
from __future__ import annotations


def slot_of(f: int, S: int, W: int) -> int:
    return f if f < S else S + (f - S) % W


def window_start(f1: int, S: int, W: int) -> int:
    return max(S, f1 - W)


def visible_frames(f1: int, S: int, W: int):
    ws = window_start(f1, S, W)
    return list(range(min(S, f1))) + list(range(ws, f1))


def rel_pos(f: int, f1: int, S: int, W: int) -> int:
    if f < S:
        return f
    return S + (f - window_start(f1, S, W))


def chunk_of(f: int, C: int) -> int:
    return f // C


def key_visible(kf: int, qf: int, f1: int, S: int, W: int, C: int,
                shot_k: int, shot_q: int) -> bool:
    ws = window_start(f1, S, W)
    in_cache = (0 <= kf < f1) and (kf < S or kf >= ws)
    if not in_cache:
        return False
    if chunk_of(kf, C) > chunk_of(qf, C):
        return False
    return kf < S or shot_k == shot_q


# ---------------------------------------------------- per-shot sink variant
# The other reading of the multi-shot attention sink (evermx.com,
# "Multi-Shot Generation"; hysenlabs.com lists a "multi-shot attention
# sink"): each shot re-anchors the sink to its own first S frames.
#   * frame f of a shot that starts at frame fs is a sink frame of that shot
#     iff f - fs < S; it lives in sink slot f - fs (replacing the previous
#     shot's), all other frames in window slot S + ((f - S) mod W);
#   * ws = max(S, f1 - W) as above; a sink slot is visible to query frame qf
#     iff it holds a frame of qf's shot; a window slot iff its frame is in
#     [ws, f1) and of qf's shot; block-causal as above;
#   * positions: a sink frame's position is its slot (f - fs); any other
#     frame's is S + (f - ws); queries likewise.

def slot_of_shot(f: int, fs: int, S: int, W: int) -> int:
    return f - fs if f - fs < S else S + (f - S) % W


def pos_shot(f: int, fs: int, f1: int, S: int, W: int) -> int:
    return f - fs if f - fs < S else S + (f - window_start(f1, S, W))


def key_visible_shot(kf: int, kslot: int, qf: int, f1: int, S: int, W: int, C: int,
                     shot_k: int, shot_q: int) -> bool:
    if not (0 <= kf < f1) or shot_k != shot_q or chunk_of(kf, C) > chunk_of(qf, C):
        return False
    return kslot < S or kf >= window_start(f1, S, W)
