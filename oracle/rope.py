"""Rotary position rotation (float64).

TEST INFRASTRUCTURE (CPU oracle); see oracle/__init__.py.

The pages name fused RoPE kernels (hysenlabs.com, "NVFP4, sequence parallel
and the async decode path"; heatdrop.ai, "The interesting bit") and RoPE made
relative to the KV cache (refft.com, relative RoPE and TriAttention
question) without the rotation itself.  Reading: the standard rotary
embedding over adjacent pairs, base 10000, applied to the leading rot_dim
dimensions; pair i (elements 2i, 2i+1) turns by angle pos * base^(-2i/rot_dim)
where pos is the frame's cache-relative position.  Dimensions past rot_dim
pass through unchanged.
"""
from __future__ import annotations

import numpy as np


def angles(pos, rot_dim: int, base: float = 10000.0) -> np.ndarray:
    """phi[..., i] = pos * base^(-2i/rot_dim), float64."""
    i = np.arange(rot_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / rot_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def rotate(x, pos, rot_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotate x[..., D] by positions pos (broadcast against x[..., 0])."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos)
    assert np.broadcast_shapes(pos.shape, x.shape[:-1]) == x.shape[:-1], "pos must broadcast to x[..., 0]"
    phi = angles(pos, rot_dim, base)
    c, s = np.cos(phi), np.sin(phi)
    y = x.copy()
    a = x[..., 0:rot_dim:2]
    b = x[..., 1:rot_dim:2]
    y[..., 0:rot_dim:2] = a * c - b * s
    y[..., 1:rot_dim:2] = a * s + b * c
    return y


# ------------------------------------------------ float32 rotation (stored keys)
# Where a rotation feeds the NVFP4 encoder (keys rotated before they are
# stored, and their re-rotation when the window slides) the rotated value
# decides codes, so its arithmetic must be fixed exactly.  The pages give no
# precision.  Reading: the rotation formula evaluated in IEEE float32 as
# written, one correctly rounded operation at a time -- the two products,
# then their difference or sum -- with the cos/sin table entries evaluated in
# float64 and rounded once to float32.  This is the plain float32 evaluation
# of the formula (no operation fused), which any float32 implementation can
# reproduce exactly.

def table_f32(n_pos: int, rot_dim: int, base: float = 10000.0) -> np.ndarray:
    """float32 [n_pos][rot_dim/2][2]: (cos, sin) of pos * base^(-2i/rot_dim),
    evaluated in float64 element by element and rounded to float32."""
    import math
    half = rot_dim // 2
    t = np.zeros((n_pos, half, 2), np.float32)
    for p in range(n_pos):
        for i in range(half):
            phi = float(p) * math.pow(base, -2.0 * i / float(rot_dim))
            t[p, i, 0] = np.float32(math.cos(phi))
            t[p, i, 1] = np.float32(math.sin(phi))
    return t


def rotate_f32(x, cs, inverse: bool = False) -> np.ndarray:
    """Rotate float32 x[..., D] pair by pair with float32 (cos, sin) rows
    cs[..., rot_dim/2, 2] (broadcast against x[..., 0]); pair i is elements
    (2i, 2i+1) and dimensions past rot_dim are copied.  Forward:
    (a, b) -> (fl(fl(a c) - fl(b s)), fl(fl(a s) + fl(b c))); the inverse
    turn uses -s."""
    x = np.asarray(x, dtype=np.float32)
    cs = np.asarray(cs, dtype=np.float32)
    rd = 2 * cs.shape[-2]
    c = cs[..., 0]
    s = -cs[..., 1] if inverse else cs[..., 1]
    y = x.copy()
    a = x[..., 0:rd:2]
    b = x[..., 1:rd:2]
    y[..., 0:rd:2] = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    y[..., 1:rd:2] = (a * s).astype(np.float32) + (b * c).astype(np.float32)
    return y
