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
