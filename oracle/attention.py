"""Masked softmax attention in float64.

TEST INFRASTRUCTURE (CPU oracle); see oracle/__init__.py.

For one head: scores s = (q . k) * scale over the keys a query may see,
p = softmax(s) over those keys, output o = sum_j p_j v_j.  This is the
attention the chunk-wise causal generator runs over its KV cache
(hysenlabs.com, "How it differs from a general diffusion pipeline"); masked
keys contribute nothing.  scale defaults to 1/sqrt(D).
"""
from __future__ import annotations

import numpy as np


def softmax_rows(s, mask):
    """Row softmax of s[Nq, Nk] over entries where mask is True (float64)."""
    s = np.asarray(s, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    assert np.all(mask.any(axis=1)), "every query must see at least one key"
    t = np.where(mask, s, -np.inf)
    m = np.max(t, axis=1, keepdims=True)
    e = np.where(mask, np.exp(t - m), 0.0)
    return e / np.sum(e, axis=1, keepdims=True)


def attend(q, k, v, mask, scale=None):
    """q[Nq, D], k[Nk, D], v[Nk, Dv], mask[Nq, Nk] -> o[Nq, Dv] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    p = softmax_rows((q @ k.T) * scale, mask)
    return p @ v
