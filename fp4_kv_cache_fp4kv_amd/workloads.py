"""Workload shapes and seeded synthetic inputs.

This module is shared by the tests, the benchmark and the CPU oracle's
callers.  It holds no step of the method: only layer shapes, stream
schedules and seeded random tensors.  The shapes stand in for the 1.3B and
5B causal video generators the LongLive 2.0 pages describe (evermx.com,
"Model Range and Hardware Requirements"); no dataset or checkpoint is
involved.

Random draws: for workload seed s, chunk step k and tensor id (Q=0, K=1,
V=2) the generator is ``numpy.random.default_rng(SeedSequence([s, k, id]))``.
Values are standard normal float32; where a workload has outliers, an
independent Bernoulli(p) mask drawn from the same generator multiplies the
chosen elements by a fixed factor.  bf16 workloads then round each value to
bf16 with round-to-nearest-even and keep it as float32 (exactly
representable) together with its uint16 bit pattern.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

Q_ID, K_ID, V_ID = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int            # attention heads
    D: int            # head dimension
    T: int            # latent tokens per frame
    C: int            # frames per chunk
    S: int            # attention-sink frames
    W: int            # window frames, including the current chunk
    n_frames: int     # stream length in frames
    seed: int
    dtype: str = "bf16"          # "f32" or "bf16" input tensors
    outlier_p: float = 0.0       # Bernoulli probability of an outlier
    outlier_scale: float = 1.0
    shot_len: Optional[int] = None   # frames per shot; None = one shot
    token_stride: int = 1        # keep every token_stride-th cached token

    @property
    def n_chunks(self) -> int:
        return -(-self.n_frames // self.C)

    @property
    def Tc(self) -> int:
        return self.T // self.token_stride

    @property
    def n_slots(self) -> int:
        return self.S + self.W

    def chunk_frames(self, c: int):
        """(f0, n) of chunk step c."""
        f0 = c * self.C
        return f0, min(self.C, self.n_frames - f0)

    def shot_of(self, f: int) -> int:
        return 0 if self.shot_len is None else f // self.shot_len


# The five configurations (listed small to large), then one GPU's head
# share.  "tiny" is the oracle-sized case; the others are shaped like one
# attention layer of the generators.
TINY = Workload("tiny", H=1, D=64, T=16, C=2, S=1, W=4, n_frames=12, seed=0,
                dtype="f32")
L13B = Workload("l13b", H=12, D=128, T=1560, C=3, S=3, W=12, n_frames=15,
                seed=2, outlier_p=0.01, outlier_scale=20.0)
L5B = Workload("l5b", H=24, D=128, T=880, C=3, S=3, W=12, n_frames=90, seed=3)
L5B_SHOTS = Workload("l5b_shots", H=24, D=128, T=880, C=3, S=3, W=12,
                     n_frames=80, seed=4, shot_len=20)
LONG = Workload("long", H=24, D=128, T=880, C=3, S=3, W=21, n_frames=720,
                seed=5, token_stride=2)
# One GPU's share of the 5B-like layer when 8 GPUs split its 24 heads: 3
# heads, 33 row blocks of 256 query rows (the case the split attention
# schedule exists for).
L5B_SHARE = Workload("l5b_share", H=3, D=128, T=880, C=3, S=3, W=12, n_frames=90, seed=6)

WORKLOADS = {w.name: w for w in (TINY, L13B, L5B, L5B_SHOTS, LONG, L5B_SHARE)}


def bf16_round(x: np.ndarray):
    """float32 -> (float32 values on the bf16 grid, uint16 bit patterns), RNE.

    Input conversion only (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    u32 = u.astype(np.uint32)
    return u32.view(np.float32), (u32 >> 16).astype(np.uint16)


def draw(w: Workload, step: int, tensor_id: int, n_tokens: Optional[int] = None):
    """Seeded tensor [n_tokens][H][D] for chunk step `step`.

    Returns (values float32, bits) where bits is the uint16 bf16 pattern
    for bf16 workloads and None for f32 workloads."""
    if n_tokens is None:
        n_tokens = w.chunk_frames(step)[1] * w.T
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, step, tensor_id]))
    x = rng.standard_normal((n_tokens, w.H, w.D), dtype=np.float32)
    if w.outlier_p > 0.0:
        m = rng.random((n_tokens, w.H, w.D), dtype=np.float32) < w.outlier_p
        x = np.where(m, x * np.float32(w.outlier_scale), x).astype(np.float32)
    if w.dtype == "bf16":
        return bf16_round(x)
    return x, None


def draw_qkv(w: Workload, step: int):
    """(q, k, v) as float32 arrays on the input grid, plus bf16 bit arrays."""
    out = []
    for tid in (Q_ID, K_ID, V_ID):
        out.append(draw(w, step, tid))
    return out
