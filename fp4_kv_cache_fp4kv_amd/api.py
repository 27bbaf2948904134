"""Thin Python binding over the C ABI (argument marshalling only).

Torch tensors provide device memory and the current stream; every step of
the path runs in the HIP kernels of libfp4kv.so.  The function names follow
include/fp4kv.h: quantize_append, rope_rel, attention_chunk.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import FP4KV_BF16, FP4KV_F32, CacheDesc, check, load

_DTYPES = {torch.float32: FP4KV_F32, torch.bfloat16: FP4KV_BF16}


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _i32_array(vals: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


def _require(t: torch.Tensor, name: str, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class FP4KVCache:
    """Caller-owned buffers of one layer's KV cache plus its descriptor.

    kv_format "nvfp4" (layout in include/fp4kv.h: codes uint8
    [H][S+W][Tc][D/2], scales uint8 [H][S+W][Tc][D/16], tensor scales float32
    [S+W], slot metadata int32 [S+W]), "nvfp4_rot" (the same layout with keys
    stored already rotated; see rerotate_window) or "bf16", the unquantized
    baseline (keys bf16 [H][S+W][Tc][D], values bf16 [H][S+W][D][Tv], no
    scales).
    """

    FORMATS = {"nvfp4": _lib.FP4KV_FORMAT_NVFP4_V1, "nvfp4_rot": _lib.FP4KV_FORMAT_NVFP4_ROT_V1,
               "bf16": _lib.FP4KV_FORMAT_BF16_V1}

    def __init__(self, H: int, D: int, T: int, C: int, S: int, W: int,
                 token_stride: int = 1, rot_dim: Optional[int] = None,
                 device: str = "cuda:0", kv_format: str = "nvfp4",
                 sink_per_shot: bool = False):
        lib = load()
        if kv_format not in self.FORMATS:
            raise ValueError(f"kv_format must be one of {sorted(self.FORMATS)}")
        self.kv_format = kv_format
        self.device = torch.device(device)
        self.H, self.D, self.T, self.C, self.S, self.W = H, D, T, C, S, W
        self.token_stride = token_stride
        self.Tc = T // token_stride
        self.rot_dim = D if rot_dim is None else rot_dim
        tag = self.FORMATS[kv_format]
        self.desc = CacheDesc(format_tag=tag, n_heads=H, head_dim=D,
                              tokens_per_frame=T, token_stride=token_stride, chunk_frames=C,
                              sink_frames=S, window_frames=W, rot_dim=self.rot_dim,
                              sink_per_shot=int(bool(sink_per_shot)))
        self.sink_per_shot = bool(sink_per_shot)
        sizes = (ctypes.c_size_t * 6)()
        check(lib.fp4kv_cache_nbytes(ctypes.byref(self.desc), sizes), "fp4kv_cache_nbytes")
        self.Tv = -(-self.Tc // 32) * 32
        n = S + W
        dev = self.device
        self.k_codes = torch.zeros(sizes[0], dtype=torch.uint8, device=dev)
        self.v_codes = torch.zeros(sizes[1], dtype=torch.uint8, device=dev)
        self.k_scales = torch.zeros(sizes[2], dtype=torch.uint8, device=dev)
        self.v_scales = torch.zeros(sizes[3], dtype=torch.uint8, device=dev)
        self.k_tscale = torch.ones(n, dtype=torch.float32, device=dev)
        self.v_tscale = torch.ones(n, dtype=torch.float32, device=dev)
        self.slot_frame = torch.full((n,), -1, dtype=torch.int32, device=dev)
        self.slot_shot = torch.zeros(n, dtype=torch.int32, device=dev)
        for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_tscale", "v_tscale",
                     "slot_frame", "slot_shot"):
            t = getattr(self, name)
            setattr(self.desc, name, t.data_ptr() if t.numel() else 0)
        self.workspace = torch.zeros(lib.fp4kv_append_workspace_bytes(), dtype=torch.uint8,
                                     device=dev)
        # attention workspace for up to one workgroup per compute unit,
        # zero-filled once as the library requires
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        self.attn_workgroups = min(cus, _lib.FP4KV_MAX_WORKGROUPS)
        self.attn_workspace = torch.zeros(
            lib.fp4kv_attention_workspace_bytes(D, self.attn_workgroups), dtype=torch.uint8,
            device=dev)
        table = rope_table(n, self.rot_dim) if self.rot_dim > 0 else torch.zeros(2)
        self.cos_sin = table.to(dev)
        self.n_pos = n

    # views in the documented layout (for tests and inspection)
    def views(self):
        H, n, Tc, Tv, D = self.H, self.S + self.W, self.Tc, self.Tv, self.D
        if self.kv_format == "bf16":
            return dict(k_codes=self.k_codes.view(torch.int16).view(H, n, Tc, D),
                        v_codes=self.v_codes.view(torch.int16).view(H, n, D, Tv),
                        k_tscale=self.k_tscale, v_tscale=self.v_tscale,
                        slot_frame=self.slot_frame, slot_shot=self.slot_shot)
        return dict(k_codes=self.k_codes.view(H, n, Tc, D // 2),
                    v_codes=self.v_codes.view(H, n, D, Tv // 2),
                    k_scales=self.k_scales.view(H, n, Tc, D // 16),
                    v_scales=self.v_scales.view(H, n, D // 16, Tv),
                    k_tscale=self.k_tscale, v_tscale=self.v_tscale,
                    slot_frame=self.slot_frame, slot_shot=self.slot_shot)

    def reset(self):
        check(load().fp4kv_cache_reset(ctypes.byref(self.desc), _stream(self.device)),
              "fp4kv_cache_reset")


def rope_table(n_pos: int, rot_dim: int, base: float = 10000.0) -> torch.Tensor:
    """Host float32 [n_pos][rot_dim/2][2] table from the library's fp4kv_rope_table."""
    buf = (ctypes.c_float * (n_pos * rot_dim))()
    check(load().fp4kv_rope_table(buf, n_pos, rot_dim, base), "fp4kv_rope_table")
    return torch.frombuffer(bytearray(buf), dtype=torch.float32).clone()


def quantize_append(cache: FP4KVCache, k: torch.Tensor, v: torch.Tensor, frame0: int,
                    n_frames: int, shots: Sequence[int],
                    tscale: Optional[torch.Tensor] = None,
                    shot_starts: Optional[Sequence[int]] = None) -> None:
    """fp4kv_quantize_append on the current stream.  shot_starts (first frame
    of each frame's shot) is required by a cache with per-shot sinks."""
    for t, nm in ((k, "k"), (v, "v")):
        _require(t, nm, device=cache.device)
    if k.dtype != v.dtype or k.dtype not in _DTYPES:
        raise ValueError("k and v must both be float32 or bfloat16")
    if k.shape != (n_frames * cache.T, cache.H, cache.D) or v.shape != k.shape:
        raise ValueError(f"k/v must have shape {(n_frames * cache.T, cache.H, cache.D)}")
    if len(shots) != n_frames:
        raise ValueError("one shot id per frame")
    if tscale is not None:
        _require(tscale, "tscale", torch.float32, cache.device)
    st = load().fp4kv_quantize_append(
        ctypes.byref(cache.desc), k.data_ptr(), v.data_ptr(), _DTYPES[k.dtype], frame0, n_frames,
        _i32_array(shots), None if shot_starts is None else _i32_array(shot_starts),
        _ptr(tscale), cache.workspace.data_ptr(), cache.workspace.numel(),
        _stream(cache.device))
    check(st, "fp4kv_quantize_append")


def quantize_append_noalloc(cache: FP4KVCache, k: torch.Tensor, v: torch.Tensor, frame0: int,
                            n_frames: int, shots: Sequence[int],
                            tscale: Optional[torch.Tensor] = None,
                            shot_starts: Optional[Sequence[int]] = None) -> None:
    """fp4kv_quantize_append_noalloc on the current stream: the same append
    with the library's own per-device workspace (no caller workspace, no
    allocation)."""
    for t, nm in ((k, "k"), (v, "v")):
        _require(t, nm, device=cache.device)
    if k.dtype != v.dtype or k.dtype not in _DTYPES:
        raise ValueError("k and v must both be float32 or bfloat16")
    if k.shape != (n_frames * cache.T, cache.H, cache.D) or v.shape != k.shape:
        raise ValueError(f"k/v must have shape {(n_frames * cache.T, cache.H, cache.D)}")
    if len(shots) != n_frames:
        raise ValueError("one shot id per frame")
    if tscale is not None:
        _require(tscale, "tscale", torch.float32, cache.device)
    st = load().fp4kv_quantize_append_noalloc(
        ctypes.byref(cache.desc), k.data_ptr(), v.data_ptr(), _DTYPES[k.dtype], frame0, n_frames,
        _i32_array(shots), None if shot_starts is None else _i32_array(shot_starts),
        _ptr(tscale), _stream(cache.device))
    check(st, "fp4kv_quantize_append_noalloc")


def quantize_append_rotated(cache: FP4KVCache, k: torch.Tensor, v: torch.Tensor, frame0: int,
                            n_frames: int, shots: Sequence[int],
                            tscale: Optional[torch.Tensor] = None,
                            shot_starts: Optional[Sequence[int]] = None,
                            f1_prev: Optional[int] = None, f1: Optional[int] = None) -> None:
    """fp4kv_quantize_append_rotated on the current stream: the whole cache
    update of an "nvfp4_rot" cache (turn the surviving window keys from the
    window ending at f1_prev, default frame0, to the one ending at f1,
    default frame0 + n_frames; append the new keys rotated)."""
    if cache.kv_format != "nvfp4_rot":
        raise ValueError("quantize_append_rotated needs a cache with kv_format 'nvfp4_rot'")
    for t, nm in ((k, "k"), (v, "v")):
        _require(t, nm, device=cache.device)
    if k.dtype != v.dtype or k.dtype not in _DTYPES:
        raise ValueError("k and v must both be float32 or bfloat16")
    if k.shape != (n_frames * cache.T, cache.H, cache.D) or v.shape != k.shape:
        raise ValueError(f"k/v must have shape {(n_frames * cache.T, cache.H, cache.D)}")
    if len(shots) != n_frames:
        raise ValueError("one shot id per frame")
    if tscale is not None:
        _require(tscale, "tscale", torch.float32, cache.device)
    f1_prev = frame0 if f1_prev is None else f1_prev
    f1 = frame0 + n_frames if f1 is None else f1
    st = load().fp4kv_quantize_append_rotated(
        ctypes.byref(cache.desc), k.data_ptr(), v.data_ptr(), _DTYPES[k.dtype], frame0, n_frames,
        _i32_array(shots), None if shot_starts is None else _i32_array(shot_starts),
        _ptr(tscale), int(f1_prev), int(f1), cache.cos_sin.data_ptr(), cache.n_pos,
        cache.workspace.data_ptr(), cache.workspace.numel(), _stream(cache.device))
    check(st, "fp4kv_quantize_append_rotated")


def rerotate_window(cache: FP4KVCache, f1_from: int, f1_to: int) -> None:
    """fp4kv_rerotate_window on the current stream: turn the surviving window
    keys of an "nvfp4_rot" cache from the window ending at f1_from to the one
    ending at f1_to (call it before the append that moves the window)."""
    if cache.kv_format != "nvfp4_rot":
        raise ValueError("rerotate_window needs a cache with kv_format 'nvfp4_rot'")
    st = load().fp4kv_rerotate_window(
        ctypes.byref(cache.desc), int(f1_from), int(f1_to), cache.cos_sin.data_ptr(), cache.n_pos,
        cache.workspace.data_ptr(), cache.workspace.numel(), _stream(cache.device))
    check(st, "fp4kv_rerotate_window")


def rope_rel(x: torch.Tensor, pos0: int, tokens_per_frame: int, cos_sin: torch.Tensor,
             rot_dim: Optional[int] = None, out: Optional[torch.Tensor] = None,
             out_dtype=torch.float32) -> torch.Tensor:
    """fp4kv_rope_rel: rotate x [n_tokens][H][D] by frame positions pos0 + t/T.

    The output is float32 by default (the attention kernel's query input);
    bf16 output is also available.  out may alias x when the dtypes match."""
    _require(x, "x")
    if x.dtype not in _DTYPES or x.dim() != 3:
        raise ValueError("x must be float32/bfloat16 [n_tokens][H][D]")
    n_tok, H, D = x.shape
    rd = D if rot_dim is None else rot_dim
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _require(out, "out", None, x.device)
    if out.dtype not in _DTYPES or out.shape != x.shape:
        raise ValueError("out must be float32/bfloat16 with the shape of x")
    _require(cos_sin, "cos_sin", torch.float32, x.device)
    n_pos = cos_sin.numel() // max(rd, 1)
    st = load().fp4kv_rope_rel(x.data_ptr(), _DTYPES[x.dtype], out.data_ptr(), _DTYPES[out.dtype],
                               n_tok, H, D, tokens_per_frame, pos0, rd, cos_sin.data_ptr(), n_pos,
                               _stream(x.device))
    check(st, "fp4kv_rope_rel")
    return out


def attention_chunk(cache: FP4KVCache, q_rot: torch.Tensor, q_frame0: int, n_q_frames: int,
                    shots: Sequence[int], out_dtype=torch.bfloat16,
                    softmax_scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, n_workgroups: int = 0,
                    split: bool = True) -> torch.Tensor:
    """fp4kv_attention_chunk: q_rot float32 or bf16 [n_q_frames*T][H][D],
    already rotated by rope_rel.  The work is split over n_workgroups
    workgroups (0 = one per compute unit) using the cache's attention
    workspace; split=False passes no workspace (one workgroup per 256-row
    block)."""
    _require(q_rot, "q_rot", None, cache.device)
    if q_rot.dtype not in _DTYPES:
        raise ValueError("q_rot must be float32 or bfloat16")
    if q_rot.shape != (n_q_frames * cache.T, cache.H, cache.D):
        raise ValueError(f"q_rot must have shape {(n_q_frames * cache.T, cache.H, cache.D)}")
    if len(shots) != n_q_frames:
        raise ValueError("one shot id per query frame")
    if out is None:
        out = torch.empty(q_rot.shape, dtype=out_dtype, device=q_rot.device)
    _require(out, "out", out_dtype, cache.device)
    scale = 1.0 / math.sqrt(cache.D) if softmax_scale is None else softmax_scale
    ws = cache.attn_workspace if split else None
    st = load().fp4kv_attention_chunk(
        ctypes.byref(cache.desc), q_rot.data_ptr(), _DTYPES[q_rot.dtype], out.data_ptr(),
        _DTYPES[out_dtype], q_frame0, n_q_frames, _i32_array(shots), cache.cos_sin.data_ptr(),
        cache.n_pos, scale, int(n_workgroups), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream(cache.device))
    check(st, "fp4kv_attention_chunk")
    return out


def frame_position(cache: FP4KVCache, f: int, f1: int, shot_start: Optional[int] = None) -> int:
    """fp4kv_frame_position: cache-relative position of frame f at the step
    ending at frame f1 (shot_start: first frame of f's shot, per-shot sinks)."""
    pos = load().fp4kv_frame_position(ctypes.byref(cache.desc), int(f), int(f1),
                                      0 if shot_start is None else int(shot_start))
    check(min(pos, 0), "fp4kv_frame_position")
    return pos


def rope_rel_frames(cache: FP4KVCache, x: torch.Tensor, frame0: int, n_frames: int,
                    shot_starts: Optional[Sequence[int]] = None,
                    out: Optional[torch.Tensor] = None, out_dtype=torch.float32) -> torch.Tensor:
    """fp4kv_rope_rel_frames: rotate one chunk's tensor x [n_frames*T][H][D]
    by its frames' cache-relative positions (computed by the library) at the
    window ending at frame0 + n_frames.  shot_starts (first frame of each
    frame's shot) is required by a cache with per-shot sinks."""
    _require(x, "x", None, cache.device)
    if x.dtype not in _DTYPES or x.shape != (n_frames * cache.T, cache.H, cache.D):
        raise ValueError(f"x must be float32/bfloat16 {(n_frames * cache.T, cache.H, cache.D)}")
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _require(out, "out", None, x.device)
    if out.dtype not in _DTYPES or out.shape != x.shape:
        raise ValueError("out must be float32/bfloat16 with the shape of x")
    st = load().fp4kv_rope_rel_frames(
        ctypes.byref(cache.desc), x.data_ptr(), _DTYPES[x.dtype], out.data_ptr(),
        _DTYPES[out.dtype], frame0, n_frames,
        None if shot_starts is None else _i32_array(shot_starts), cache.cos_sin.data_ptr(),
        cache.n_pos, _stream(cache.device))
    check(st, "fp4kv_rope_rel_frames")
    return out


def rope_append(cache: FP4KVCache, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                frame0: int, n_frames: int, shots: Sequence[int],
                shot_starts: Optional[Sequence[int]] = None,
                q_out: Optional[torch.Tensor] = None, q_out_dtype=torch.float32) -> torch.Tensor:
    """fp4kv_rope_append on the current stream: rotate the chunk's queries
    (as rope_rel_frames) and append its keys and values (as quantize_append
    with computed tensor scales) in one call: one kernel for bfloat16 keys
    and values, two for float32.  Returns the rotated queries."""
    if cache.kv_format != "nvfp4":
        raise ValueError("rope_append needs a cache with kv_format 'nvfp4'")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, nm, device=cache.device)
    shape = (n_frames * cache.T, cache.H, cache.D)
    if k.dtype != v.dtype or k.dtype not in _DTYPES or q.dtype not in _DTYPES:
        raise ValueError("q, k and v must be float32 or bfloat16 (k and v alike)")
    if q.shape != shape or k.shape != shape or v.shape != shape:
        raise ValueError(f"q/k/v must have shape {shape}")
    if len(shots) != n_frames:
        raise ValueError("one shot id per frame")
    if q_out is None:
        q_out = torch.empty(shape, dtype=q_out_dtype, device=q.device)
    _require(q_out, "q_out", None, cache.device)
    if q_out.dtype not in _DTYPES or q_out.shape != shape:
        raise ValueError("q_out must be float32/bfloat16 with the shape of q")
    st = load().fp4kv_rope_append(
        ctypes.byref(cache.desc), q.data_ptr(), _DTYPES[q.dtype], q_out.data_ptr(),
        _DTYPES[q_out.dtype], k.data_ptr(), v.data_ptr(), _DTYPES[k.dtype], frame0, n_frames,
        _i32_array(shots), None if shot_starts is None else _i32_array(shot_starts),
        cache.cos_sin.data_ptr(), cache.n_pos, cache.workspace.data_ptr(),
        cache.workspace.numel(), _stream(cache.device))
    check(st, "fp4kv_rope_append")
    return q_out
