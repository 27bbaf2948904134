"""ctypes declarations of the C ABI in include/fp4kv.h.

Loads the in-tree libfp4kv.so built for gfx950.  There is no fallback: if
the library is missing, every call raises.  Import torch before loading so
the library binds to the HIP runtime torch already loaded (same SONAME).
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4kv.so")

FP4KV_OK = 0
FP4KV_EINVAL = -1
FP4KV_ESHAPE = -2
FP4KV_EALIGN = -3
FP4KV_EFORMAT = -4
FP4KV_EDEVICE = -5
FP4KV_F32 = 0
FP4KV_BF16 = 1
FP4KV_FORMAT_NVFP4_V1 = 0x3146564E
FP4KV_FORMAT_BF16_V1 = 0x36314642
FP4KV_FORMAT_NVFP4_ROT_V1 = 0x3152564E
FP4KV_MAX_FRAMES = 64
FP4KV_MAX_WORKGROUPS = 4096
FP4KV_MAX_SLOTS = 64

EXPORTED = ("fp4kv_strerror", "fp4kv_abi_version", "fp4kv_cache_nbytes", "fp4kv_cache_reset",
            "fp4kv_append_workspace_bytes", "fp4kv_quantize_append", "fp4kv_rope_table",
            "fp4kv_rope_rel", "fp4kv_attention_chunk", "fp4kv_attention_workspace_bytes",
            "fp4kv_rerotate_window", "fp4kv_quantize_append_rotated",
            "fp4kv_quantize_append_noalloc", "fp4kv_frame_position", "fp4kv_rope_rel_frames",
            "fp4kv_rope_append")


class CacheDesc(ctypes.Structure):
    """Mirror of struct fp4kv_cache."""
    _fields_ = [
        ("format_tag", ctypes.c_uint32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tokens_per_frame", ctypes.c_int32),
        ("token_stride", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32),
        ("sink_frames", ctypes.c_int32),
        ("window_frames", ctypes.c_int32),
        ("rot_dim", ctypes.c_int32),
        ("sink_per_shot", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("k_tscale", ctypes.c_void_p),
        ("v_tscale", ctypes.c_void_p),
        ("slot_frame", ctypes.c_void_p),
        ("slot_shot", ctypes.c_void_p),
    ]


class FP4KVError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({strerror(status)})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load and declare the library (once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m fp4_kv_cache_fp4kv_amd.build")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    c_int, c_i32, c_i64, c_f = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    vp = ctypes.c_void_p
    lib.fp4kv_strerror.argtypes = [c_int]
    lib.fp4kv_strerror.restype = ctypes.c_char_p
    lib.fp4kv_abi_version.argtypes = []
    lib.fp4kv_abi_version.restype = c_int
    lib.fp4kv_cache_nbytes.argtypes = [P(CacheDesc), P(ctypes.c_size_t)]
    lib.fp4kv_cache_nbytes.restype = c_int
    lib.fp4kv_cache_reset.argtypes = [P(CacheDesc), vp]
    lib.fp4kv_cache_reset.restype = c_int
    lib.fp4kv_append_workspace_bytes.argtypes = []
    lib.fp4kv_append_workspace_bytes.restype = ctypes.c_size_t
    lib.fp4kv_quantize_append.argtypes = [P(CacheDesc), vp, vp, c_int, c_i32, c_i32, P(c_i32),
                                          P(c_i32),
                                          vp, vp, ctypes.c_size_t, vp]
    lib.fp4kv_quantize_append.restype = c_int
    lib.fp4kv_quantize_append_noalloc.argtypes = [P(CacheDesc), vp, vp, c_int, c_i32, c_i32,
                                                  P(c_i32), P(c_i32), vp, vp]
    lib.fp4kv_quantize_append_noalloc.restype = c_int
    lib.fp4kv_frame_position.argtypes = [P(CacheDesc), c_i32, c_i32, c_i32]
    lib.fp4kv_frame_position.restype = c_int
    lib.fp4kv_rope_rel_frames.argtypes = [P(CacheDesc), vp, c_int, vp, c_int, c_i32, c_i32,
                                          P(c_i32), vp, c_i32, vp]
    lib.fp4kv_rope_rel_frames.restype = c_int
    lib.fp4kv_rope_append.argtypes = [P(CacheDesc), vp, c_int, vp, c_int, vp, vp, c_int, c_i32,
                                      c_i32, P(c_i32), P(c_i32), vp, c_i32, vp, ctypes.c_size_t,
                                      vp]
    lib.fp4kv_rope_append.restype = c_int
    lib.fp4kv_rerotate_window.argtypes = [P(CacheDesc), c_i32, c_i32, vp, c_i32, vp,
                                          ctypes.c_size_t, vp]
    lib.fp4kv_rerotate_window.restype = c_int
    lib.fp4kv_quantize_append_rotated.argtypes = [P(CacheDesc), vp, vp, c_int, c_i32, c_i32,
                                                  P(c_i32), P(c_i32), vp, c_i32, c_i32, vp,
                                                  c_i32, vp, ctypes.c_size_t, vp]
    lib.fp4kv_quantize_append_rotated.restype = c_int
    lib.fp4kv_rope_table.argtypes = [P(c_f), c_i32, c_i32, ctypes.c_double]
    lib.fp4kv_rope_table.restype = c_int
    lib.fp4kv_rope_rel.argtypes = [vp, c_int, vp, c_int, c_i64, c_i32, c_i32, c_i32, c_i32,
                                   c_i32, vp, c_i32, vp]
    lib.fp4kv_rope_rel.restype = c_int
    lib.fp4kv_attention_chunk.argtypes = [P(CacheDesc), vp, c_int, vp, c_int, c_i32, c_i32,
                                          P(c_i32), vp, c_i32, c_f, c_i32, vp, ctypes.c_size_t,
                                          vp]
    lib.fp4kv_attention_chunk.restype = c_int
    lib.fp4kv_attention_workspace_bytes.argtypes = [c_i32, c_i32]
    lib.fp4kv_attention_workspace_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().fp4kv_strerror(status).decode()


def check(status: int, where: str) -> None:
    if status != FP4KV_OK:
        raise FP4KVError(status, where)
