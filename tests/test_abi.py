"""C-ABI checks that need no GPU: the built library loads, exports every
function include/fp4kv.h declares, and rejects bad arguments on the host
with the documented status codes before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

from fp4_kv_cache_fp4kv_amd import _lib
from fp4_kv_cache_fp4kv_amd._lib import CacheDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4kv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libfp4kv.so not built (python -m fp4_kv_cache_fp4kv_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4kv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_path_calls():
    names = declared_functions()
    for n in ("fp4kv_quantize_append", "fp4kv_attention_chunk", "fp4kv_rope_rel"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fp4kv_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    assert set(declared_functions()) == set(_lib.EXPORTED)


def test_ctypes_struct_matches_c_layout():
    # uint32 + 8 int32 = 36 bytes, pointers start at 40
    assert CacheDesc.k_codes.offset == 40
    assert ctypes.sizeof(CacheDesc) == 40 + 8 * 8


def _desc(**kw):
    d = dict(format_tag=_lib.FP4KV_FORMAT_NVFP4_V1, n_heads=2, head_dim=128, tokens_per_frame=32,
             token_stride=1, chunk_frames=3, sink_frames=3, window_frames=12, rot_dim=128)
    d.update(kw)
    c = CacheDesc(**d)
    for i, name in enumerate(("k_codes", "v_codes", "k_scales", "v_scales", "k_tscale",
                              "v_tscale", "slot_frame", "slot_shot")):
        setattr(c, name, 0x10000 * (i + 1))   # aligned fake addresses, never dereferenced
    return c


def test_strerror_and_version():
    lib = _lib.load()
    assert lib.fp4kv_abi_version() == 6
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.fp4kv_strerror(st)
    assert lib.fp4kv_append_workspace_bytes() >= 64 * 33 * 4   # re-rotation maxima


def test_append_workspace_layout():
    """The append workspace as the header states it: 76,288 bytes; the
    partial maxima [2][256], the re-encoding maxima [64][256] and the 64
    previous key scales first, then the one-pass kernel's grid barrier in
    the last 8448 bytes (33 lines of 64 words, 256-byte aligned), whose
    error word sits 128 bytes before the end."""
    lib = _lib.load()
    n = lib.fp4kv_append_workspace_bytes()
    assert n == 76288
    front = (2 * 256 + 64 * 256 + 64) * 4
    barrier = 33 * 64 * 4
    assert barrier == 8448 and front <= n - barrier and (n - barrier) % 256 == 0
    error_word = n - barrier + (32 * 64 + 32) * 4
    assert error_word == n - 128


def test_attention_workspace_bytes():
    lib = _lib.load()
    counters = 4 * _lib.FP4KV_MAX_WORKGROUPS
    # per workgroup: 2 partial results x 256 rows x (D floats + (m, l))
    assert lib.fp4kv_attention_workspace_bytes(128, 1) == counters + 2 * 256 * (4 * 128 + 8)
    assert lib.fp4kv_attention_workspace_bytes(64, 256) == counters + 256 * 2 * 256 * (4 * 64 + 8)
    assert lib.fp4kv_attention_workspace_bytes(128, 256) < 70_000_000
    for d, n in ((96, 4), (128, 0), (128, -1), (64, _lib.FP4KV_MAX_WORKGROUPS + 1)):
        assert lib.fp4kv_attention_workspace_bytes(d, n) == 0


def test_cache_nbytes():
    lib = _lib.load()
    out = (ctypes.c_size_t * 6)()
    c = _desc(token_stride=2)             # T = 32 -> Tc = 16 kept tokens, Tv = 32
    assert lib.fp4kv_cache_nbytes(ctypes.byref(c), out) == 0
    hs = 2 * 15
    assert list(out) == [hs * 16 * 64, hs * 128 * 16, hs * 16 * 8, hs * 8 * 32, 15 * 4, 15 * 4]
    c = _desc(tokens_per_frame=1560)      # Tv = 1568
    assert lib.fp4kv_cache_nbytes(ctypes.byref(c), out) == 0
    assert out[1] == hs * 128 * 784 and out[3] == hs * 8 * 1568


@pytest.mark.parametrize("field,value,status", [
    ("format_tag", 0x1234, -4),
    ("head_dim", 96, -2),
    ("head_dim", 256, -2),
    ("n_heads", 0, -1),
    ("token_stride", 3, -1),
    ("tokens_per_frame", 33, 0),       # fine with stride 1
    ("tokens_per_frame", 8388576, 0),  # largest frame at D = 128: 2 * D * Tv < 2^31
    ("tokens_per_frame", 8388577, -2), # Tv rounds up to 2^23: one slot reaches 2 GiB
    ("tokens_per_frame", 2**31 - 1, -2),
    ("window_frames", 2, -2),          # W < C
    ("sink_frames", 60, -2),           # S + W > 64
    ("rot_dim", 129, -1),
    ("rot_dim", 7, -1),
    ("sink_frames", -1, -1),
])
def test_descriptor_validation(field, value, status):
    lib = _lib.load()
    out = (ctypes.c_size_t * 6)()
    c = _desc(**{field: value})
    assert lib.fp4kv_cache_nbytes(ctypes.byref(c), out) == status


def test_bf16_format_sizes():
    lib = _lib.load()
    c = _desc(format_tag=_lib.FP4KV_FORMAT_BF16_V1)
    out = (ctypes.c_size_t * 6)()
    assert lib.fp4kv_cache_nbytes(ctypes.byref(c), out) == 0
    H, n, Tc, Tv, D = 2, 15, 32, 32, 128
    assert list(out) == [H * n * Tc * D * 2, H * n * D * Tv * 2, 0, 0, n * 4, n * 4]
    c = _desc(format_tag=0x12345678)
    assert lib.fp4kv_cache_nbytes(ctypes.byref(c), out) == _lib.FP4KV_EFORMAT


def test_rotated_format_has_the_nvfp4_sizes():
    lib = _lib.load()
    a, b = (ctypes.c_size_t * 6)(), (ctypes.c_size_t * 6)()
    assert lib.fp4kv_cache_nbytes(ctypes.byref(_desc()), a) == 0
    c = _desc(format_tag=_lib.FP4KV_FORMAT_NVFP4_ROT_V1)
    assert lib.fp4kv_cache_nbytes(ctypes.byref(c), b) == 0
    assert list(a) == list(b)


def test_rerotate_validation_before_launch():
    lib = _lib.load()
    c = _desc(format_tag=_lib.FP4KV_FORMAT_NVFP4_ROT_V1)     # S = 3, W = 12, C = 3
    A, Wk = 0x100000, 0x4000000
    ws = lib.fp4kv_append_workspace_bytes()
    call = lambda **kw: lib.fp4kv_rerotate_window(
        ctypes.byref(kw.get("c", c)), kw.get("f0", 15), kw.get("f1", 18), kw.get("cs", A),
        kw.get("npos", 15), kw.get("ws", Wk), kw.get("wsb", ws), None)
    assert call(c=_desc()) == -1                     # keys stored before rotation
    assert call(c=_desc(format_tag=_lib.FP4KV_FORMAT_BF16_V1)) == -1
    assert call(c=_desc(format_tag=7)) == -4
    assert call(f0=-1) == -1
    assert call(f0=18, f1=15) == -1                  # the window only moves forward
    assert call(ws=None) == -1
    assert call(cs=None) == -1
    assert call(wsb=ws - 1) == -2
    assert call(ws=Wk + 8) == -3
    assert call(cs=A + 4) == -3
    assert call(npos=3) == -2                        # delta 3 needs table row 3
    # nothing to move: window not full yet, no move, or nothing survives
    assert call(f0=6, f1=9) == 0
    assert call(f0=18, f1=18) == 0
    assert call(f0=15, f1=30) == 0
    r0 = _desc(format_tag=_lib.FP4KV_FORMAT_NVFP4_ROT_V1, rot_dim=0)
    assert call(c=r0, f0=6, f1=9, cs=None) == 0       # rot_dim 0 needs no table


def test_append_rotated_validation_before_launch():
    lib = _lib.load()
    c = _desc(format_tag=_lib.FP4KV_FORMAT_NVFP4_ROT_V1)     # S = 3, W = 12, C = 3
    A, Wk = 0x100000, 0x4000000
    shots = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    ws = lib.fp4kv_append_workspace_bytes()
    call = lambda **kw: lib.fp4kv_quantize_append_rotated(
        ctypes.byref(kw.get("c", c)), A, A, 1, kw.get("f0", 15), kw.get("n", 3), shots, None,
        None, kw.get("fp", 15), kw.get("f1", 18), kw.get("cs", A), kw.get("npos", 15),
        kw.get("ws", Wk), ws, None)
    assert call(c=_desc()) == -1                     # keys stored before rotation
    assert call(fp=-1) == -1
    assert call(fp=19) == -1                         # f1_prev > f1
    assert call(f1=17) == -1                         # frames past the window end
    assert call(fp=16) == -1                         # re-encoded and written frames overlap
    assert call(cs=None) == -1
    assert call(cs=A + 4) == -3
    assert call(npos=3) == -2                        # window move of 3 needs row 3
    assert call(npos=12) == -2                       # position 14 of frame 17
    assert call(f0=1, n=3, fp=21, f1=21) == -1       # frame 3 is not in the window [9, 21)
    assert call(f0=3, n=3, fp=21, f1=21) == -1       # frames 3..5 left the window
    assert call(n=0) == -1


def test_stride_must_divide_tokens():
    lib = _lib.load()
    out = (ctypes.c_size_t * 6)()
    c = _desc(token_stride=2, tokens_per_frame=33)
    assert lib.fp4kv_cache_nbytes(ctypes.byref(c), out) == -2


def test_append_validation_before_launch():
    lib = _lib.load()
    c = _desc()
    shots = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    ws = lib.fp4kv_append_workspace_bytes()
    A = 0x100000
    starts = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    call = lambda **kw: lib.fp4kv_quantize_append(
        ctypes.byref(kw.get("c", c)), kw.get("k", A), kw.get("v", A), kw.get("dt", 1),
        kw.get("f0", 0), kw.get("n", 3), kw.get("shots", shots), kw.get("starts", None), None,
        kw.get("ws", A), kw.get("wsb", ws), None)
    assert call(k=None) == -1
    assert call(dt=7) == -1
    assert call(n=0) == -1
    assert call(f0=3, n=13) == -1     # frames 3 and 15 share a window slot
    assert call(f0=0, n=16) == -1     # sink + window + one more
    assert call(f0=-1) == -1
    assert call(wsb=ws - 1) == -2
    assert call(k=A + 8) == -3
    assert call(ws=A + 4) == -3
    assert call(shots=None) == -1
    ps = _desc(sink_per_shot=1)
    assert call(c=ps) == -1                     # per-shot sinks need shot starts
    assert call(c=ps, f0=2, n=1, starts=(ctypes.c_int32 * 4)(3, 0, 0, 0)) == -1   # start > frame
    assert call(c=_desc(sink_per_shot=2)) == -1
    bad = _desc()
    bad.k_codes = 0x10008
    assert call(c=bad) == -3
    bad.k_codes = 0
    assert call(c=bad) == -1


def test_append_noalloc_validation_before_launch():
    """The no-alloc append validates like the workspace append, before it
    touches the device (only invalid calls here: a valid one would launch)."""
    lib = _lib.load()
    c = _desc()
    shots = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    A = 0x100000
    call = lambda **kw: lib.fp4kv_quantize_append_noalloc(
        ctypes.byref(kw.get("c", c)), kw.get("k", A), kw.get("v", A), kw.get("dt", 1),
        kw.get("f0", 0), kw.get("n", 3), kw.get("shots", shots), kw.get("starts", None),
        kw.get("ts", None), None)
    assert call(k=None) == -1
    assert call(dt=7) == -1
    assert call(n=0) == -1
    assert call(n=65) == -1
    assert call(f0=3, n=13) == -1
    assert call(k=A + 8) == -3
    assert call(ts=A + 2) == -3
    assert call(shots=None) == -1
    assert call(c=_desc(format_tag=7)) == -4
    assert call(c=_desc(sink_per_shot=1)) == -1


def test_frame_position_matches_the_oracle_rule():
    """The library's cache-relative position of every frame of every step of
    wrapping streams equals the oracle's (ring.rel_pos, ring.pos_shot); frames
    outside sink and window are rejected (host only, no GPU)."""
    from oracle import ring
    lib = _lib.load()
    for S, W, C in ((3, 12, 3), (0, 4, 2), (1, 4, 2), (2, 6, 3), (5, 21, 3)):
        c = _desc(sink_frames=S, window_frames=W, chunk_frames=C)
        for f1 in range(1, 60):
            ws = max(S, f1 - W)
            for f in range(0, f1 + 1):
                got = lib.fp4kv_frame_position(ctypes.byref(c), f, f1, 0)
                if f < f1 and (f < S or f >= ws):
                    assert got == ring.rel_pos(f, f1, S, W), (S, W, f, f1)
                else:
                    assert got == -1, (S, W, f, f1)
    c = _desc(sink_frames=2, window_frames=6, chunk_frames=3, sink_per_shot=1)
    for f1 in range(1, 40):
        for f in range(max(0, f1 - 6), f1):
            for fs in range(0, f + 1):
                got = lib.fp4kv_frame_position(ctypes.byref(c), f, f1, fs)
                want = ring.pos_shot(f, fs, f1, 2, 6)
                if f - fs < 2 or f >= max(2, f1 - 6):
                    assert got == want, (f, f1, fs)
                else:
                    assert got == -1
    assert lib.fp4kv_frame_position(ctypes.byref(c), 5, 9, 6) == -1   # start after frame
    assert lib.fp4kv_frame_position(ctypes.byref(_desc(format_tag=3)), 0, 1, 0) == -4


def test_rope_frames_and_rope_append_validation_before_launch():
    lib = _lib.load()
    c = _desc()                                   # H2 D128 T32 C3 S3 W12, rot_dim 128
    A, B, K, V = 0x100000, 0x200000, 0x300000, 0x400000
    shots = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    ws = lib.fp4kv_append_workspace_bytes()
    rf = lambda **kw: lib.fp4kv_rope_rel_frames(
        ctypes.byref(kw.get("c", c)), kw.get("x", A), kw.get("dt", 1), kw.get("y", B),
        kw.get("odt", 0), kw.get("f0", 0), kw.get("n", 3), kw.get("starts", None),
        kw.get("cs", A), kw.get("npos", 15), None)
    assert rf(x=None) == -1
    assert rf(n=0) == -1
    assert rf(n=65) == -1
    assert rf(f0=-1) == -1
    assert rf(npos=2) == -2            # position 2 is past a 2-row table
    assert rf(cs=None) == -1
    assert rf(y=B + 4) == -3
    assert rf(x=A, y=A, dt=1, odt=0) == -1       # in place needs matching dtypes
    assert rf(c=_desc(sink_per_shot=1)) == -1    # per-shot sinks need shot starts
    assert rf(f0=0, n=16, c=_desc(window_frames=12)) == -1   # frames 0..2 before the window
    assert rf(c=_desc(format_tag=3)) == -4
    ra = lambda **kw: lib.fp4kv_rope_append(
        ctypes.byref(kw.get("c", c)), kw.get("q", A), kw.get("qdt", 1), kw.get("qr", B),
        kw.get("qrdt", 0), kw.get("k", K), kw.get("v", V), kw.get("kvdt", 1), kw.get("f0", 0),
        kw.get("n", 3), kw.get("shots", shots), kw.get("starts", None), kw.get("cs", A),
        kw.get("npos", 15), kw.get("ws", A), kw.get("wsb", ws), None)
    assert ra(q=None) == -1
    assert ra(k=None) == -1
    assert ra(kvdt=4) == -1
    assert ra(wsb=ws - 1) == -2
    assert ra(ws=None) == -1
    assert ra(qr=K) == -1              # the rotated queries would overwrite K
    assert ra(qr=V) == -1
    assert ra(npos=1) == -2
    assert ra(c=_desc(format_tag=_lib.FP4KV_FORMAT_BF16_V1)) == -1
    assert ra(c=_desc(format_tag=_lib.FP4KV_FORMAT_NVFP4_ROT_V1)) == -1
    assert ra(f0=3, n=13) == -1        # frames 3 and 15 share a window slot


def test_rope_validation_before_launch():
    lib = _lib.load()
    A = 0x100000
    call = lambda **kw: lib.fp4kv_rope_rel(
        kw.get("x", A), kw.get("dt", 1), kw.get("y", A), kw.get("odt", 1), kw.get("n", 64), 2,
        kw.get("D", 128), kw.get("T", 16), kw.get("pos0", 0), kw.get("rd", 128), kw.get("cs", A),
        kw.get("npos", 4), None)
    assert call(x=None) == -1
    assert call(D=100) == -2
    assert call(rd=130) == -1
    assert call(pos0=4) == -2          # position past the table
    assert call(n=80) == -2            # 5 frames, 4 positions
    assert call(y=A + 2) == -3
    assert call(dt=0) == -1            # in place needs matching dtypes
    assert call(odt=3) == -1
    assert call(n=0) == 0              # nothing to do, nothing launched
    assert call(cs=None) == -1
    assert call(rd=0, cs=None, n=0) == 0   # rot_dim 0 reads no table
    assert call(rd=0, pos0=40, n=0) == 0
    assert call(rd=0, cs=None, n=2**62) == -2   # too large, rejected before the size product


def test_attention_validation_before_launch():
    lib = _lib.load()
    c = _desc()
    A, B = 0x100000, 0x200000
    shots = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    W = 0x4000000
    ws_bytes = lib.fp4kv_attention_workspace_bytes(128, 4)
    call = lambda **kw: lib.fp4kv_attention_chunk(
        ctypes.byref(kw.get("c", c)), kw.get("q", A), kw.get("qdt", 0), kw.get("o", B),
        kw.get("dt", 1), kw.get("f0", 0), kw.get("n", 3), kw.get("shots", shots), kw.get("cs", A),
        kw.get("npos", 15), kw.get("scale", 0.088), kw.get("nwg", 4), kw.get("ws", W),
        kw.get("wsb", ws_bytes), None)
    assert call(nwg=-1) == -1
    assert call(nwg=_lib.FP4KV_MAX_WORKGROUPS + 1) == -1
    assert call(wsb=ws_bytes - 1) == -2          # too small for 4 workgroups
    assert call(nwg=5) == -2
    assert call(ws=W + 8) == -3
    assert call(q=None) == -1
    assert call(o=A) == -1             # aliasing
    assert call(n=0) == -1
    assert call(n=65) == -1
    assert call(npos=14) == -2
    assert call(scale=0.0) == -1
    assert call(scale=float("inf")) == -1
    assert call(q=A + 4) == -3
    assert call(dt=5) == -1
    assert call(qdt=2) == -1
    assert call(c=_desc(format_tag=1)) == -4
    assert call(cs=None) == -1                       # keys stored before rotation need it
    rot = _desc(format_tag=_lib.FP4KV_FORMAT_NVFP4_ROT_V1)
    assert call(c=rot, cs=None, npos=0, n=0) == -1   # validation still runs


def test_rope_table_host_values():
    import math
    buf = (ctypes.c_float * (6 * 8))()
    assert _lib.load().fp4kv_rope_table(buf, 6, 8, 10000.0) == 0
    for p in range(6):
        for i in range(4):
            ang = p * 10000.0 ** (-2 * i / 8)
            assert abs(buf[(p * 4 + i) * 2] - math.cos(ang)) < 1e-7
            assert abs(buf[(p * 4 + i) * 2 + 1] - math.sin(ang)) < 1e-7
    assert _lib.load().fp4kv_rope_table(buf, 6, 7, 10000.0) == -1


def test_rope_table_matches_the_oracle_table_bit_for_bit():
    # keys stored rotated are encoded from rotations by this table, so the
    # library's host table and the oracle's must agree exactly
    import numpy as np
    from oracle import rope
    for n_pos, rd in ((15, 128), (8, 64), (21, 96)):
        buf = (ctypes.c_float * (n_pos * rd))()
        assert _lib.load().fp4kv_rope_table(buf, n_pos, rd, 10000.0) == 0
        lib_t = np.frombuffer(bytearray(buf), dtype=np.float32).reshape(n_pos, rd // 2, 2)
        assert np.array_equal(lib_t.view(np.uint32), rope.table_f32(n_pos, rd).view(np.uint32))
