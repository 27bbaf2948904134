"""GPU parity at the edges of the cache descriptor and of one call (same bar
as the other attention tests: cache bytes bit-exact, attention max-abs 1e-2 /
mean-abs 1e-3 against the oracle):

  * no sink frames (S = 0) on a wrapping stream;
  * one token per frame with a one-frame window and one-frame chunks;
  * an odd frame size well below one 64-key tile (T = 33);
  * the largest cache, S + W = 64 slots, through a wrap of the ring;
  * the largest call, 64 frames in one chunk (block-causal inside it);
  * the smallest rotary width, rot_dim = 2;
  * a requested workgroup count far above the key tiles (clamped).
"""
import pytest

from fp4_kv_cache_fp4kv_amd import workloads as wl
from test_gpu_attention import _run_stream

pytestmark = pytest.mark.gpu


def test_no_sink_frames_wrapping():
    w = wl.Workload("s0", H=2, D=64, T=24, C=2, S=0, W=4, n_frames=14, seed=61, dtype="f32")
    _run_stream(w, list(range(w.n_chunks)))


def test_one_token_frames_one_frame_window():
    w = wl.Workload("t1", H=4, D=128, T=1, C=1, S=1, W=1, n_frames=6, seed=62)
    _run_stream(w, list(range(w.n_chunks)))


def test_odd_frame_size_below_one_tile():
    w = wl.Workload("t33", H=2, D=64, T=33, C=3, S=2, W=6, n_frames=15, seed=63, dtype="f32")
    _run_stream(w, list(range(w.n_chunks)))


def test_largest_cache_64_slots_through_a_wrap():
    w = wl.Workload("slots64", H=2, D=64, T=16, C=4, S=4, W=60, n_frames=72, seed=64,
                    dtype="f32")
    _run_stream(w, [0, 7, 15, 16, 17])


def test_largest_call_64_frames_in_one_chunk():
    w = wl.Workload("c64", H=2, D=64, T=4, C=64, S=0, W=64, n_frames=64, seed=65, dtype="f32")
    _run_stream(w, [0])


def test_smallest_rotary_width():
    w = wl.Workload("rd2", H=2, D=128, T=40, C=2, S=1, W=4, n_frames=10, seed=66)
    _run_stream(w, [0, 2, 4], rot_dim=2)


def test_workgroup_request_above_the_key_tiles():
    w = wl.Workload("wg", H=2, D=128, T=100, C=3, S=1, W=6, n_frames=12, seed=67,
                    outlier_p=0.01, outlier_scale=20.0)
    _run_stream(w, [1, 3], n_wg=4096)
