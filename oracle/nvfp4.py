"""NVFP4 encoding and decoding, written from the format definition.

TEST INFRASTRUCTURE (CPU oracle); see oracle/__init__.py.

The pages say the KV cache is held in NVFP4, the same 4-bit floating-point
format as the W4A4 weights and activations (hysenlabs.com, "NVFP4, sequence
parallel and the async decode path"; evermx.com, "NVFP4 Quantization
End-to-End").  They do not spell the format out.  The public definition of
NVFP4 is used:
  * elements are E2M1 (1 sign, 2 exponent, 1 mantissa bit; magnitudes
    0, 0.5, 1, 1.5, 2, 3, 4, 6);
  * every 16 consecutive elements share one E4M3 scale (OCP E4M3FN:
    bias 7, largest finite 448, no infinities, subnormals 2^-9 .. 7*2^-9);
  * one FP32 scale covers the whole tensor.

Readings where the format leaves a choice (all conversions round to nearest,
ties to even):
  * tensor scale g = amax / 2688 (2688 = 6 * 448, so the largest block maps
    to the largest E4M3 scale), g = 1 when amax = 0;
  * block scale code s8 = E4M3(a_b / (6 g)), saturating at 448;
  * element code m = E2M1(|x| * (1 / (value(s8) * g))), saturating at 6,
    with the reciprocal correctly rounded, and magnitude 0 for every element
    of a block whose scale decodes to 0 and for every zero element;
  * the sign bit is the IEEE sign bit of x, so negative zero and small
    negatives encode as 0x8;
  * two elements per byte, element 2j in the low nibble.
All arithmetic the encoder does is float32 with IEEE rounding, exactly as
written below; the search for the nearest code is done in float64, where
every float32 input and every midpoint is exact.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
E4M3_MAX = 448.0
E2M1_MAX = 6.0
TENSOR_DIVISOR = 2688.0  # 6 * 448
BLOCK = 16

# E2M1 magnitude of each 3-bit code (sign handled separately).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e4m3_decode(code) -> np.ndarray:
    """E4M3FN byte -> float64 value (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    normal = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    sub = (m / 8.0) * 2.0 ** -6
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(sign == 1, -v, v)


# Non-negative finite E4M3 values in code order 0x00..0x7E; increasing.
_E4M3_POS = e4m3_decode(np.arange(0x7F))


def _nearest_even(x: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to x (x >= 0, grid increasing,
    grid[0] = 0), ties to the even index, values past the end -> last."""
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(grid, x, side="left")          # grid[hi-1] < x <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    dlo = x - grid[lo]
    dhi = grid[hi] - x
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(x >= grid[-1], len(grid) - 1, idx)  # saturate
    return idx.astype(np.int64)


def e4m3_encode(s) -> np.ndarray:
    """Non-negative float32 -> E4M3FN code (uint8), RNE, saturating to 448."""
    s = np.asarray(s, dtype=np.float32)
    assert not np.any(np.isnan(s)) and np.all(s >= 0)
    return _nearest_even(s.astype(np.float64), _E4M3_POS).astype(np.uint8)


def e2m1_encode_mag(y) -> np.ndarray:
    """|y| (float32, may be +inf) -> 3-bit E2M1 magnitude code, RNE, saturating."""
    y = np.asarray(y, dtype=np.float32)
    assert not np.any(np.isnan(y)) and np.all(y >= 0)
    return _nearest_even(y.astype(np.float64), E2M1_VALUES).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    """4-bit E2M1 code -> float64 value."""
    c = np.asarray(code).astype(np.int64)
    v = E2M1_VALUES[c & 7]
    return np.where((c >> 3) & 1, -v, v)


def tensor_scale(x) -> np.float32:
    """Per-tensor FP32 scale g of one appended tensor (float32 array)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(TENSOR_DIVISOR))


def encode_blocks(x, g):
    """NVFP4 encode of float32 x[..., D] (D % 16 == 0) with tensor scale g.

    Returns (codes uint8[..., D] one 4-bit code per element,
             scales uint8[..., D/16] E4M3 block-scale codes)."""
    x = np.asarray(x, dtype=np.float32)
    g = np.float32(g)
    assert np.all(np.isfinite(x)) and np.isfinite(g) and g > 0
    D = x.shape[-1]
    assert D % BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (D // BLOCK, BLOCK))
    a = np.max(np.abs(xb), axis=-1)                       # float32, exact
    d = np.float32(np.float32(6.0) * g)                   # fl(6 g)
    s = (a / d).astype(np.float32)                        # fl(a_b / d)
    s8 = e4m3_encode(np.where(np.isinf(s), np.float32(np.inf), s))
    sv = e4m3_decode(s8).astype(np.float32)               # exact in float32
    Sb = (sv * g).astype(np.float32)                      # fl(sv g)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = (np.float32(1.0) / Sb).astype(np.float32)     # fl(1 / S_b)
        y = (np.abs(xb) * r[..., None]).astype(np.float32)  # fl(|x| r)
    zero = (sv[..., None] == 0) | (xb == 0)
    y = np.where(zero, np.float32(0.0), y)
    m = e2m1_encode_mag(y)
    sign = np.signbit(xb).astype(np.uint8)
    codes = (sign << 3) | m
    return codes.reshape(x.shape), s8


def decode_blocks(codes, scales, g) -> np.ndarray:
    """Inverse map: float32 x_hat = sign * fl(fl(E2M1(m) * value(s8)) * g)."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    cb = codes.reshape(codes.shape[:-1] + (D // BLOCK, BLOCK))
    mag = E2M1_VALUES[cb & 7].astype(np.float32)
    sv = e4m3_decode(scales).astype(np.float32)
    prod = (mag * sv[..., None]).astype(np.float32)       # exact
    val = (prod * np.float32(g)).astype(np.float32)
    val = np.where((cb >> 3) & 1, -val, val).astype(np.float32)
    return val.reshape(codes.shape)


def pack_nibbles(codes) -> np.ndarray:
    """uint8 codes[..., D] -> bytes[..., D/2]; element 2j low, 2j+1 high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
