// Device helpers shared by the codec, RoPE and attention kernels (gfx950).
//
// NVFP4 element formats, written from their bit layouts:
//   E2M1  1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
//         0, 0.5, 1, 1.5, 2, 3, 4, 6.
//   E4M3  OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; largest
//         finite 448, subnormals m * 2^-9, no infinities.
// The KV cache is held in this format (evermx.com, "NVFP4 Quantization
// End-to-End"; hysenlabs.com, "NVFP4, sequence parallel and the async decode
// path").  All roundings are to nearest, ties to even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4kv {

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------------------ E4M3
// Code of a non-negative float32 s (may be +inf): nearest E4M3FN value,
// ties to even code, values >= 448 saturate to 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_sat(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  uint32_t bits = __float_as_uint(s);
  int e = (int)(bits >> 23) - 127;                 // float32 exponent of s
  if (e < -6) {
    // E4M3 subnormal range: the grid step is 2^-9 (q = 8 is 2^-6, code 8).
    return (uint32_t)rintf(s * 512.0f);
  }
  // Normal range: 8 grid steps per binade; s * 2^(3-e) lies in [8, 16).
  float scaled = s * __uint_as_float((uint32_t)(127 + 3 - e) << 23);
  uint32_t q = (uint32_t)rintf(scaled);            // 8..16; 16 carries up
  return ((uint32_t)(e + 7) << 3) + (q - 8u);
}

// Exact float32 value of a non-negative E4M3 code (0x00..0x7E).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  uint32_t e = code >> 3, m = code & 7u;
  float sub = (float)m * (1.0f / 512.0f);
  float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// ------------------------------------------------------------------ E2M1
// 3-bit magnitude code of y >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to
// the even code, saturating at 6.  Each threshold is a midpoint between two
// neighbours; '>' sends the tie down and '>=' sends it up, whichever
// neighbour has the even code.  NaN gives 0.
__device__ __forceinline__ uint32_t e2m1_encode_mag(float y) {
  return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
         (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
         (uint32_t)(y > 5.0f);
}

// float32 magnitude of a 3-bit E2M1 code (exact).
__device__ __forceinline__ float e2m1_value(uint32_t mag) {
  // mag >= 2: 2^(e-1) * (1 + m/2) with e = mag >> 1, m = mag & 1.
  float nrm = __uint_as_float((((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22));
  return mag >= 2u ? nrm : 0.5f * (float)mag;
}

// ------------------------------------------------------------------ RoPE
// Rotate the pair (a, b) by the angle whose cosine and sine are (c, s):
// (a c - b s, a s + b c).  The inverse rotation passes -s.
__device__ __forceinline__ void rotate_pair(float a, float b, float c, float s,
                                            float &ra, float &rb) {
  ra = a * c - b * s;
  rb = a * s + b * c;
}

// The same turn with every product rounded to float32 before the sum is
// rounded (no fused multiply-add): the arithmetic of rotations whose result
// is stored or NVFP4-encoded, so that it can be reproduced exactly.
__device__ __forceinline__ void rotate_pair_exact(float a, float b, float c, float s,
                                                  float &ra, float &rb) {
#pragma clang fp contract(off)
  ra = a * c - b * s;
  rb = a * s + b * c;
}

}  // namespace fp4kv
