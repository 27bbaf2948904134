// One unit of the relative-RoPE rotation: 8 consecutive elements of one
// (token, head) row, rotated in float32 by the position of the token's frame
// (four rotary pairs, 32 bytes of table).  Each product is rounded before
// the sum (rotate_pair_exact), so keys rotated here before they are stored
// encode to the same codes wherever the rotation is reproduced.  Shared by
// the rotation kernel and the kernel that fuses it with the append's amax.
#pragma once

#include "fp4kv_device.hpp"
#include "internal.hpp"

namespace fp4kv {

// The unit's 8 input elements (one 16- or 32-byte read).
struct RopeIn {
  uint4 a, b;   // b is used by float32 inputs only
};
__device__ __forceinline__ RopeIn rope_load(const RopeParams &p, long long u) {
  const long long off = u * 8;   // units are consecutive 8-element groups
  RopeIn in;
  if (p.in_bf16) {
    in.a = *(const uint4 *)((const uint16_t *)p.x + off);
    in.b = make_uint4(0, 0, 0, 0);
  } else {
    in.a = *(const uint4 *)((const float *)p.x + off);
    in.b = *(const uint4 *)((const float *)p.x + off + 4);
  }
  return in;
}

// Rotates unit u from its loaded elements and stores it.
__device__ __forceinline__ void rope_finish(const RopeParams &p, long long u, const RopeIn &in) {
  const int groups = p.D >> 3;
  const int half = p.rot_dim >> 1;
  const int gi = (int)(u % groups);
  const long long row = u / groups;          // token * H + head
  const long long tok = row / p.H;
  const long long frame = tok / p.T;
  const int pos = p.per_frame ? p.pos[frame] : p.pos0 + (int)frame;
  const long long off = row * p.D + gi * 8;
  float x[8];
  if (p.in_bf16) {
    const uint32_t w[4] = {in.a.x, in.a.y, in.a.z, in.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    x[0] = __uint_as_float(in.a.x); x[1] = __uint_as_float(in.a.y);
    x[2] = __uint_as_float(in.a.z); x[3] = __uint_as_float(in.a.w);
    x[4] = __uint_as_float(in.b.x); x[5] = __uint_as_float(in.b.y);
    x[6] = __uint_as_float(in.b.z); x[7] = __uint_as_float(in.b.w);
  }
  const float *tab = p.cos_sin + (long long)pos * p.rot_dim;
  float r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pair = gi * 4 + i;
    r[2 * i] = x[2 * i];
    r[2 * i + 1] = x[2 * i + 1];
    if (pair < half) {
      const float2 cs = *(const float2 *)(tab + 2 * pair);
      rotate_pair_exact(x[2 * i], x[2 * i + 1], cs.x, cs.y, r[2 * i], r[2 * i + 1]);
    }
  }
  if (p.out_f32) {
    float4 *dst = (float4 *)((float *)p.y + off);
    dst[0] = make_float4(r[0], r[1], r[2], r[3]);
    dst[1] = make_float4(r[4], r[5], r[6], r[7]);
  } else {
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[i] = f32_to_bf16_bits(r[2 * i]) | (f32_to_bf16_bits(r[2 * i + 1]) << 16);
    *(uint4 *)((uint16_t *)p.y + off) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

__device__ __forceinline__ void rope_unit(const RopeParams &p, long long u) {
  rope_finish(p, u, rope_load(p, u));
}

// Units (8-element groups) of a rotation.
__host__ __device__ inline long long rope_units(const RopeParams &p) {
  return p.n_tokens * p.H * (p.D >> 3);
}

}  // namespace fp4kv
