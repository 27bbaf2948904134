// Relative RoPE: rotate a [n_tokens][H][D] tensor by cache-relative frame
// positions ("fused Triton RoPE", hysenlabs.com, "NVFP4, sequence parallel
// and the async decode path"; relative RoPE, refft.com, question "How do
// KV-cache relative RoPE and TriAttention work together ...").
//
// One thread per 8 consecutive elements of one (token, head) row: four rotary
// pairs and 32 bytes of table.  Memory-bound: 2 or 4 bytes read and 2 or 4
// written per element.  Products are rounded before the sum (no fused
// multiply-add), so keys rotated here before they are stored encode to the
// same codes wherever the rotation is reproduced.
#include "fp4kv_device.hpp"
#include "internal.hpp"

namespace fp4kv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void rope_kernel(RopeParams p) {
  const int groups = p.D >> 3;
  const long long n = p.n_tokens * p.H * groups;
  const int half = p.rot_dim >> 1;
  for (long long u = (long long)blockIdx.x * kThreads + threadIdx.x; u < n;
       u += (long long)gridDim.x * kThreads) {
    const int gi = (int)(u % groups);
    const long long row = u / groups;          // token * H + head
    const long long tok = row / p.H;
    const int pos = p.pos0 + (int)(tok / p.T);
    const long long off = row * p.D + gi * 8;
    float x[8];
    if (p.in_bf16) {
      const uint4 v = *(const uint4 *)((const uint16_t *)p.x + off);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *(const float4 *)((const float *)p.x + off);
      const float4 b = *(const float4 *)((const float *)p.x + off + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
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
}

}  // namespace

hipError_t launch_rope(const RopeParams &p, hipStream_t s) {
  const long long n = p.n_tokens * p.H * (p.D >> 3);
  long long blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fp4kv
