// NVFP4 codec: per-tensor amax and in-place quantized append into the ring
// of sink + window slots ("in-place quantized KV-cache updates",
// hysenlabs.com, "NVFP4, sequence parallel and the async decode path").
//
// Two kernels per call, on the caller's stream:
//   amax_kernel    grid (kAmaxBlocks, 2): max |x| over the kept tokens of K
//                  (y = 0) and V (y = 1); the last workgroup to arrive folds
//                  the partial maxima into g = amax / 2688 and re-zeroes its
//                  arrival counter.  No workgroup waits for another.
//   encode_kernel  one thread per 16-element block of one (token, head) row;
//                  threads are ordered like the cache so each wave writes
//                  512 contiguous code bytes and 64 contiguous scale bytes.
#include "fp4kv_device.hpp"
#include "internal.hpp"

namespace fp4kv {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *red) {
  v = wave_max_u32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) r = r > red[w] ? r : red[w];
  return r;
}

// |x| bit patterns compare like the values for non-negative floats, so the
// maximum is taken on integers: bf16 halves are widened to float32 bits.
__global__ __launch_bounds__(kThreads) void amax_kernel(AppendParams p) {
  __shared__ uint32_t red[kThreads / 64];
  __shared__ int last;
  const int y = blockIdx.y;
  const int es = p.in_bf16 ? 2 : 4;
  const long long row_bytes = (long long)p.H * p.D * es;    // one token, all heads
  const int chunks_per_row = (int)(row_bytes / 16);
  const long long n_rows = (long long)p.n_frames * p.Tc;
  const long long n_chunks = n_rows * chunks_per_row;
  const uint8_t *base = (const uint8_t *)p.x[y];
  uint32_t m = 0;
  for (long long c = (long long)blockIdx.x * kThreads + threadIdx.x; c < n_chunks;
       c += (long long)gridDim.x * kThreads) {
    const long long r = c / chunks_per_row;
    const int within = (int)(c - r * chunks_per_row);
    const long long frame = r / p.Tc;
    const long long tc = r - frame * p.Tc;
    const long long tok = frame * p.T + tc * p.stride;
    const uint4 v = *(const uint4 *)(base + tok * row_bytes + (long long)within * 16);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (p.in_bf16) {
        const uint32_t lo = (w[i] & 0x7FFFu) << 16, hi = w[i] & 0x7FFF0000u;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
      } else {
        const uint32_t a = w[i] & 0x7FFFFFFFu;
        m = m > a ? m : a;
      }
    }
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) {
    __hip_atomic_store(&p.ws_partial[y * kAmaxBlocks + blockIdx.x], m, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    const uint32_t arrived = atomicAdd(&p.ws_counter[y], 1u);
    last = (arrived == (uint32_t)gridDim.x - 1u);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  uint32_t mm = 0;
  for (int i = threadIdx.x; i < (int)gridDim.x; i += kThreads) {
    const uint32_t v = __hip_atomic_load(&p.ws_partial[y * kAmaxBlocks + i], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    mm = mm > v ? mm : v;
  }
  __syncthreads();  // red[] is reused
  mm = block_max_u32(mm, red);
  if (threadIdx.x == 0) {
    const float amax = __uint_as_float(mm);
    // g = amax / (6 * 448): the largest block then maps to the largest E4M3
    // scale.  A tensor of zeros gets g = 1.
    p.ws_scale[y] = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
    p.ws_counter[y] = 0u;
  }
}

// Encode one 16-element block: returns the two packed code words; *scale8
// receives the E4M3 scale code.  Every step rounds once, in float32, as the
// format definition states.
__device__ __forceinline__ uint2 encode_block(const float (&x)[16], float g, float d,
                                              uint32_t *scale8) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i]));
  const float s = __fdiv_rn(a, d);
  const uint32_t s8 = e4m3_encode_sat(s);
  const float sv = e4m3_value(s8);
  const float Sb = sv * g;
  const float r = __frcp_rn(Sb);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float ax = fabsf(x[i]);
    uint32_t m = e2m1_encode_mag(ax * r);
    m = (sv == 0.0f || ax == 0.0f) ? 0u : m;
    const uint32_t code = ((__float_as_uint(x[i]) >> 31) << 3) | m;
    w[i >> 3] |= code << (4 * (i & 7));
  }
  *scale8 = s8;
  return make_uint2(w[0], w[1]);
}

__device__ __forceinline__ void load_block(const AppendParams &p, int y, long long src,
                                           float (&x)[16]) {
  if (p.in_bf16) {
    const uint4 *q = (const uint4 *)((const uint16_t *)p.x[y] + src);
    const uint4 v0 = q[0], v1 = q[1];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 *q = (const float4 *)((const float *)p.x[y] + src);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = q[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
  }
}

__device__ __forceinline__ int slot_of(const AppendParams &p, int f) {
  return f < p.S ? f : p.S + (f - p.S) % p.W;
}

// blockIdx.y = 0: keys, token-major rows.  One thread per (token, 16-block);
// blocks vary fastest, so a wave reads whole 256-byte rows and writes 512
// contiguous code bytes.
// blockIdx.y = 1: values, dimension-major.  One thread per (8 tokens,
// 16-block); it writes one 4-byte word (8 token nibbles) in each of the
// block's 16 dimension rows plus 8 scale bytes.  Padding tokens Tc..Tv-1 of
// the last group are written as zeros.
__global__ __launch_bounds__(kThreads) void encode_kernel(AppendParams p) {
  const int y = blockIdx.y;
  const float g = p.tscale_in ? p.tscale_in[y] : p.ws_scale[y];
  const float d = 6.0f * g;
  const int nb = p.D >> 4;                                   // blocks per row

  if (blockIdx.x == 0 && threadIdx.x < p.n_frames) {
    const int j = threadIdx.x, f = p.frame0 + j;
    const int slot = slot_of(p, f);
    p.tscale[y][slot] = g;
    if (y == 0) {
      p.slot_frame[slot] = f;
      p.slot_shot[slot] = p.shot[j];
    }
  }

  if (y == 0) {
    const long long units = (long long)p.H * p.n_frames * p.Tc * nb;
    for (long long u = (long long)blockIdx.x * kThreads + threadIdx.x; u < units;
         u += (long long)gridDim.x * kThreads) {
      const int b = (int)(u % nb);
      long long rest = u / nb;
      const int tc = (int)(rest % p.Tc);
      rest /= p.Tc;
      const int j = (int)(rest % p.n_frames);
      const int h = (int)(rest / p.n_frames);
      const int slot = slot_of(p, p.frame0 + j);
      const long long tok = (long long)j * p.T + (long long)tc * p.stride;
      float x[16];
      load_block(p, 0, (tok * p.H + h) * p.D + b * 16, x);
      uint32_t s8;
      const uint2 packed = encode_block(x, g, d, &s8);
      const long long row = ((long long)h * p.n_slots + slot) * p.Tc + tc;
      *(uint2 *)(p.codes[0] + row * (p.D >> 1) + b * 8) = packed;
      p.scales[0][row * nb + b] = (uint8_t)s8;
    }
    return;
  }

  const int groups = p.Tv >> 3;                              // 8-token groups
  const long long units = (long long)p.H * p.n_frames * groups * nb;
  for (long long u = (long long)blockIdx.x * kThreads + threadIdx.x; u < units;
       u += (long long)gridDim.x * kThreads) {
    const int b = (int)(u % nb);
    long long rest = u / nb;
    const int grp = (int)(rest % groups);
    rest /= groups;
    const int j = (int)(rest % p.n_frames);
    const int h = (int)(rest / p.n_frames);
    const int slot = slot_of(p, p.frame0 + j);
    uint32_t rows[16];                                       // one word per dimension
#pragma unroll
    for (int r = 0; r < 16; ++r) rows[r] = 0u;
    uint32_t sc_lo = 0u, sc_hi = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tc = 8 * grp + i;
      if (tc < p.Tc) {
        const long long tok = (long long)j * p.T + (long long)tc * p.stride;
        float x[16];
        load_block(p, 1, (tok * p.H + h) * p.D + b * 16, x);
        uint32_t s8;
        const uint2 packed = encode_block(x, g, d, &s8);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t code = ((r < 8 ? packed.x : packed.y) >> (4 * (r & 7))) & 0xFu;
          rows[r] |= code << (4 * i);
        }
        if (i < 4) sc_lo |= s8 << (8 * i);
        else sc_hi |= s8 << (8 * (i - 4));
      }
    }
    const long long vrow0 = ((long long)h * p.n_slots + slot) * p.D + 16 * b;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      *(uint32_t *)(p.codes[1] + (vrow0 + r) * (p.Tv >> 1) + 4 * grp) = rows[r];
    const long long srow = ((long long)h * p.n_slots + slot) * nb + b;
    *(uint2 *)(p.scales[1] + srow * p.Tv + 8 * grp) = make_uint2(sc_lo, sc_hi);
  }
}

__global__ void reset_kernel(int32_t *slot_frame, int32_t *slot_shot, float *kt, float *vt, int n) {
  const int i = threadIdx.x;
  if (i < n) {
    slot_frame[i] = -1;
    slot_shot[i] = 0;
    kt[i] = 1.0f;
    vt[i] = 1.0f;
  }
}

}  // namespace

hipError_t launch_cache_reset(const fp4kv_cache &c, hipStream_t s) {
  const int n = c.sink_frames + c.window_frames;
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(64), 0, s, c.slot_frame, c.slot_shot,
                     c.k_tscale, c.v_tscale, n);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams &p, hipStream_t s) {
  if (!p.tscale_in) {
    hipLaunchKernelGGL(amax_kernel, dim3(kAmaxBlocks, 2), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long units = (long long)p.H * p.n_frames * p.Tc * (p.D >> 4);
  // grid sized for the key pass; the value pass has 8x fewer threads and
  // strides over the same grid
  long long blocks = (units + kThreads - 1) / kThreads;
  if (blocks > 65535) blocks = 65535;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(encode_kernel, dim3((unsigned)blocks, 2), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fp4kv
