// NVFP4 codec: per-tensor amax and in-place quantized append into the ring
// of sink + window slots ("in-place quantized KV-cache updates",
// hysenlabs.com, "NVFP4, sequence parallel and the async decode path").
//
// NVFP4 caches take two kernels per call, on the caller's stream:
//   amax_kernel    grid (kAmaxBlocks, 2): partial max |x| over the kept
//                  tokens of K (y = 0) and V (y = 1), one per workgroup.
//   encode_kernel  NVFP4 encode of both tensors straight into their cache
//                  slots (layouts in include/fp4kv.h), plus the slot metadata.
// The bf16 baseline format takes one kernel (store_bf16_kernel): a copy into
// the same ring layout.  For caches that store keys rotated, the same two
// kernels also turn the appended keys by their positions and re-encode the
// window slots a window move turns (grid rows / workgroups of their own).
#include <cstdlib>
#include <mutex>

#include "fp4kv_device.hpp"
#include "internal.hpp"
#include "rope_unit.hpp"

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
// maximum is taken on integers: bf16 halves with a packed 16-bit max, float32
// words directly.  Each thread keeps kAmaxUnroll 16-byte loads in flight.
constexpr int kAmaxUnroll = 4;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fold_max(uint32_t m, const uint4 &v, bool bf16) {
  if (bf16) {
    u16x2 acc = __builtin_bit_cast(u16x2, m);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    return __builtin_bit_cast(uint32_t, acc);
  }
  m = max(m, v.x & 0x7FFFFFFFu);
  m = max(m, v.y & 0x7FFFFFFFu);
  m = max(m, v.z & 0x7FFFFFFFu);
  return max(m, v.w & 0x7FFFFFFFu);
}

// Key block b of appended kept token (frame j, tc) and head h, as float32,
// turned by the frame's position when keys are stored rotated.
__device__ __forceinline__ void load_key_block(const AppendParams &p, int j, int tc, int h, int b,
                                              float (&x)[16]);

// Re-encoded window slot s: partial max |decoded key turned back| of this
// workgroup's share of the slot's (key row, block) pairs.
__device__ __forceinline__ void rerot_amax(const AppendParams &p, int s, uint32_t *red);

// This thread's max |x| (bit pattern) over the 16-byte chunks first,
// first + step, ... of appended tensor y (0 = K, 1 = V), kept tokens only.
__device__ __forceinline__ uint32_t amax_chunks(const AppendParams &p, int y, uint32_t first,
                                                uint32_t step) {
  const bool bf16 = p.in_bf16;
  const uint32_t row_chunks = (uint32_t)(p.H * p.D * (bf16 ? 2 : 4) / 16);  // one token
  const uint32_t n_chunks = (uint32_t)(p.n_frames * p.Tc) * row_chunks;
  const uint4 *base = (const uint4 *)p.x[y];
  uint32_t m = 0;
  for (uint32_t c0 = first; c0 < n_chunks; c0 += step * kAmaxUnroll) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k) {
      const uint32_t c = c0 + k * step;
      uint32_t addr = c;
      if (p.stride != 1) {   // kept token r is stored token r * stride (frames hold T tokens)
        const uint32_t r = c / row_chunks;
        const uint32_t frame = r / (uint32_t)p.Tc, tc = r - frame * (uint32_t)p.Tc;
        addr = (frame * (uint32_t)p.T + tc * (uint32_t)p.stride) * row_chunks + (c - r * row_chunks);
      }
      v[k] = c < n_chunks ? base[addr] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k) m = fold_max(m, v[k], bf16);
  }
  if (bf16) m = max(m & 0xFFFFu, m >> 16) << 16;   // bf16 bits -> float32 bits
  return m;
}

// Partial max |x| of appended tensor y (0 = K, 1 = V) over the kept tokens,
// taken by workgroup bx of nbx and stored as ws_partial[y][bx].
__device__ __forceinline__ void amax_part(const AppendParams &p, int y, int bx, int nbx,
                                          uint32_t *red) {
  uint32_t m = amax_chunks(p, y, (uint32_t)bx * kThreads + threadIdx.x, (uint32_t)nbx * kThreads);
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) p.ws_partial[y * kAmaxBlocks + bx] = m;
}

__global__ __launch_bounds__(kThreads) void amax_kernel(AppendParams p) {
  __shared__ uint32_t red[kThreads / 64];
  const int y = blockIdx.y;
  if (y >= p.amax_tensors) {               // window slots re-encoded by this call
    rerot_amax(p, p.S + (y - p.amax_tensors), red);
    return;
  }
  if (y == 0 && p.rotate_keys) {           // keys turned before they are stored
    const int nb = p.D >> 4;
    const uint32_t units = (uint32_t)(p.n_frames * p.Tc * p.H * nb);
    uint32_t m = 0;
    for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units;
         u += gridDim.x * kThreads) {
      const int b = (int)(u % nb);
      uint32_t rest = u / nb;
      const int h = (int)(rest % p.H);
      rest /= p.H;
      const int tc = (int)(rest % p.Tc);
      const int j = (int)(rest / p.Tc);
      float x[16];
      load_key_block(p, j, tc, h, b, x);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) p.ws_partial[blockIdx.x] = m;
    return;
  }
  amax_part(p, y, (int)blockIdx.x, (int)gridDim.x, red);
}

// Tensor scale g = amax / 2688 from the kAmaxBlocks partial maxima of tensor
// y (2688 = 6 * 448: the largest block then maps to the largest E4M3 scale;
// a tensor of zeros gets g = 1).  Every encode workgroup folds the partials
// itself, so no workgroup waits for another and no atomics are needed.
__device__ __forceinline__ float tensor_scale(const AppendParams &p, int y, uint32_t *red) {
  uint32_t m = 0;
  for (int i = threadIdx.x; i < kAmaxBlocks; i += kThreads)
    m = max(m, p.ws_partial[y * kAmaxBlocks + i]);
  m = block_max_u32(m, red);
  const float amax = __uint_as_float(m);
  return amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
}

// A caller-supplied tensor scale is used when it is finite and positive; any
// other value (zero, negative, infinite, NaN) is replaced by 1, so the cache
// never holds a scale that makes decoding or attention undefined.
__device__ __forceinline__ float caller_scale(float g) {
  return (g > 0.0f && g <= 3.4028235e38f) ? g : 1.0f;
}

// Encode one 16-element block: returns the two packed code words; *scale8
// receives the E4M3 scale code.  Every step rounds once, in float32, as the
// format definition states.  The element step y = x * r goes through the
// gfx950 float32 -> E2M1 conversion (scale 1), which rounds to nearest even
// and saturates exactly like e2m1_encode_mag (checked on every non-NaN
// float32); the sign of y is the sign of x.  x = 0 keeps its signed zero; a
// zero block scale zeroes every magnitude.
__device__ __forceinline__ uint2 encode_block(const float (&x)[16], float g, float d,
                                              uint32_t *scale8) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i]));
  const float s = __fdiv_rn(a, d);
  const uint32_t s8 = e4m3_encode_sat(s);
  const float sv = e4m3_value(s8);
  const float Sb = sv * g;
  float r = __frcp_rn(Sb);
  r = sv == 0.0f ? 0.0f : r;
  float y[16];
  if (__builtin_isinf(r)) {     // block scale below 2^-128: 0 * inf must stay 0
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = x[i] == 0.0f ? x[i] : x[i] * r;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = x[i] * r;
  }
  uint32_t w0 = 0u, w1 = 0u;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[0], y[1], 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[2], y[3], 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[4], y[5], 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[6], y[7], 1.0f, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[8], y[9], 1.0f, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[10], y[11], 1.0f, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[12], y[13], 1.0f, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[14], y[15], 1.0f, 3);
  *scale8 = s8;
  return make_uint2(w0, w1);
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

// Slot of appended frame j (computed on the host for either sink mode).
__device__ __forceinline__ int slot_of(const AppendParams &p, int j) { return p.slot[j]; }

// ---- keys stored rotated (FP4KV_FORMAT_NVFP4_ROT_V1) ----
// Every turn here feeds the encoder, so it uses rotate_pair_exact (products
// rounded before the sum).  Pair (2e, 2e+1) of key block b is rotary pair
// 8b + e; pairs past rot_dim / 2 are kept.

__device__ __forceinline__ void turn_block(float (&x)[16], const float *row, int b, int half_rot,
                                           bool back) {
  const float2 *cs = (const float2 *)row;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pair = 8 * b + e;
    if (pair < half_rot) {
      const float2 t = cs[pair];
      float ra, rb;
      rotate_pair_exact(x[2 * e], x[2 * e + 1], t.x, back ? -t.y : t.y, ra, rb);
      x[2 * e] = ra;
      x[2 * e + 1] = rb;
    }
  }
}

__device__ __forceinline__ void load_key_block(const AppendParams &p, int j, int tc, int h, int b,
                                              float (&x)[16]) {
  const long long tok = (long long)j * p.T + (long long)tc * p.stride;
  load_block(p, 0, (tok * p.H + h) * p.D + b * 16, x);
  if (p.rotate_keys)
    turn_block(x, p.cos_sin + (long long)p.pos[j] * (2 * p.half_rot), b, p.half_rot, false);
}

__device__ __forceinline__ bool rerot_slot(const AppendParams &p, int s) {
  const int f = p.slot_frame[s];
  return f >= p.rr_f_lo && f < p.rr_f_hi;
}

__device__ __forceinline__ long long rerot_row(const AppendParams &p, int s, uint32_t r) {
  const int h = (int)(r / (uint32_t)p.Tc), tc = (int)(r - (uint32_t)h * (uint32_t)p.Tc);
  return ((long long)h * p.n_slots + s) * p.Tc + tc;
}

// Stored key block (codes w, scale code s8, tensor scale g) decoded as
// sign * fl(fl(E2M1 * E4M3) * g) and turned back by the window move.  The
// gfx950 FP4 -> float32 conversion with scale 1 gives sign * E2M1 exactly
// (element 2i from the low nibble of byte i).
__device__ __forceinline__ void decode_turn(const AppendParams &p, uint2 w, uint32_t s8, float g,
                                            int b, float (&x)[16]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const float sv = e4m3_value(s8);
  const f32x2 e[8] = {   // the byte selector must be a constant
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.x, 1.0f, 0),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.x, 1.0f, 1),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.x, 1.0f, 2),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.x, 1.0f, 3),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.y, 1.0f, 0),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.y, 1.0f, 1),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.y, 1.0f, 2),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w.y, 1.0f, 3)};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = (e[i].x * sv) * g;
    x[2 * i + 1] = (e[i].y * sv) * g;
  }
  turn_block(x, p.rr_cs, b, p.half_rot, true);
}

__device__ __forceinline__ void rerot_amax(const AppendParams &p, int s, uint32_t *red) {
  if (!rerot_slot(p, s)) return;            // uniform over the workgroup
  const float g = p.tscale[0][s];
  const int nb = p.D >> 4;
  const uint32_t units = (uint32_t)(p.H * p.Tc * nb);
  uint32_t m = 0;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units; u += gridDim.x * kThreads) {
    const int b = (int)(u % (uint32_t)nb);
    const long long row = rerot_row(p, s, u / (uint32_t)nb);
    const uint2 w = *(const uint2 *)(p.codes[0] + row * (p.D >> 1) + b * 8);
    float x[16];
    decode_turn(p, w, p.scales[0][row * nb + b], g, b, x);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) {
    p.ws_rr[s * kAmaxBlocks + blockIdx.x] = m;
    if (blockIdx.x == 0) p.ws_rr_g[s] = g;
  }
}

// Workgroup rb of the re-encoding: slot S + rb / rr_blocks, one thread per
// (key row, block), in place, with g = amax / 2688 of the turned slot.
__device__ __forceinline__ void rerot_encode(const AppendParams &p, int rb, uint32_t *red) {
  const int s = p.S + rb / p.rr_blocks, blk = rb % p.rr_blocks;
  if (!rerot_slot(p, s)) return;            // uniform over the workgroup
  uint32_t m = 0;
  for (int i = threadIdx.x; i < kAmaxBlocks; i += kThreads) m = max(m, p.ws_rr[s * kAmaxBlocks + i]);
  m = block_max_u32(m, red);
  const float amax = __uint_as_float(m);
  const float g = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
  const float d = 6.0f * g;
  if (blk == 0 && threadIdx.x == 0) p.tscale[0][s] = g;
  const int nb = p.D >> 4;
  const uint32_t units = (uint32_t)(p.H * p.Tc * nb);
  const uint32_t u = (uint32_t)blk * kThreads + threadIdx.x;
  if (u >= units) return;
  const int b = (int)(u % (uint32_t)nb);
  const long long row = rerot_row(p, s, u / (uint32_t)nb);
  uint2 *cp = (uint2 *)(p.codes[0] + row * (p.D >> 1) + b * 8);
  float x[16];
  decode_turn(p, *cp, p.scales[0][row * nb + b], p.ws_rr_g[s], b, x);
  uint32_t s8;
  *cp = encode_block(x, g, d, &s8);
  p.scales[0][row * nb + b] = (uint8_t)s8;
}

// The step's first kernel when queries are rotated and a chunk appended in
// one call: workgroups [0, 2 kAmaxBlocks) take the partial maxima of K and V
// (as amax_kernel), the rest rotate the queries' units [0, n) (as
// rope_kernel).  encode_rope_kernel follows on the same stream with the
// remaining units.  The value encode is a few long-running workgroups (each
// thread encodes 8 blocks), so the second kernel has idle CUs that part of
// the rotation fills: with 5 of 8 eighths of the rotation in the first
// kernel, the 1.3B-like step's append and rotation took 26.1 us cold instead
// of 27.9 us with all of it there, and the 5B-like step's 27.5 instead of
// 29.0 us.
constexpr int kRopeFirstEighths = 5;
__global__ __launch_bounds__(kThreads) void rope_amax_kernel(RopeParams rp, AppendParams ap,
                                                             long long n) {
  __shared__ uint32_t red[kThreads / 64];
  const int b = (int)blockIdx.x;
  if (b < 2 * kAmaxBlocks) {
    amax_part(ap, b / kAmaxBlocks, b % kAmaxBlocks, kAmaxBlocks, red);
    return;
  }
  const long long nb = (long long)gridDim.x - 2 * kAmaxBlocks;
  for (long long u = (long long)(b - 2 * kAmaxBlocks) * kThreads + threadIdx.x; u < n;
       u += nb * kThreads)
    rope_unit(rp, u);
}

// One launch encodes both tensors.  Workgroups [0, p.v_blocks) encode the
// values, dimension-major: one thread per (8 tokens, 16-block) writes one
// 4-byte word (8 token nibbles) in each of the block's 16 dimension rows plus
// 8 scale bytes; padding tokens Tc..Tv-1 of the last group are written as
// zeros.  They start first because each thread carries 8 blocks.  The other
// workgroups encode the keys, token-major: one thread per (token, 16-block),
// blocks fastest, so a wave reads whole rows and writes contiguous bytes.
// Workgroups past both re-encode the window slots a window move turns.
__device__ __forceinline__ void encode_wg(const AppendParams &p, int bid, uint32_t *red) {
  const int nb = p.D >> 4;                                   // blocks per row
  if (bid >= p.v_blocks + p.k_blocks) {
    rerot_encode(p, bid - p.v_blocks - p.k_blocks, red);
    return;
  }
  const bool is_v = bid < p.v_blocks;
  const int y = is_v ? 1 : 0;
  const float g = p.tscale_in ? caller_scale(p.tscale_in[y]) : tensor_scale(p, y, red);
  const float d = 6.0f * g;

  if ((bid == 0 || bid == p.v_blocks) && (int)threadIdx.x < p.n_frames) {
    const int j = threadIdx.x, f = p.frame0 + j;
    const int slot = slot_of(p, j);
    p.tscale[y][slot] = g;
    if (y == 0) {
      p.slot_frame[slot] = f;
      p.slot_shot[slot] = p.shot[j];
    }
  }

  if (!is_v) {
    const uint32_t units = (uint32_t)(p.H * p.n_frames * p.Tc * nb);
    const uint32_t u = (uint32_t)(bid - p.v_blocks) * kThreads + threadIdx.x;
    if (u >= units) return;
    const int b = (int)(u % nb);
    uint32_t rest = u / nb;
    const int tc = (int)(rest % p.Tc);
    rest /= p.Tc;
    const int j = (int)(rest % p.n_frames);
    const int h = (int)(rest / p.n_frames);
    const int slot = slot_of(p, j);
    float x[16];
    load_key_block(p, j, tc, h, b, x);
    uint32_t s8;
    const uint2 packed = encode_block(x, g, d, &s8);
    const long long row = ((long long)h * p.n_slots + slot) * p.Tc + tc;
    *(uint2 *)(p.codes[0] + row * (p.D >> 1) + b * 8) = packed;
    p.scales[0][row * nb + b] = (uint8_t)s8;
    return;
  }

  const int groups = p.Tv >> 3;                              // 8-token groups
  const uint32_t units = (uint32_t)(p.H * p.n_frames * groups * nb);
  const uint32_t u = (uint32_t)bid * kThreads + threadIdx.x;
  if (u >= units) return;
  const int b = (int)(u % nb);
  uint32_t rest = u / nb;
  const int grp = (int)(rest % groups);
  rest /= groups;
  const int j = (int)(rest % p.n_frames);
  const int h = (int)(rest / p.n_frames);
  const int slot = slot_of(p, j);
  uint32_t rows[16];                                         // one word per dimension
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
__global__ __launch_bounds__(kThreads) void encode_kernel(AppendParams p) {
  __shared__ uint32_t red[kThreads / 64];
  encode_wg(p, (int)blockIdx.x, red);
}

// The step's second kernel: the encode (workgroups [0, v_blocks + k_blocks))
// and, in the workgroups after it, the query rotation's units [u0, n), which
// fill the CUs that the few long-running value workgroups leave idle.
__global__ __launch_bounds__(kThreads) void encode_rope_kernel(AppendParams p, RopeParams rp,
                                                               long long u0) {
  __shared__ uint32_t red[kThreads / 64];
  const int enc = p.v_blocks + p.k_blocks;
  if ((int)blockIdx.x < enc) {
    encode_wg(p, (int)blockIdx.x, red);
    return;
  }
  const long long n = rope_units(rp);
  const long long nb = (long long)gridDim.x - enc;
  for (long long u = u0 + (long long)((int)blockIdx.x - enc) * kThreads + threadIdx.x; u < n;
       u += nb * kThreads)
    rope_unit(rp, u);
}

// ---- the step's prologue in one pass (bf16 inputs) ----
// One launch over a grid that is resident all at once (four workgroups per
// CU, sized on the host from the kernel's occupancy):
//   1. every thread loads one item, 4 kept tokens x one 16-element block of
//      K or of V (128 bytes), and keeps it in registers; the workgroup's
//      partial maxima of K and V go to the workspace;
//   2. the workgroup arrives at a grid barrier, then rotates its share of
//      the queries while the others arrive;
//   3. once every workgroup has arrived, each folds the partial maxima into
//      g = amax / 2688 per tensor and every thread encodes the item it
//      holds.  The two threads of adjacent lanes hold the two 4-token halves
//      of one 8-token value group and exchange their 16-bit halves of the
//      group's code words.
// K and V are read from memory once, against twice for the two-kernel form.
// Cross-workgroup words (partial maxima, barrier counts and phases) are
// written and read with device-coherent accesses that do not stop in an
// XCD's L2, and a store is complete (vmcnt(0)) before the arrival that
// publishes it.  Atomics on one address are served one at a time, so the
// barrier has two levels: workgroup w counts in at group w % kBarGroups,
// the last of each group at the top count, and the last of those flips
// every group's phase word, which only that group's workgroups poll.  Each
// count is cleared by its last arrival, so the workspace is left as found;
// it must hold zeros before its first use.  A wait that exceeds
// kBarrierSpins polls (part of the grid kept from starting, e.g. by another
// such grid on a concurrent stream) gives up: the workgroup sets the error
// word and takes the maxima of K and V over all their elements itself, which
// gives the same tensor scales and needs no other workgroup, so every call
// completes with the same bytes.  The environment variable
// FP4KV_BARRIER_SPINS, read on every call, sets a lower limit, so that tests
// can force this path.
constexpr int kBarrierSpins = 1 << 20;
constexpr int kSc1 = 16;   // cache-policy operand: sc1, a device-coherent access
constexpr uint32_t kBufferWord3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(uint32_t *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, (int)kBufferWord3);
}

__device__ __forceinline__ void block_max2_u32(uint32_t &a, uint32_t &b, uint32_t (*red)[kThreads / 64]) {
  a = wave_max_u32(a);
  b = wave_max_u32(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = a;
    red[1][wave] = b;
  }
  __syncthreads();
  a = red[0][0];
  b = red[1][0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) {
    a = a > red[0][w] ? a : red[0][w];
    b = b > red[1][w] ? b : red[1][w];
  }
  __syncthreads();   // red is reused
}

// Items of the one-pass prologue: K items first, then V items; each is
// (head h, frame j, 4-token quarter-group qg, block b) with the two halves
// of an 8-token group in adjacent lanes and b next, so 16 lanes read a
// whole (token, head) row per token.  V items cover the padded tokens up to
// Tv (a multiple of 8); K items stop at the last kept token's 8-token group.
__host__ __device__ inline long long prologue_k_items(const AppendParams &p) {
  return (long long)p.H * p.n_frames * ((p.Tc + 7) >> 3) * (p.D >> 4) * 2;
}
__host__ __device__ inline long long prologue_v_items(const AppendParams &p) {
  return (long long)p.H * p.n_frames * (p.Tv >> 3) * (p.D >> 4) * 2;
}

__global__ __launch_bounds__(kThreads, 4) void prologue_kernel(RopeParams rp, AppendParams p) {
  __shared__ uint32_t red[2][kThreads / 64];
  __shared__ int go;
  const int G = (int)gridDim.x;
  const int nb = p.D >> 4;
  const uint32_t k_items = (uint32_t)prologue_k_items(p);
  const uint32_t n_items = k_items + (uint32_t)prologue_v_items(p);
  const uint32_t u = blockIdx.x * kThreads + threadIdx.x;
  // K items and V items are even in number, so both threads of a lane pair
  // hold items of the same tensor, group and block
  const bool has = u < n_items;
  const bool is_v = u >= k_items;
  const uint32_t iu = is_v ? u - k_items : u;
  const int groups = is_v ? (p.Tv >> 3) : ((p.Tc + 7) >> 3);
  const int half = (int)(iu & 1u);
  uint32_t rest = iu >> 1;
  const int b = (int)(rest % nb);
  rest /= nb;
  const int grp = (int)(rest % groups);
  rest /= groups;
  const int j = (int)(rest % p.n_frames);
  const int h = (int)(rest / p.n_frames);
  const int tc0 = 8 * grp + 4 * half;   // first of the item's 4 tokens

  // ---- 1. the item, 4 tokens of one block, held until the encode
  uint4 w[8];
  {
    const uint16_t *src = (const uint16_t *)p.x[is_v ? 1 : 0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tc = tc0 + i;
      if (has && tc < p.Tc) {
        const long long tok = (long long)j * p.T + (long long)tc * p.stride;
        const uint4 *q = (const uint4 *)(src + (tok * p.H + h) * p.D + b * 16);
        w[2 * i] = q[0];
        w[2 * i + 1] = q[1];
      } else {
        w[2 * i] = make_uint4(0, 0, 0, 0);
        w[2 * i + 1] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fold_max(m, w[i], true);
  m = max(m & 0xFFFFu, m >> 16) << 16;   // bf16 bits -> float32 bits
  uint32_t mk = (has && !is_v) ? m : 0u, mv = (has && is_v) ? m : 0u;
  block_max2_u32(mk, mv, red);

  // ---- 2. publish the partial maxima, arrive, rotate the queries' share
  const __amdgpu_buffer_rsrc_t part = ws_rsrc(p.ws_rr, (uint32_t)(2 * G * 4));
  const int n_groups = G < kBarGroups ? G : kBarGroups;
  const int grp_of_wg = (int)blockIdx.x % n_groups;
  const uint32_t grp_size = (uint32_t)((G - grp_of_wg + n_groups - 1) / n_groups);
  uint32_t *cnt = p.ws_bar + grp_of_wg * kBarLine, *phase = cnt + kWsBarPhase;
  uint32_t *top = p.ws_bar + kWsBarTop, *err = p.ws_bar + kWsBarError;
  uint32_t phase0 = 0;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_raw_buffer_store_b32(mk, part, 4 * (int)blockIdx.x, 0, kSc1);
    __builtin_amdgcn_raw_buffer_store_b32(mv, part, 4 * (G + (int)blockIdx.x), 0, kSc1);
    phase0 = __hip_atomic_load(phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the maxima are stored and the phase is read before the arrival counts
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == grp_size - 1u) {   // the group is complete: reset, count it in
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t old_top =
          __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old_top == (uint32_t)n_groups - 1u) {   // every group: reset, release all
        // (nothing reads the top count again during the call, so the release
        // need not wait for its reset)
        __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // every group's phase flips: all phases are equal between calls
        // (zero at first, and each call flips every group of its grid, whose
        // size is fixed per device)
        for (int g2 = 0; g2 < n_groups; ++g2)
          __hip_atomic_store(p.ws_bar + g2 * kBarLine + kWsBarPhase, phase0 ^ 1u,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  {
    // four units' reads in flight per thread
    const long long n = rope_units(rp), step = (long long)G * kThreads;
    for (long long q = u; q < n; q += 4 * step) {
      RopeIn in[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (q + k * step < n) in[k] = rope_load(rp, q + k * step);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (q + k * step < n) rope_finish(rp, q + k * step, in[k]);
    }
  }

  // ---- 3. wait for every arrival, fold the maxima, encode the item
  if (threadIdx.x == 0) {
    int ok = 1;
    for (int it = 0; __hip_atomic_load(phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == phase0;
         ++it) {
      if (it >= p.spin_limit) {
        __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    go = ok;
  }
  __syncthreads();
  uint32_t ak = 0u, av = 0u;
  if (go) {
    for (int i = threadIdx.x; i < G; i += kThreads) {
      ak = max(ak, __builtin_amdgcn_raw_buffer_load_b32(part, 4 * i, 0, kSc1));
      av = max(av, __builtin_amdgcn_raw_buffer_load_b32(part, 4 * (G + i), 0, kSc1));
    }
  } else {   // the wait gave up: the maxima over every element, alone
    ak = amax_chunks(p, 0, threadIdx.x, kThreads);
    av = amax_chunks(p, 1, threadIdx.x, kThreads);
  }
  block_max2_u32(ak, av, red);
  const float amax_k = __uint_as_float(ak), amax_v = __uint_as_float(av);
  const float gk = amax_k > 0.0f ? __fdiv_rn(amax_k, 2688.0f) : 1.0f;
  const float gv = amax_v > 0.0f ? __fdiv_rn(amax_v, 2688.0f) : 1.0f;
  if (blockIdx.x == 0 && (int)threadIdx.x < p.n_frames) {
    const int jj = threadIdx.x, slot = slot_of(p, jj);
    p.tscale[0][slot] = gk;
    p.tscale[1][slot] = gv;
    p.slot_frame[slot] = p.frame0 + jj;
    p.slot_shot[slot] = p.shot[jj];
  }
  const float g = is_v ? gv : gk;
  const float d = 6.0f * g;
  const int slot = has ? slot_of(p, j) : 0;
  uint32_t rows[16];   // values: 4 token nibbles (16 bits) per dimension
#pragma unroll
  for (int r = 0; r < 16; ++r) rows[r] = 0u;
  uint32_t sc = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tc = tc0 + i;
    if (!has || tc >= p.Tc) continue;   // past the frame: no key; value padding stays zero
    const uint32_t ww[8] = {w[2 * i].x, w[2 * i].y, w[2 * i].z, w[2 * i].w,
                            w[2 * i + 1].x, w[2 * i + 1].y, w[2 * i + 1].z, w[2 * i + 1].w};
    float x[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[2 * e] = __uint_as_float(ww[e] << 16);
      x[2 * e + 1] = __uint_as_float(ww[e] & 0xFFFF0000u);
    }
    uint32_t s8;
    const uint2 packed = encode_block(x, g, d, &s8);
    if (!is_v) {
      const long long row = ((long long)h * p.n_slots + slot) * p.Tc + tc;
      *(uint2 *)(p.codes[0] + row * (p.D >> 1) + b * 8) = packed;
      p.scales[0][row * nb + b] = (uint8_t)s8;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t code = ((r < 8 ? packed.x : packed.y) >> (4 * (r & 7))) & 0xFu;
        rows[r] |= code << (4 * i);
      }
      sc |= s8 << (8 * i);
    }
  }
  // Value word of dimension r of the group: the even lane's 4 tokens in the
  // low 16 bits, the odd lane's in the high 16 bits.  The even lane writes
  // dimensions 0-7 and the odd lane 8-15, each taking the other's half by
  // one exchange per word.  Every lane takes part (shuffles need them all).
  uint32_t word[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t give = half ? rows[r] : rows[r + 8];
    const uint32_t got = (uint32_t)__shfl_xor((int)give, 1, 64);
    word[r] = half ? (got | (rows[r + 8] << 16)) : (rows[r] | (got << 16));
  }
  if (has && is_v) {
    const long long vrow0 = ((long long)h * p.n_slots + slot) * p.D + 16 * b + 8 * half;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      *(uint32_t *)(p.codes[1] + (vrow0 + r) * (p.Tv >> 1) + 4 * grp) = word[r];
    const long long srow = ((long long)h * p.n_slots + slot) * nb + b;
    *(uint32_t *)(p.scales[1] + srow * p.Tv + tc0) = sc;
  }
}

// ---- bf16 baseline format: the append stores bf16, no quantization ----

// float32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(uint32_t u) {
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 8 consecutive inputs as 4 words of packed bf16 pairs.
__device__ __forceinline__ uint4 load8_bf16(const AppendParams &p, int y, long long src) {
  if (p.in_bf16) return *(const uint4 *)((const uint16_t *)p.x[y] + src);
  const uint4 a = *(const uint4 *)((const float *)p.x[y] + src);
  const uint4 b = *(const uint4 *)((const float *)p.x[y] + src + 4);
  return make_uint4(bf16_rne(a.x) | (bf16_rne(a.y) << 16), bf16_rne(a.z) | (bf16_rne(a.w) << 16),
                    bf16_rne(b.x) | (bf16_rne(b.y) << 16), bf16_rne(b.z) | (bf16_rne(b.w) << 16));
}

// Workgroups [0, p.v_blocks) store values: one thread per (head, frame,
// 8-token group, 8 dimensions) transposes an 8 x 8 tile into 8 dimension
// rows of 16 bytes (padding tokens as zeros).  The others store keys: one
// thread per (token, head, 8 dimensions) copies 16 bytes.
__global__ __launch_bounds__(kThreads) void store_bf16_kernel(AppendParams p) {
  const int n8 = p.D >> 3;
  if ((int)blockIdx.x >= p.v_blocks) {
    const uint32_t units = (uint32_t)(p.n_frames * p.Tc * p.H * n8);
    const uint32_t u = (blockIdx.x - p.v_blocks) * kThreads + threadIdx.x;
    if ((int)blockIdx.x == p.v_blocks && threadIdx.x < p.n_frames) {
      const int j = threadIdx.x, f = p.frame0 + j, sl = slot_of(p, j);
      p.tscale[0][sl] = 1.0f;
      p.tscale[1][sl] = 1.0f;
      p.slot_frame[sl] = f;
      p.slot_shot[sl] = p.shot[j];
    }
    if (u >= units) return;
    const int c8 = (int)(u % n8);
    uint32_t rest = u / n8;
    const int h = (int)(rest % p.H);
    rest /= p.H;
    const int tc = (int)(rest % p.Tc);
    const int j = (int)(rest / p.Tc);
    const long long tok = (long long)j * p.T + (long long)tc * p.stride;
    const uint4 v = load8_bf16(p, 0, (tok * p.H + h) * p.D + 8 * c8);
    const int slot = slot_of(p, j);
    const long long row = ((long long)h * p.n_slots + slot) * p.Tc + tc;
    *(uint4 *)(p.codes[0] + (row * p.D + 8 * c8) * 2) = v;
    return;
  }
  const int g8s = p.Tv >> 3;
  const uint32_t units = (uint32_t)(p.H * p.n_frames * n8 * g8s);
  const uint32_t u = blockIdx.x * kThreads + threadIdx.x;
  if (u >= units) return;
  const int g8 = (int)(u % g8s);
  uint32_t rest = u / g8s;
  const int c8 = (int)(rest % n8);
  rest /= n8;
  const int j = (int)(rest % p.n_frames);
  const int h = (int)(rest / p.n_frames);
  uint32_t e[8][4];   // e[token][word]: dims 8*c8 .. +7 of 8 tokens
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tc = 8 * g8 + i;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (tc < p.Tc) {
      const long long tok = (long long)j * p.T + (long long)tc * p.stride;
      v = load8_bf16(p, 1, (tok * p.H + h) * p.D + 8 * c8);
    }
    e[i][0] = v.x; e[i][1] = v.y; e[i][2] = v.z; e[i][3] = v.w;
  }
  const int slot = slot_of(p, j);
  const long long vrow0 = ((long long)h * p.n_slots + slot) * p.D + 8 * c8;
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {   // dimension 8*c8+dd across the 8 tokens
    uint32_t w[4];
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
      const uint32_t lo = (e[2 * t2][dd >> 1] >> (16 * (dd & 1))) & 0xFFFFu;
      const uint32_t hi = (e[2 * t2 + 1][dd >> 1] >> (16 * (dd & 1))) & 0xFFFFu;
      w[t2] = lo | (hi << 16);
    }
    *(uint4 *)(p.codes[1] + ((vrow0 + dd) * p.Tv + 8 * g8) * 2) = make_uint4(w[0], w[1], w[2], w[3]);
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

// ---- append workspace for callers that cannot allocate ----
// fp4kv_quantize_append_noalloc keeps the append's workspace (partial maxima,
// and the one-pass kernel's grid barrier) in this array instead of a caller
// buffer.  Each device holds its own copy for the life of the process; every
// call on a device shares it, so calls that overlap in time on one device
// race.  Nothing needs clearing between calls: every partial maximum read is
// written by the same call first, and the barrier words, zero at load, are
// left at zero counts by every call.
static __device__ __align__(256) uint8_t scratch[kWsBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device
}  // namespace

hipError_t append_scratch(void **out, size_t *bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // once per device, with that device current: the host-side name of the
    // array is not a device address, so only this pointer is ever used
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t launch_cache_reset(const fp4kv_cache &c, hipStream_t s) {
  const int n = c.sink_frames + c.window_frames;
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(64), 0, s, c.slot_frame, c.slot_shot,
                     c.k_tscale, c.v_tscale, n);
  return hipGetLastError();
}

namespace {

// Workgroup counts of the encode kernel (and of the bf16 store kernel).
void append_blocks(AppendParams &p) {
  if (p.bf16_cache) {
    const long long v_units = (long long)p.H * p.n_frames * (p.D >> 3) * (p.Tv >> 3);
    p.v_blocks = (int)((v_units + kThreads - 1) / kThreads);
    return;
  }
  const long long k_units = (long long)p.H * p.n_frames * p.Tc * (p.D >> 4);
  const long long v_units = (long long)p.H * p.n_frames * (p.Tv >> 3) * (p.D >> 4);
  const long long rr_units = (long long)p.H * p.Tc * (p.D >> 4);   // per re-encoded slot
  p.v_blocks = (int)((v_units + kThreads - 1) / kThreads);
  p.k_blocks = (int)((k_units + kThreads - 1) / kThreads);
  p.rr_blocks = p.rr_slots > 0 ? (int)((rr_units + kThreads - 1) / kThreads) : 0;
}

hipError_t launch_encode(const AppendParams &p, hipStream_t s) {
  const long long blocks = (long long)p.v_blocks + p.k_blocks + (long long)p.rr_slots * p.rr_blocks;
  if (blocks > 0)
    hipLaunchKernelGGL(encode_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

namespace {
// Workgroups of prologue_kernel that one device holds at once: compute
// units x resident workgroups per unit (resolved once per device).
std::mutex g_resident_mu;
int g_resident[kMaxDevices];

hipError_t prologue_resident(int *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_resident_mu);
  if (!g_resident[dev]) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prologue_kernel, kThreads, 0);
    if (e != hipSuccess) return e;
    g_resident[dev] = cus * (per_cu < 0 ? 0 : per_cu);
    if (!g_resident[dev]) g_resident[dev] = -1;
  }
  *out = g_resident[dev];
  return hipSuccess;
}

// The one-pass kernel for an NVFP4 append of bf16 inputs with computed
// tensor scales (and the rotation rp, which may have no tokens), when every
// item has a thread in a grid that the device holds at once.  The grid is
// all that fits, so the rotation's reads in flight fill every compute unit
// (workgroups past the items rotate only).  *done tells whether it ran.
hipError_t launch_one_pass(const RopeParams &rp, const AppendParams &ap, hipStream_t s,
                           bool *done) {
  *done = false;
  if (!ap.in_bf16 || ap.tscale_in || ap.bf16_cache || ap.rotate_keys || ap.rr_slots > 0 ||
      ap.n_frames < 1)
    return hipSuccess;
  int resident = 0;
  hipError_t e = prologue_resident(&resident);
  if (e != hipSuccess) return e;
  const long long items = prologue_k_items(ap) + prologue_v_items(ap);
  const long long need = (items + kThreads - 1) / kThreads;
  const long long grid = resident < kPrologueMaxGrid ? resident : kPrologueMaxGrid;
  if (resident <= 0 || need > grid) return hipSuccess;
  AppendParams a = ap;
  a.spin_limit = kBarrierSpins;
  if (const char *env = getenv("FP4KV_BARRIER_SPINS")) {
    char *end = nullptr;
    const long v = strtol(env, &end, 10);
    if (end != env && v >= 0 && v <= kBarrierSpins) a.spin_limit = (int)v;
  }
  hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, rp, a);
  *done = true;
  return hipGetLastError();
}
}  // namespace

hipError_t launch_append(const AppendParams &p_in, hipStream_t s) {
  AppendParams p = p_in;
  append_blocks(p);
  if (p.bf16_cache) {
    const long long k_units = (long long)p.n_frames * p.Tc * p.H * (p.D >> 3);
    const long long k_blocks = (k_units + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(store_bf16_kernel, dim3((unsigned)(p.v_blocks + k_blocks)), dim3(kThreads),
                       0, s, p);
    return hipGetLastError();
  }
  p.amax_tensors = (p.n_frames > 0 && !p.tscale_in) ? 2 : 0;
  {
    RopeParams none = {};   // no queries to rotate
    none.D = p.D;
    none.H = p.H;
    none.T = p.T;
    bool done = false;
    hipError_t e = launch_one_pass(none, p, s, &done);
    if (e != hipSuccess || done) return e;
  }
  const int amax_y = p.amax_tensors + p.rr_slots;
  if (amax_y > 0) {
    hipLaunchKernelGGL(amax_kernel, dim3(kAmaxBlocks, amax_y), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_encode(p, s);
}


hipError_t launch_rope_append(const RopeParams &rp, const AppendParams &ap_in, hipStream_t s) {
  AppendParams ap = ap_in;   // NVFP4 cache, computed tensor scales, no window move
  append_blocks(ap);
  ap.amax_tensors = 2;
  bool done = false;
  hipError_t e = launch_one_pass(rp, ap, s, &done);
  if (e != hipSuccess || done) return e;
  const long long n = rope_units(rp);
  const long long n1 = n * kRopeFirstEighths / 8;   // units rotated in the first kernel
  auto blocks_for = [](long long units) {
    long long b = (units + kThreads - 1) / kThreads;
    return b > 8192 ? 8192 : b;
  };
  hipLaunchKernelGGL(rope_amax_kernel, dim3((unsigned)(2 * kAmaxBlocks + blocks_for(n1))),
                     dim3(kThreads), 0, s, rp, ap, n1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long enc = (long long)ap.v_blocks + ap.k_blocks;
  hipLaunchKernelGGL(encode_rope_kernel, dim3((unsigned)(enc + blocks_for(n - n1))),
                     dim3(kThreads), 0, s, ap, rp, n1);
  return hipGetLastError();
}

}  // namespace fp4kv
