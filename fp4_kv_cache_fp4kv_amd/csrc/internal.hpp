// Internal launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4kv.h"

namespace fp4kv {

// Number of partial maxima per tensor in the append workspace.
constexpr int kAmaxBlocks = 256;

// Partial maxima per cache slot in the re-rotation's amax pass.
constexpr int kRotParts = 32;

// Workspace of fp4kv_quantize_append: uint32 partial maxima [2][kAmaxBlocks]
// (float32 bit patterns of max |x| per workgroup of the amax pass).  The
// window re-rotation uses the same workspace: partial maxima
// [FP4KV_MAX_SLOTS][kRotParts], then the old tensor scales [FP4KV_MAX_SLOTS].
constexpr size_t kAppendWsBytes = 2 * kAmaxBlocks * sizeof(uint32_t);
constexpr size_t kRotWsBytes = (size_t)FP4KV_MAX_SLOTS * (kRotParts + 1) * sizeof(uint32_t);
constexpr size_t kWsBytes = kAppendWsBytes > kRotWsBytes ? kAppendWsBytes : kRotWsBytes;

struct AppendParams {
  const void *x[2];        // K, V inputs [n_frames*T][H][D]
  uint8_t *codes[2];
  uint8_t *scales[2];
  float *tscale[2];
  int32_t *slot_frame, *slot_shot;
  const float *tscale_in;  // device [2] or null
  uint32_t *ws_partial;    // [2][kAmaxBlocks]
  int H, D, T, stride, Tc, Tv, S, W, n_slots, frame0, n_frames;
  int in_bf16;
  int bf16_cache;          // FP4KV_FORMAT_BF16_V1: store bf16, no quantization
  int v_blocks;            // workgroups of the value pass in encode_kernel
  int32_t shot[FP4KV_MAX_FRAMES];
  int32_t slot[FP4KV_MAX_FRAMES];   // cache slot of each frame (host-computed)
};

// Window re-rotation of keys stored rotated (FP4KV_FORMAT_NVFP4_ROT_V1).
struct RerotParams {
  uint8_t *codes, *scales;   // key codes and block scales
  float *tscale;             // key tensor scales [n_slots]
  const int32_t *slot_frame;
  const float *cs;           // table row delta: (cos, sin) per rotary pair
  uint32_t *ws_max;          // [n_slots][kRotParts] partial maxima
  float *ws_g;               // [n_slots] tensor scales before the call
  int H, D, Tc, S, n_slots, half_rot;
  int f_lo, f_hi;            // window frames f_lo <= f < f_hi are turned
};

struct RopeParams {
  const void *x;
  void *y;
  const float *cos_sin;
  long long n_tokens;
  int H, D, T, pos0, rot_dim, in_bf16, out_f32;
};

struct AttnParams {
  const void *q;           // rotated queries [Nq][H][D], float32 or bf16
  void *o;                 // [Nq][H][D]
  const uint8_t *k_codes, *v_codes, *k_scales, *v_scales;
  const float *k_tscale, *v_tscale;
  const int32_t *slot_frame, *slot_shot;
  const float *cos_sin;
  int H, T, Tc, Tv, C, S, W, n_slots, rot_dim;
  int q_frame0, n_q_frames, Nq, q_f32;
  int bf16_cache;          // keys and values are bf16 (FP4KV_FORMAT_BF16_V1)
  int sink_per_shot;       // sink slots hold the first S frames of each shot
  float scale_log2;        // softmax_scale * log2(e)
  int n_wg;                // workgroups of the split schedule
  float *ws_o;             // partial g_v * acc [2 n_wg][256 rows][D]
  float2 *ws_ml;           // partial (m, l) [2 n_wg][256 rows]
  int *ws_cnt;             // pieces counted in per row block [n_wg], zero between launches
  int32_t q_shot[FP4KV_MAX_FRAMES];
};

hipError_t launch_cache_reset(const fp4kv_cache &c, hipStream_t s);
hipError_t launch_append(const AppendParams &p, hipStream_t s);
hipError_t launch_rerotate(const RerotParams &p, int window_slots, hipStream_t s);
hipError_t launch_rope(const RopeParams &p, hipStream_t s);
hipError_t launch_attention(const AttnParams &p, int head_dim, int out_f32, hipStream_t s);

// Attention workspace: FP4KV_MAX_WORKGROUPS counters, then per workgroup two
// partial (m, l) rows [2 n_wg][256] float2, then two partial outputs
// [2 n_wg][256][D] float.
constexpr size_t kAttnCounterBytes = FP4KV_MAX_WORKGROUPS * sizeof(int32_t);
constexpr int kAttnRows = 256;
inline size_t attn_workspace_bytes(int head_dim, long long n_wg) {
  return kAttnCounterBytes + (size_t)n_wg * 2 * kAttnRows * (8 + 4 * (size_t)head_dim);
}

}  // namespace fp4kv
