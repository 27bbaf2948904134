// Internal launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4kv.h"

namespace fp4kv {

// Number of partial maxima per tensor in the append workspace.
constexpr int kAmaxBlocks = 256;

// Workspace of the append and the window re-rotation: uint32 partial maxima
// (float32 bit patterns of max |x| per workgroup of the amax pass) of the
// appended K and V [2][kAmaxBlocks], then of each re-encoded window slot
// [FP4KV_MAX_SLOTS][kAmaxBlocks], then the slots' previous key tensor scales
// [FP4KV_MAX_SLOTS] (float32).
// The one-pass step prologue keeps its partial maxima [2][grid] in the
// re-encoding region and its grid barrier in the last 8448 bytes: for each
// of kBarGroups groups of workgroups a 256-byte line with the group's
// arrival count (word 0) and the phase its workgroups watch (word 32), then
// a line with the count of groups complete (word 0) and a sticky error word
// (word 32) set when a wait gave up.  The barrier words must be zero before
// the first use and every call leaves the counts at zero.
constexpr size_t kWsRrOffset = 2 * kAmaxBlocks;                        // in uint32
constexpr size_t kWsRrGOffset = kWsRrOffset + (size_t)FP4KV_MAX_SLOTS * kAmaxBlocks;
constexpr size_t kWsBarOffset = (kWsRrGOffset + FP4KV_MAX_SLOTS + 63) / 64 * 64;
constexpr int kBarGroups = 32, kBarLine = 64;   // a line is 64 words
constexpr int kWsBarPhase = 32, kWsBarWords = (kBarGroups + 1) * kBarLine;
constexpr int kWsBarTop = kBarGroups * kBarLine, kWsBarError = kWsBarTop + 32;
constexpr size_t kWsBytes = (kWsBarOffset + kWsBarWords) * sizeof(uint32_t);
// Largest grid of the one-pass prologue: its partial maxima fill the
// re-encoding region.
constexpr int kPrologueMaxGrid = (int)(FP4KV_MAX_SLOTS * kAmaxBlocks / 2);

struct AppendParams {
  const void *x[2];        // K, V inputs [n_frames*T][H][D]
  uint8_t *codes[2];
  uint8_t *scales[2];
  float *tscale[2];
  int32_t *slot_frame, *slot_shot;
  const float *tscale_in;  // device [2] or null
  uint32_t *ws_partial;    // [2][kAmaxBlocks]
  uint32_t *ws_bar;        // grid barrier words of the one-pass prologue
  int spin_limit;          // polls before a one-pass barrier wait gives up
  int H, D, T, stride, Tc, Tv, S, W, n_slots, frame0, n_frames;
  int in_bf16;
  int bf16_cache;          // FP4KV_FORMAT_BF16_V1: store bf16, no quantization
  int v_blocks;            // workgroups of the value pass in encode_kernel
  int k_blocks;            // workgroups of the key pass
  int amax_tensors;        // 2 when the amax pass covers the appended K and V, else 0
  // Keys stored rotated (FP4KV_FORMAT_NVFP4_ROT_V1).  half_rot > 0 with
  // rotate_keys: appended keys are turned by their frame's position first.
  // rr_slots > 0: the window slots whose frame f has rr_f_lo <= f < rr_f_hi
  // are decoded, turned back by table row rr_cs and encoded again in place.
  const float *cos_sin;    // rotary table [n_pos][half_rot][2]
  const float *rr_cs;      // table row of the window move (cos, sin) [half_rot]
  uint32_t *ws_rr;         // [FP4KV_MAX_SLOTS][kAmaxBlocks] partial maxima
  float *ws_rr_g;          // [FP4KV_MAX_SLOTS] key tensor scales before the call
  int half_rot, rotate_keys;
  int rr_slots, rr_f_lo, rr_f_hi, rr_blocks;
  int32_t shot[FP4KV_MAX_FRAMES];
  int32_t slot[FP4KV_MAX_FRAMES];   // cache slot of each frame (host-computed)
  int32_t pos[FP4KV_MAX_FRAMES];    // position of each frame (rotated keys)
};

struct RopeParams {
  const void *x;
  void *y;
  const float *cos_sin;
  long long n_tokens;
  int H, D, T, pos0, rot_dim, in_bf16, out_f32;
  int per_frame;                    // 1: token t turns by pos[t / T], else pos0 + t / T
  int32_t pos[FP4KV_MAX_FRAMES];
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
  int sat_half;            // rotary pairs of the query (rot_dim / 2 of the cache)
  float scale_log2;        // softmax_scale * log2(e)
  int n_wg;                // workgroups of the split schedule
  float *ws_o;             // partial g_v * acc [2 n_wg][256 rows][D]
  float2 *ws_ml;           // partial (m, l) [2 n_wg][256 rows]
  int *ws_cnt;             // pieces counted in per row block [n_wg], zero between launches
  int merge_pass;          // pieces of cut row blocks are combined by merge_kernel
  int32_t q_shot[FP4KV_MAX_FRAMES];
};

hipError_t launch_cache_reset(const fp4kv_cache &c, hipStream_t s);
hipError_t launch_append(const AppendParams &p, hipStream_t s);
// Device address and size of the library's own append workspace on the
// current device (resolved once per device).
hipError_t append_scratch(void **out, size_t *bytes);
hipError_t launch_rope(const RopeParams &p, hipStream_t s);
// The queries' rotation and the append of one chunk in two kernels: the
// rotation fused with the append's amax pass, then the encode.
hipError_t launch_rope_append(const RopeParams &rp, const AppendParams &ap, hipStream_t s);
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
