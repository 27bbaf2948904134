// C ABI: host-side validation, then launches on the caller's stream.
// Every check runs before anything is enqueued; see include/fp4kv.h.
#include <math.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "fp4kv.h"
#include "internal.hpp"

#include <algorithm>

using namespace fp4kv;

namespace {

constexpr int kAbiVersion = 6;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Value rows hold Tc tokens padded to a multiple of 32.
int padded_tokens(const fp4kv_cache *c) {
  const int tc = c->tokens_per_frame / c->token_stride;
  return (tc + 31) / 32 * 32;
}

// Shape checks of a cache descriptor (no pointer reads).
int check_shape(const fp4kv_cache *c) {
  if (!c) return FP4KV_EINVAL;
  if (c->format_tag != FP4KV_FORMAT_NVFP4_V1 && c->format_tag != FP4KV_FORMAT_BF16_V1 &&
      c->format_tag != FP4KV_FORMAT_NVFP4_ROT_V1)
    return FP4KV_EFORMAT;
  if (c->n_heads < 1 || c->tokens_per_frame < 1 || c->chunk_frames < 1 || c->sink_frames < 0)
    return FP4KV_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return FP4KV_ESHAPE;
  if (c->token_stride != 1 && c->token_stride != 2) return FP4KV_EINVAL;
  if (c->tokens_per_frame % c->token_stride != 0) return FP4KV_ESHAPE;
  if (c->window_frames < c->chunk_frames) return FP4KV_ESHAPE;
  if (c->sink_frames + c->window_frames > FP4KV_MAX_SLOTS) return FP4KV_ESHAPE;
  if (c->rot_dim < 0 || c->rot_dim > c->head_dim || (c->rot_dim & 1)) return FP4KV_EINVAL;
  if (c->sink_per_shot != 0 && c->sink_per_shot != 1) return FP4KV_EINVAL;
  // One (head, slot) of the largest layout (bf16 values, D x Tv) stays below
  // 2 GiB: the kernels address inside a slot with 32-bit offsets and sizes.
  const long long tv = ((long long)(c->tokens_per_frame / c->token_stride) + 31) / 32 * 32;
  if (2ll * c->head_dim * tv >= (1ll << 31)) return FP4KV_ESHAPE;
  const long long rows = (long long)c->n_heads * (c->sink_frames + c->window_frames) *
                         (c->tokens_per_frame / c->token_stride);
  if (rows * c->head_dim > (1ll << 40)) return FP4KV_ESHAPE;
  return FP4KV_OK;
}

bool is_bf16(const fp4kv_cache *c) { return c->format_tag == FP4KV_FORMAT_BF16_V1; }

// Keys stored already rotated by their cache-relative position.
bool keys_rotated(const fp4kv_cache *c) { return c->format_tag == FP4KV_FORMAT_NVFP4_ROT_V1; }

int window_start(const fp4kv_cache *c, long long f1) {
  return (int)std::max<long long>(c->sink_frames, f1 - c->window_frames);
}

int check_buffers(const fp4kv_cache *c) {
  const void *ptrs[] = {c->k_codes, c->v_codes, c->k_tscale, c->v_tscale,
                        c->slot_frame, c->slot_shot, c->k_scales, c->v_scales};
  const int n = is_bf16(c) ? 6 : 8;   // the bf16 format has no scale buffers
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return FP4KV_EINVAL;
    if (!aligned16(ptrs[i])) return FP4KV_EALIGN;
  }
  return FP4KV_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? FP4KV_OK : FP4KV_EDEVICE; }

// Workspace fields of the codec's parameters.
void set_append_ws(AppendParams &p, void *workspace) {
  p.ws_partial = (uint32_t *)workspace;
  p.ws_bar = (uint32_t *)workspace + kWsBarOffset;
  p.ws_rr = (uint32_t *)workspace + kWsRrOffset;
  p.ws_rr_g = (float *)((uint32_t *)workspace + kWsRrGOffset);
}

// Caller workspace of an append: present, large enough, aligned.
int check_append_ws(const void *workspace, size_t workspace_bytes) {
  if (!workspace) return FP4KV_EINVAL;
  if (workspace_bytes < kWsBytes) return FP4KV_ESHAPE;
  if (!aligned16(workspace)) return FP4KV_EALIGN;
  return FP4KV_OK;
}

// Cache fields of the codec's parameters; no frames, no window move.
void fill_append(AppendParams &p, const fp4kv_cache *c, void *workspace) {
  memset(&p, 0, sizeof(p));
  p.codes[0] = c->k_codes;
  p.codes[1] = c->v_codes;
  p.scales[0] = c->k_scales;
  p.scales[1] = c->v_scales;
  p.tscale[0] = c->k_tscale;
  p.tscale[1] = c->v_tscale;
  p.slot_frame = c->slot_frame;
  p.slot_shot = c->slot_shot;
  set_append_ws(p, workspace);
  p.H = c->n_heads;
  p.D = c->head_dim;
  p.T = c->tokens_per_frame;
  p.stride = c->token_stride;
  p.Tc = c->tokens_per_frame / c->token_stride;
  p.Tv = padded_tokens(c);
  p.S = c->sink_frames;
  p.W = c->window_frames;
  p.n_slots = c->sink_frames + c->window_frames;
  p.half_rot = c->rot_dim / 2;
  p.bf16_cache = is_bf16(c);
}

// Validation and parameters shared by the appends (nothing enqueued).
// The workspace is checked and set by the caller (set_append_ws).
int prepare_append(AppendParams &p, const fp4kv_cache *c, const void *k, const void *v,
                   int in_dtype, int32_t frame0, int32_t n_frames, const int32_t *frame_shot,
                   const int32_t *frame_shot_start, const float *tscale_in) {
  int st = check_shape(c);
  if (st) return st;
  if ((st = check_buffers(c))) return st;
  if (!k || !v || !frame_shot) return FP4KV_EINVAL;
  if (in_dtype != FP4KV_F32 && in_dtype != FP4KV_BF16) return FP4KV_EINVAL;
  if (frame0 < 0 || n_frames < 1 || n_frames > FP4KV_MAX_FRAMES) return FP4KV_EINVAL;
  if (c->sink_per_shot && !frame_shot_start) return FP4KV_EINVAL;
  int32_t slots[FP4KV_MAX_FRAMES];
  {  // the frames must land in distinct slots (a chunk, or a bulk re-append)
    uint64_t used = 0;
    const int S = c->sink_frames, W = c->window_frames;
    for (int j = 0; j < n_frames; ++j) {
      const long long f = (long long)frame0 + j;
      long long rel = f;   // index from the sink's anchor frame
      if (c->sink_per_shot) {
        if (frame_shot_start[j] < 0 || frame_shot_start[j] > f) return FP4KV_EINVAL;
        rel = f - frame_shot_start[j];
      }
      const int slot = rel < S ? (int)rel : S + (int)((f - S) % W);
      if (used >> slot & 1ull) return FP4KV_EINVAL;
      used |= 1ull << slot;
      slots[j] = slot;
    }
  }
  if ((long long)frame0 + n_frames > (1ll << 30)) return FP4KV_EINVAL;
  if (!aligned16(k) || !aligned16(v)) return FP4KV_EALIGN;
  if (tscale_in && ((uintptr_t)tscale_in & 3u)) return FP4KV_EALIGN;

  fill_append(p, c, nullptr);
  p.x[0] = k;
  p.x[1] = v;
  p.tscale_in = tscale_in;
  p.frame0 = frame0;
  p.n_frames = n_frames;
  p.in_bf16 = in_dtype == FP4KV_BF16;
  for (int j = 0; j < n_frames; ++j) {
    p.shot[j] = frame_shot[j];
    p.slot[j] = slots[j];
  }
  return FP4KV_OK;
}

// Window move f1_from -> f1_to of a cache that stores keys rotated: the
// window slots to re-encode (rr_slots = 0 when nothing moves or survives).
int prepare_window_move(AppendParams &p, const fp4kv_cache *c, int32_t f1_from, int32_t f1_to,
                        const float *cos_sin, int32_t n_pos) {
  if (c->rot_dim > 0 && !cos_sin) return FP4KV_EINVAL;
  if ((uintptr_t)cos_sin & 7u) return FP4KV_EALIGN;
  const int ws0 = window_start(c, f1_from), ws1 = window_start(c, f1_to);
  const int delta = ws1 - ws0;
  p.rr_slots = 0;
  if (delta == 0 || ws1 >= f1_from) return FP4KV_OK;
  if (c->rot_dim > 0 && delta >= n_pos) return FP4KV_ESHAPE;
  const long long units = (long long)c->n_heads * (c->tokens_per_frame / c->token_stride) *
                          (c->head_dim / 16);   // (key row, block) pairs of one slot
  if (units >= (1ll << 31)) return FP4KV_ESHAPE;
  p.rr_cs = c->rot_dim > 0 ? cos_sin + (size_t)delta * c->rot_dim : nullptr;
  p.rr_slots = c->window_frames;
  p.rr_f_lo = ws1;
  p.rr_f_hi = f1_from;
  return FP4KV_OK;
}

// Cache-relative position of frame f at the step whose frames end at f1:
// a sink frame keeps its index from the sink's anchor (frame 0, or with
// per-shot sinks its shot's first frame fs); a window frame is S + (f - ws)
// with ws = max(S, f1 - W).  -1 for a frame that is neither.
long long frame_pos(const fp4kv_cache *c, long long f, long long f1, long long fs) {
  const long long S = c->sink_frames;
  const long long rel = c->sink_per_shot ? f - fs : f;
  if (f < 0 || f >= f1 || rel < 0) return -1;
  if (rel < S) return rel;
  const long long ws = std::max<long long>(S, f1 - c->window_frames);
  return f < ws ? -1 : S + (f - ws);
}

// Rotation of the chunk frame0 .. frame0 + n_frames - 1 of a tensor
// [n_frames * T][H][D] by the frames' cache-relative positions at the window
// ending at f1 = frame0 + n_frames, positions computed here per frame.
int prepare_rope_frames(RopeParams &p, const fp4kv_cache *c, const void *x, int in_dtype, void *y,
                        int out_dtype, int32_t frame0, int32_t n_frames,
                        const int32_t *frame_shot_start, const float *cos_sin, int32_t n_pos) {
  if (!x || !y) return FP4KV_EINVAL;
  if (in_dtype != FP4KV_F32 && in_dtype != FP4KV_BF16) return FP4KV_EINVAL;
  if (out_dtype != FP4KV_F32 && out_dtype != FP4KV_BF16) return FP4KV_EINVAL;
  if (frame0 < 0 || n_frames < 1 || n_frames > FP4KV_MAX_FRAMES) return FP4KV_EINVAL;
  if ((long long)frame0 + n_frames > (1ll << 30)) return FP4KV_EINVAL;
  if (c->sink_per_shot && !frame_shot_start) return FP4KV_EINVAL;
  if (c->rot_dim > 0 && (!cos_sin || n_pos < 1)) return FP4KV_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)cos_sin & 7u)) return FP4KV_EALIGN;
  if (x == y && in_dtype != out_dtype) return FP4KV_EINVAL;
  memset(&p, 0, sizeof(p));
  const long long f1 = (long long)frame0 + n_frames;
  for (int j = 0; j < n_frames; ++j) {
    const long long f = (long long)frame0 + j;
    long long fs = 0;
    if (c->sink_per_shot) {
      fs = frame_shot_start[j];
      if (fs < 0 || fs > f) return FP4KV_EINVAL;
    }
    const long long pos = frame_pos(c, f, f1, fs);
    if (pos < 0) return FP4KV_EINVAL;            // a frame outside sink and window
    if (c->rot_dim > 0 && pos >= n_pos) return FP4KV_ESHAPE;
    p.pos[j] = (int32_t)pos;
  }
  p.x = x;
  p.y = y;
  p.out_f32 = out_dtype == FP4KV_F32;
  p.cos_sin = cos_sin;
  p.n_tokens = (long long)n_frames * c->tokens_per_frame;
  p.H = c->n_heads;
  p.D = c->head_dim;
  p.T = c->tokens_per_frame;
  p.rot_dim = c->rot_dim;
  p.in_bf16 = in_dtype == FP4KV_BF16;
  p.per_frame = 1;
  if (p.n_tokens * p.H * (long long)p.D > (1ll << 40)) return FP4KV_ESHAPE;
  return FP4KV_OK;
}

}  // namespace

extern "C" {

const char *fp4kv_strerror(int status) {
  switch (status) {
    case FP4KV_OK: return "ok";
    case FP4KV_EINVAL: return "invalid argument (null pointer or value out of range)";
    case FP4KV_ESHAPE: return "inconsistent shapes";
    case FP4KV_EALIGN: return "pointer not 16-byte aligned";
    case FP4KV_EFORMAT: return "cache descriptor has an unknown format tag";
    case FP4KV_EDEVICE: return "HIP launch error";
    default: return "unknown status";
  }
}

int fp4kv_abi_version(void) { return kAbiVersion; }

int fp4kv_cache_nbytes(const fp4kv_cache *c, size_t out[6]) {
  int st = check_shape(c);
  if (st) return st;
  if (!out) return FP4KV_EINVAL;
  const size_t slots = (size_t)(c->sink_frames + c->window_frames);
  const size_t tc = (size_t)(c->tokens_per_frame / c->token_stride);
  const size_t tv = (size_t)padded_tokens(c);
  const size_t hs = (size_t)c->n_heads * slots, d = (size_t)c->head_dim;
  if (is_bf16(c)) {
    out[0] = hs * tc * d * 2;
    out[1] = hs * d * tv * 2;
    out[2] = out[3] = 0;
  } else {
    out[0] = hs * tc * (d / 2);
    out[1] = hs * d * (tv / 2);
    out[2] = hs * tc * (d / 16);
    out[3] = hs * (d / 16) * tv;
  }
  out[4] = slots * sizeof(float);
  out[5] = slots * sizeof(int32_t);
  return FP4KV_OK;
}

int fp4kv_cache_reset(const fp4kv_cache *c, void *stream) {
  int st = check_shape(c);
  if (st) return st;
  if ((st = check_buffers(c))) return st;
  return from_hip(launch_cache_reset(*c, (hipStream_t)stream));
}

size_t fp4kv_append_workspace_bytes(void) { return kWsBytes; }

int fp4kv_quantize_append(const fp4kv_cache *c, const void *k, const void *v, int in_dtype,
                          int32_t frame0, int32_t n_frames, const int32_t *frame_shot,
                          const int32_t *frame_shot_start, const float *tscale_in,
                          void *workspace, size_t workspace_bytes, void *stream) {
  AppendParams p;
  int st = prepare_append(p, c, k, v, in_dtype, frame0, n_frames, frame_shot, frame_shot_start,
                          tscale_in);
  if (st) return st;
  if ((st = check_append_ws(workspace, workspace_bytes))) return st;
  set_append_ws(p, workspace);
  return from_hip(launch_append(p, (hipStream_t)stream));
}

int fp4kv_quantize_append_noalloc(const fp4kv_cache *c, const void *k, const void *v,
                                  int in_dtype, int32_t frame0, int32_t n_frames,
                                  const int32_t *frame_shot, const int32_t *frame_shot_start,
                                  const float *tscale_in, void *stream) {
  AppendParams p;
  int st = prepare_append(p, c, k, v, in_dtype, frame0, n_frames, frame_shot, frame_shot_start,
                          tscale_in);
  if (st) return st;
  void *ws = nullptr;
  size_t ws_bytes = 0;
  if (append_scratch(&ws, &ws_bytes) != hipSuccess) return FP4KV_EDEVICE;
  if ((st = check_append_ws(ws, ws_bytes))) return st;   // the array's fixed size
  set_append_ws(p, ws);
  return from_hip(launch_append(p, (hipStream_t)stream));
}

int fp4kv_quantize_append_rotated(const fp4kv_cache *c, const void *k, const void *v,
                                  int in_dtype, int32_t frame0, int32_t n_frames,
                                  const int32_t *frame_shot, const int32_t *frame_shot_start,
                                  const float *tscale_in, int32_t f1_prev, int32_t f1,
                                  const float *cos_sin, int32_t n_pos, void *workspace,
                                  size_t workspace_bytes, void *stream) {
  AppendParams p;
  int st = prepare_append(p, c, k, v, in_dtype, frame0, n_frames, frame_shot, frame_shot_start,
                          tscale_in);
  if (st) return st;
  if ((st = check_append_ws(workspace, workspace_bytes))) return st;
  set_append_ws(p, workspace);
  if (!keys_rotated(c)) return FP4KV_EINVAL;
  if (f1_prev < 0 || f1 < f1_prev || f1 > (1 << 30) || (long long)frame0 + n_frames > f1)
    return FP4KV_EINVAL;
  if ((st = prepare_window_move(p, c, f1_prev, f1, cos_sin, n_pos))) return st;
  // frames re-encoded by the move and frames written by the append must differ
  if (p.rr_slots > 0 && frame0 < f1_prev) return FP4KV_EINVAL;
  const int S = c->sink_frames, ws = window_start(c, f1);
  for (int j = 0; j < n_frames; ++j) {   // cache-relative position at the window ending at f1
    const int f = frame0 + j;
    const int rel = c->sink_per_shot ? f - frame_shot_start[j] : f;
    const int pos = rel < S ? rel : S + (f - ws);
    if (pos < 0) return FP4KV_EINVAL;    // neither a sink frame nor in the window
    if (c->rot_dim > 0 && pos >= n_pos) return FP4KV_ESHAPE;
    p.pos[j] = pos;
  }
  p.rotate_keys = 1;
  p.cos_sin = cos_sin;
  return from_hip(launch_append(p, (hipStream_t)stream));
}

int fp4kv_rerotate_window(const fp4kv_cache *c, int32_t f1_from, int32_t f1_to,
                          const float *cos_sin, int32_t n_pos, void *workspace,
                          size_t workspace_bytes, void *stream) {
  int st = check_shape(c);
  if (st) return st;
  if ((st = check_buffers(c))) return st;
  if (!keys_rotated(c)) return FP4KV_EINVAL;
  if (f1_from < 0 || f1_to < f1_from || f1_to > (1 << 30) || !workspace) return FP4KV_EINVAL;
  if (workspace_bytes < kWsBytes) return FP4KV_ESHAPE;
  if (!aligned16(workspace)) return FP4KV_EALIGN;
  AppendParams p;
  fill_append(p, c, workspace);
  if ((st = prepare_window_move(p, c, f1_from, f1_to, cos_sin, n_pos))) return st;
  if (p.rr_slots == 0) return FP4KV_OK;                // nothing survives a move
  return from_hip(launch_append(p, (hipStream_t)stream));
}

int fp4kv_rope_table(float *cos_sin, int32_t n_pos, int32_t rot_dim, double base) {
  if (!cos_sin || n_pos < 1 || rot_dim < 2 || (rot_dim & 1) || !(base > 1.0)) return FP4KV_EINVAL;
  const int half = rot_dim / 2;
  for (int p = 0; p < n_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double theta = pow(base, -2.0 * i / (double)rot_dim);
      const double phi = (double)p * theta;
      cos_sin[((size_t)p * half + i) * 2 + 0] = (float)cos(phi);
      cos_sin[((size_t)p * half + i) * 2 + 1] = (float)sin(phi);
    }
  return FP4KV_OK;
}

int fp4kv_rope_rel(const void *x, int in_dtype, void *y, int out_dtype, int64_t n_tokens,
                   int32_t n_heads, int32_t head_dim, int32_t tokens_per_frame, int32_t pos0,
                   int32_t rot_dim, const float *cos_sin, int32_t n_pos, void *stream) {
  if (!x || !y || (!cos_sin && rot_dim > 0)) return FP4KV_EINVAL;
  if (in_dtype != FP4KV_F32 && in_dtype != FP4KV_BF16) return FP4KV_EINVAL;
  if (out_dtype != FP4KV_F32 && out_dtype != FP4KV_BF16) return FP4KV_EINVAL;
  if (n_tokens < 0 || n_heads < 1 || tokens_per_frame < 1 || pos0 < 0 || n_pos < 1)
    return FP4KV_EINVAL;
  if (head_dim < 8 || head_dim % 8) return FP4KV_ESHAPE;
  if (rot_dim < 0 || rot_dim > head_dim || (rot_dim & 1)) return FP4KV_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)cos_sin & 7u)) return FP4KV_EALIGN;
  if (x == y && in_dtype != out_dtype) return FP4KV_EINVAL;
  if (n_tokens == 0) return FP4KV_OK;
  if (rot_dim > 0 && (long long)pos0 + (n_tokens - 1) / tokens_per_frame >= n_pos)
    return FP4KV_ESHAPE;   // rot_dim 0 reads no table
  if (n_tokens > (1ll << 40) || n_tokens * n_heads * (long long)head_dim > (1ll << 40))
    return FP4KV_ESHAPE;
  RopeParams p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.y = y;
  p.out_f32 = out_dtype == FP4KV_F32;
  p.cos_sin = cos_sin;
  p.n_tokens = n_tokens;
  p.H = n_heads;
  p.D = head_dim;
  p.T = tokens_per_frame;
  p.pos0 = pos0;
  p.rot_dim = rot_dim;
  p.in_bf16 = in_dtype == FP4KV_BF16;
  return from_hip(launch_rope(p, (hipStream_t)stream));
}

int fp4kv_frame_position(const fp4kv_cache *c, int32_t frame, int32_t f1, int32_t shot_start) {
  int st = check_shape(c);
  if (st) return st;
  if (frame < 0 || f1 > (1 << 30) || (c->sink_per_shot && (shot_start < 0 || shot_start > frame)))
    return FP4KV_EINVAL;
  const long long pos = frame_pos(c, frame, f1, c->sink_per_shot ? shot_start : 0);
  return pos < 0 ? FP4KV_EINVAL : (int)pos;
}

int fp4kv_rope_rel_frames(const fp4kv_cache *c, const void *x, int in_dtype, void *y,
                          int out_dtype, int32_t frame0, int32_t n_frames,
                          const int32_t *frame_shot_start, const float *cos_sin, int32_t n_pos,
                          void *stream) {
  int st = check_shape(c);
  if (st) return st;
  RopeParams p;
  if ((st = prepare_rope_frames(p, c, x, in_dtype, y, out_dtype, frame0, n_frames,
                                frame_shot_start, cos_sin, n_pos)))
    return st;
  return from_hip(launch_rope(p, (hipStream_t)stream));
}

int fp4kv_rope_append(const fp4kv_cache *c, const void *q, int q_dtype, void *q_rot,
                      int q_rot_dtype, const void *k, const void *v, int kv_dtype, int32_t frame0,
                      int32_t n_frames, const int32_t *frame_shot, const int32_t *frame_shot_start,
                      const float *cos_sin, int32_t n_pos, void *workspace,
                      size_t workspace_bytes, void *stream) {
  AppendParams ap;
  int st = prepare_append(ap, c, k, v, kv_dtype, frame0, n_frames, frame_shot, frame_shot_start,
                          nullptr);
  if (st) return st;
  if (c->format_tag != FP4KV_FORMAT_NVFP4_V1) return FP4KV_EINVAL;
  if ((st = check_append_ws(workspace, workspace_bytes))) return st;
  set_append_ws(ap, workspace);
  RopeParams rp;
  if ((st = prepare_rope_frames(rp, c, q, q_dtype, q_rot, q_rot_dtype, frame0, n_frames,
                                frame_shot_start, cos_sin, n_pos)))
    return st;
  if (q_rot == k || q_rot == v) return FP4KV_EINVAL;   // K and V are read by both kernels
  return from_hip(launch_rope_append(rp, ap, (hipStream_t)stream));
}

int fp4kv_attention_chunk(const fp4kv_cache *c, const void *q_rot, int q_dtype, void *o,
                          int out_dtype, int32_t q_frame0, int32_t n_q_frames,
                          const int32_t *q_shot, const float *cos_sin, int32_t n_pos,
                          float softmax_scale, int32_t n_workgroups, void *workspace,
                          size_t workspace_bytes, void *stream) {
  int st = check_shape(c);
  if (st) return st;
  if ((st = check_buffers(c))) return st;
  const bool rotated = keys_rotated(c);   // no key rotation, no table
  if (!q_rot || !o || !q_shot || (!cos_sin && !rotated)) return FP4KV_EINVAL;
  if (out_dtype != FP4KV_F32 && out_dtype != FP4KV_BF16) return FP4KV_EINVAL;
  if (q_dtype != FP4KV_F32 && q_dtype != FP4KV_BF16) return FP4KV_EINVAL;
  if (q_frame0 < 0 || n_q_frames < 1 || n_q_frames > FP4KV_MAX_FRAMES) return FP4KV_EINVAL;
  if ((long long)q_frame0 + n_q_frames > (1ll << 30)) return FP4KV_EINVAL;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return FP4KV_EINVAL;
  if (!rotated && n_pos < c->sink_frames + c->window_frames) return FP4KV_ESHAPE;
  if (!aligned16(q_rot) || !aligned16(o) || ((uintptr_t)cos_sin & 7u)) return FP4KV_EALIGN;
  if (q_rot == o) return FP4KV_EINVAL;
  const long long nq = (long long)n_q_frames * c->tokens_per_frame;
  if (nq > (1ll << 30) || nq * c->n_heads > (1ll << 31)) return FP4KV_ESHAPE;

  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q = q_rot;
  p.q_f32 = q_dtype == FP4KV_F32;
  p.bf16_cache = is_bf16(c);
  p.o = o;
  p.k_codes = c->k_codes;
  p.v_codes = c->v_codes;
  p.k_scales = c->k_scales;
  p.v_scales = c->v_scales;
  p.k_tscale = c->k_tscale;
  p.v_tscale = c->v_tscale;
  p.slot_frame = c->slot_frame;
  p.slot_shot = c->slot_shot;
  p.cos_sin = cos_sin;
  p.H = c->n_heads;
  p.T = c->tokens_per_frame;
  p.Tc = c->tokens_per_frame / c->token_stride;
  p.Tv = padded_tokens(c);
  p.C = c->chunk_frames;
  p.S = c->sink_frames;
  p.W = c->window_frames;
  p.n_slots = c->sink_frames + c->window_frames;
  p.rot_dim = rotated ? 0 : c->rot_dim;   // rot_dim 0: the kernel turns nothing
  p.q_frame0 = q_frame0;
  p.n_q_frames = n_q_frames;
  p.Nq = (int)nq;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.sink_per_shot = c->sink_per_shot;
  p.sat_half = c->rot_dim / 2;
  for (int j = 0; j < n_q_frames; ++j) p.q_shot[j] = q_shot[j];

  // Work split: equal ranges of the virtual key tiles (n_v per row block)
  // over n_wg workgroups; without a workspace, one row block per workgroup.
  const long long n_rb = (nq + kAttnRows - 1) / kAttnRows * c->n_heads;
  const long long n_v = (long long)p.n_slots * ((p.Tc + 63) / 64);
  long long n_wg = n_rb;
  if (workspace) {
    if (n_workgroups < 0 || n_workgroups > FP4KV_MAX_WORKGROUPS) return FP4KV_EINVAL;
    if (!aligned16(workspace)) return FP4KV_EALIGN;
    if (n_workgroups == 0) {
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return FP4KV_EDEVICE;
      n_wg = std::min<long long>(std::min(cus, FP4KV_MAX_WORKGROUPS),
                                 std::max<long long>(1, n_rb * n_v / 4));
    } else {
      n_wg = n_workgroups;
    }
    n_wg = std::min(n_wg, n_rb * n_v);   // no empty range
    // Many pieces per row block (at least 4 on average): combine them in a
    // second kernel spread over the row blocks' 32-row slices instead of in
    // the one workgroup that finishes a row block last.
    p.merge_pass = n_wg >= 3 * n_rb;
    if (workspace_bytes < attn_workspace_bytes(c->head_dim, n_wg)) return FP4KV_ESHAPE;
    uint8_t *ws = (uint8_t *)workspace;
    p.ws_cnt = (int32_t *)ws;
    p.ws_ml = (float2 *)(ws + kAttnCounterBytes);
    p.ws_o = (float *)(ws + kAttnCounterBytes + (size_t)n_wg * 2 * kAttnRows * sizeof(float2));
  }
  if (n_wg > (1ll << 30)) return FP4KV_ESHAPE;
  p.n_wg = (int)n_wg;
  return from_hip(launch_attention(p, c->head_dim, out_dtype == FP4KV_F32, (hipStream_t)stream));
}

size_t fp4kv_attention_workspace_bytes(int32_t head_dim, int32_t n_workgroups) {
  if ((head_dim != 64 && head_dim != 128) || n_workgroups < 1 ||
      n_workgroups > FP4KV_MAX_WORKGROUPS)
    return 0;
  return attn_workspace_bytes(head_dim, n_workgroups);
}

}  // extern "C"
