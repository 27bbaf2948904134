/*
 * fp4kv.h - C ABI of the MI355X (gfx950) FP4 KV-cache chunk-attention library.
 *
 * The library implements the per-step hot path of chunk-wise causal attention
 * for autoregressive long-video diffusion over a 4-bit NVFP4 KV cache, the
 * mechanisms the LongLive 2.0 pages name:
 *   - an NVFP4 KV cache written in place ("in-place quantized KV-cache
 *     updates"; hysenlabs.com, section "NVFP4, sequence parallel and the async
 *     decode path"; evermx.com, section "NVFP4 Quantization End-to-End");
 *   - KV-cache relative RoPE (aiany.app, section "What Sets It Apart";
 *     refft.com, question "How do KV-cache relative RoPE and TriAttention work
 *     together ...");
 *   - attention sinks plus a bounded window (heatdrop.ai, section "What it
 *     does") with multi-shot masking (evermx.com, section "Multi-Shot
 *     Generation");
 *   - FP4 KV dequantization fused into attention ("faster FP4 KV
 *     dequantization", hysenlabs.com, same section as above).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers owned by the caller;
 *     the library never allocates, frees or keeps them.  Pointers marked
 *     "host" are read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; no call synchronizes the device.
 *   - Every call validates its arguments on the host before enqueuing
 *     anything.  On a negative status nothing was enqueued, except
 *     FP4KV_EDEVICE, which reports a launch error returned by HIP.
 *   - Faults inside kernels (e.g. device pointers that are too small) are not
 *     detected by the library and surface at the caller's next
 *     synchronization.
 *   - Tensors are dense, row-major, with the innermost dimension last.
 *   - Inputs must be finite; NaN and Inf inputs give unspecified codes.
 *   - The library keeps no mutable global state, except the per-device
 *     workspace of fp4kv_quantize_append_noalloc, so calls on different
 *     streams and caches may run concurrently.  Calls that touch the same
 *     cache buffers must be ordered by the caller (same stream or events).
 */
#ifndef FP4KV_H
#define FP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define FP4KV_OK        0
#define FP4KV_EINVAL  (-1)  /* null pointer, or a value out of its range      */
#define FP4KV_ESHAPE  (-2)  /* sizes inconsistent with each other             */
#define FP4KV_EALIGN  (-3)  /* pointer not aligned as documented              */
#define FP4KV_EFORMAT (-4)  /* cache descriptor carries an unknown format tag */
#define FP4KV_EDEVICE (-5)  /* HIP reported an error when launching           */

/* ---------------------------------------------------------------- dtypes */
#define FP4KV_F32  0
#define FP4KV_BF16 1

/* Format tag of the NVFP4 cache layout described below. */
#define FP4KV_FORMAT_NVFP4_V1 0x3146564Eu
/* Baseline format: keys and values kept as bf16 (see fp4kv_cache). */
#define FP4KV_FORMAT_BF16_V1  0x36314642u
/* NVFP4 layout with keys stored after rotation (see fp4kv_cache). */
#define FP4KV_FORMAT_NVFP4_ROT_V1 0x3152564Eu

/* Limits.  Frames per call and cache slots are passed to kernels by value. */
#define FP4KV_MAX_FRAMES 64   /* frames per append or attention call      */
#define FP4KV_MAX_SLOTS  64   /* sink + window frames (S + W)             */
#define FP4KV_MAX_WORKGROUPS 4096 /* attention work split                  */

/*
 * fp4kv_cache - descriptor of one layer's NVFP4 KV cache.
 *
 * The cache holds S sink frames (the first S frames of the stream, never
 * evicted) and a ring of W window frames that includes the current chunk:
 * frame f lives in slot f if f < S, else in slot S + ((f - S) mod W).
 *
 * Per-shot sink (sink_per_shot = 1; the other reading of the multi-shot
 * attention sink, evermx.com "Multi-Shot Generation"): every shot re-anchors
 * the sink to its own first S frames.  Frame f of a shot starting at frame
 * fs lives in sink slot f - fs if f - fs < S (replacing the previous shot's
 * sink frame), else in slot S + ((f - S) mod W).  A sink slot is visible
 * only to queries of its own shot, at position f - fs; a cut inside a chunk
 * therefore leaves the earlier shot's frames of that chunk without a sink.
 * Queries of a frame qf are rotated by qf - fs if qf - fs < S, else by
 * S + (qf - ws), which need not be consecutive within a chunk (rotate each
 * frame with its own pos0).
 * Each cached frame keeps Tc = tokens_per_frame / token_stride tokens
 * (in-frame token t is kept iff t mod token_stride == 0).
 *
 * Keys are stored BEFORE rotary rotation; attention rotates them by their
 * cache-relative position at every step, so stored codes never change when
 * the window slides.
 *
 * Rotate-at-write format FP4KV_FORMAT_NVFP4_ROT_V1 (the other reading of
 * KV-cache relative RoPE; refft.com, question "How do KV-cache relative
 * RoPE and TriAttention work together ..."): the same buffers and layout,
 * but k_codes hold keys ALREADY rotated by their cache-relative position
 * (pos(f) below, for the window that ends after the append).  One call per
 * step, fp4kv_quantize_append_rotated, turns the surviving window keys and
 * appends the new keys rotated; the same result comes from
 * fp4kv_rerotate_window, fp4kv_rope_rel of the new keys (float32 output)
 * and fp4kv_quantize_append.  Attention then uses keys as stored.  Each
 * window key is re-encoded once per step it survives, which adds rounding
 * error.
 *
 * NVFP4 blocks are 16 consecutive elements along D for keys and values.
 * Keys are stored token-major; values are stored dimension-major so that the
 * attention kernel reads, for one dimension, consecutive tokens (the
 * reduction axis of P.V).  Tv = Tc rounded up to a multiple of 32; value
 * entries of padding tokens Tc..Tv-1 are written as zeros and never read
 * unmasked.
 *
 * Buffers (device, caller-owned, 16-byte aligned, contiguous):
 *   k_codes   uint8 [H][S+W][Tc][D/2]   E2M1 codes of a key row, two per byte:
 *                                       element 2j in the low nibble, sign in
 *                                       bit 3 of each nibble
 *   k_scales  uint8 [H][S+W][Tc][D/16]  E4M3 (OCP E4M3FN) scale per key block
 *   v_codes   uint8 [H][S+W][D][Tv/2]   E2M1 codes of one value dimension
 *                                       across tokens: token 2j low nibble,
 *                                       token 2j+1 high nibble
 *   v_scales  uint8 [H][S+W][D/16][Tv]  E4M3 scale of value block b of a token
 *   k_tscale, v_tscale  float [S+W]     FP32 tensor scale of the append that
 *                                       wrote the slot
 *   slot_frame          int32 [S+W]     frame in the slot, -1 when empty
 *   slot_shot           int32 [S+W]     shot id of that frame
 * A decoded element is sign * E2M1(code) * E4M3(scale) * tensor_scale.
 * These buffers are opaque bytes: never cast or convert them.
 *
 * Size limits (FP4KV_ESHAPE otherwise): one (head, slot) of the bf16 value
 * layout, 2 * D * Tv bytes, stays below 2^31 (Tv <= 8388576 at D = 128,
 * 16777184 at D = 64), and the whole cache holds at most 2^40 elements per
 * code array (H * (S + W) * Tc * D).
 *
 * Baseline format FP4KV_FORMAT_BF16_V1 (the unquantized cache that NVFP4 is
 * measured against; same ring, slots and attention): k_codes holds bf16
 * [H][S+W][Tc][D], v_codes bf16 [H][S+W][D][Tv] (padding tokens zero),
 * k_scales and v_scales are not used (0 bytes, may be NULL), and the tensor
 * scales are written as 1.  The append rounds its inputs to bf16 (nearest
 * even) and ignores tscale_in.  Attention converts the bf16 values to f16
 * MFMA operands, so they must lie within the f16 range (|x| <= 65504);
 * values below 2^-14 lose precision as f16 subnormals.
 */
typedef struct fp4kv_cache {
  uint32_t format_tag;        /* FP4KV_FORMAT_NVFP4_V1 (or _BF16_V1)          */
  int32_t  n_heads;           /* H >= 1                                      */
  int32_t  head_dim;          /* D: 64 or 128                                */
  int32_t  tokens_per_frame;  /* T >= 1                                      */
  int32_t  token_stride;      /* 1 or 2; T % token_stride == 0               */
  int32_t  chunk_frames;      /* C >= 1: frames per chunk (block-causal unit) */
  int32_t  sink_frames;       /* S >= 0                                      */
  int32_t  window_frames;     /* W >= C; S + W <= FP4KV_MAX_SLOTS            */
  int32_t  rot_dim;           /* even, 0 <= rot_dim <= D: rotated leading dims */
  int32_t  sink_per_shot;     /* 0: stream sink; 1: per-shot sink (see below)  */
  uint8_t *k_codes, *v_codes;
  uint8_t *k_scales, *v_scales;
  float   *k_tscale, *v_tscale;
  int32_t *slot_frame, *slot_shot;
} fp4kv_cache;

/* Human-readable text for a status code (static storage). */
const char *fp4kv_strerror(int status);

/* Library ABI version (increments when any signature or layout changes). */
int fp4kv_abi_version(void);

/*
 * fp4kv_cache_nbytes - byte sizes of the cache buffers (host only, no GPU).
 * out[0] = k_codes, out[1] = v_codes, out[2] = k_scales, out[3] = v_scales,
 * out[4] = each of k_tscale / v_tscale, out[5] = each of slot_frame /
 * slot_shot.  Pointer fields of `c` are not read.
 */
int fp4kv_cache_nbytes(const fp4kv_cache *c, size_t out[6]);

/*
 * fp4kv_cache_reset - mark every slot empty: slot_frame := -1,
 * slot_shot := 0, k_tscale = v_tscale := 1.  Codes and scales are left as
 * they are (an empty slot is never read).  Uses a fill kernel, so it may be
 * captured in a HIP graph.
 */
int fp4kv_cache_reset(const fp4kv_cache *c, void *stream);

/* Bytes of device workspace fp4kv_quantize_append and fp4kv_rope_append
 * need (constant, 76,288). */
size_t fp4kv_append_workspace_bytes(void);

/*
 * fp4kv_quantize_append - NVFP4-encode a chunk of new keys and values and
 * write it in place into the cache slots of frames frame0 .. frame0+n-1
 * ("in-place quantized KV-cache updates"; hysenlabs.com, section "NVFP4,
 * sequence parallel and the async decode path").
 *
 *   k, v        device, [n_frames * T][H][D] of in_dtype (FP4KV_F32 or
 *               FP4KV_BF16), 16-byte aligned.  Only kept tokens are read.
 *   frame0      >= 0, first frame of the chunk.
 *   n_frames    1 .. FP4KV_MAX_FRAMES, frames that land in distinct slots:
 *               a chunk (a partial last chunk is allowed), or a bulk
 *               re-append of cached frames (KV-recache: e.g. the sink frames
 *               0..S-1 in one call, the window frames in another), which
 *               share one tensor scale per call.
 *   frame_shot  host [n_frames]: shot id of each frame (written to slot_shot).
 *   frame_shot_start  host [n_frames]: first frame of each frame's shot
 *               (0 <= start <= frame), used when sink_per_shot = 1 (it picks
 *               the slot); may be NULL otherwise.
 *   tscale_in   device float[2] = {g_k, g_v} to use as tensor scales (finite,
 *               > 0), or NULL to compute g = amax / 2688 over the kept tokens
 *               of each of K and V (g = 1 when amax = 0).
 *   workspace   device, fp4kv_append_workspace_bytes() bytes, 16-byte
 *               aligned.  It holds the partial maxima of K and V and, for
 *               bf16 inputs with computed tensor scales, the grid barrier of
 *               the one-pass kernel in its last 8448 bytes, which must hold
 *               zeros before the first call that uses the workspace (every
 *               call leaves them so; the rest needs no initialization).
 *               Calls that overlap in time must use different workspaces.
 *
 * Kernels: bf16 inputs with computed tensor scales (NVFP4 format, nothing
 * stored rotated) take one kernel that reads K and V once, as in
 * fp4kv_rope_append; float32 inputs, caller tensor scales, the other
 * formats and chunks too large for that kernel's grid take two (partial
 * maxima, then the encode).
 *
 * Encoding, per 16-element block b along D of one (token, head) row, all in
 * IEEE float32 with round-to-nearest-even:
 *   d = 6 * g;  s8 = E4M3_satfinite(a_b / d)  (a_b = max |x| of the block);
 *   S = value(s8) * g;  r = 1 / S;  code = signbit(x) << 3 | E2M1_sat(|x| * r),
 *   with magnitude 0 when value(s8) = 0 or x = 0.
 * Re-appending the same frames with the same data rewrites identical bytes.
 * Slots of other frames are untouched.
 */
int fp4kv_quantize_append(const fp4kv_cache *c, const void *k, const void *v,
                          int in_dtype, int32_t frame0, int32_t n_frames,
                          const int32_t *frame_shot, const int32_t *frame_shot_start,
                          const float *tscale_in, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * fp4kv_quantize_append_noalloc - fp4kv_quantize_append without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, encoding, results and errors are those of
 * fp4kv_quantize_append; the workspace is a fixed array of
 * fp4kv_append_workspace_bytes() bytes that the library keeps in device
 * memory, one per device, for the life of the process (resolved on the first
 * call on each device).  The call allocates nothing.  All calls on one device
 * share that array: calls that overlap in time on one device race and must
 * be ordered by the caller (same stream or events).  The array is zero when
 * the library is loaded, which the one-pass kernel's barrier words need, and
 * every call leaves those words at zero counts.  No input size changes the
 * workspace it needs.  FP4KV_EDEVICE if the array's device address cannot
 * be obtained.
 */
int fp4kv_quantize_append_noalloc(const fp4kv_cache *c, const void *k, const void *v,
                                  int in_dtype, int32_t frame0, int32_t n_frames,
                                  const int32_t *frame_shot, const int32_t *frame_shot_start,
                                  const float *tscale_in, void *stream);

/*
 * fp4kv_quantize_append_rotated - the cache update of a
 * FP4KV_FORMAT_NVFP4_ROT_V1 cache in one call (two kernels): the window
 * move of fp4kv_rerotate_window(c, f1_prev, f1), then the append of
 * fp4kv_quantize_append with each key turned first by its frame's position
 * at the window ending at f1 (pair (2i, 2i+1), i < rot_dim/2:
 * (a, b) -> (fl(fl(a c) - fl(b s)), fl(fl(a s) + fl(b c))), float32, from
 * the float32 value of the input); the key tensor scale is taken over the
 * turned keys.  Arguments as in fp4kv_quantize_append, plus:
 *   f1_prev    window end the stored rotations belong to (normally frame0);
 *   f1         window end after the call (normally frame0 + n_frames);
 *              0 <= f1_prev <= f1, frame0 + n_frames <= f1.  Every frame
 *              must be a sink frame or lie in the window [ws(f1), f1).
 *   cos_sin    device table (fp4kv_rope_table, cache->rot_dim) with n_pos
 *              rows, more than any position and the window move; may be
 *              NULL when rot_dim = 0.
 * When the window start moves, the appended frames must all be >= f1_prev
 * (the re-encoded frames and the written frames are then distinct).
 * Errors: FP4KV_EINVAL for a cache of another format.
 */
int fp4kv_quantize_append_rotated(const fp4kv_cache *c, const void *k, const void *v,
                                  int in_dtype, int32_t frame0, int32_t n_frames,
                                  const int32_t *frame_shot, const int32_t *frame_shot_start,
                                  const float *tscale_in, int32_t f1_prev, int32_t f1,
                                  const float *cos_sin, int32_t n_pos, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * fp4kv_rerotate_window - move the stored key rotations of a
 * FP4KV_FORMAT_NVFP4_ROT_V1 cache from the window ending at frame f1_from
 * to the one ending at f1_to (KV-cache relative RoPE, rotate-at-write
 * reading; refft.com, question "How do KV-cache relative RoPE and
 * TriAttention work together ...").
 *
 * With ws(f1) = max(S, f1 - W) and delta = ws(f1_to) - ws(f1_from), every
 * window slot (slot >= S) whose frame f has ws(f1_to) <= f < f1_from is
 * turned by -delta: each key element is decoded as
 * sign * fl(fl(E2M1 * E4M3) * g), pair (2i, 2i+1), i < rot_dim/2, becomes
 * (fl(fl(a c) + fl(b s)), fl(fl(b c) - fl(a s))) with (c, s) = cos_sin[delta][i]
 * (float32, no fused multiply-add), and the slot's keys are encoded again
 * as in fp4kv_quantize_append with a new tensor scale amax / 2688 over the
 * slot (all heads).  Sink slots, values and slot metadata are untouched.
 * Nothing is enqueued when delta = 0 or no window frame survives.
 *   f1_from     0 <= f1_from <= f1_to: the window end the stored rotations
 *               belong to (the end of the previous append).
 *   cos_sin     device table from fp4kv_rope_table (cache->rot_dim) with
 *               n_pos > delta rows; may be NULL when rot_dim = 0.
 *   workspace   device, fp4kv_append_workspace_bytes() bytes, 16-byte
 *               aligned (partial maxima between the call's two kernels).
 * Errors: FP4KV_EINVAL for a cache of another format.
 */
int fp4kv_rerotate_window(const fp4kv_cache *c, int32_t f1_from, int32_t f1_to,
                          const float *cos_sin, int32_t n_pos, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * fp4kv_rope_table - fill a rotary table on the host (no GPU):
 *   cos_sin[p][i][0] = cos(p * base^(-2i/rot_dim)),
 *   cos_sin[p][i][1] = sin(p * base^(-2i/rot_dim)),
 * for p < n_pos, i < rot_dim/2, computed in double and rounded to float.
 * cos_sin is host memory of n_pos * rot_dim * sizeof(float) bytes; copy it
 * to the device for the calls below.
 */
int fp4kv_rope_table(float *cos_sin, int32_t n_pos, int32_t rot_dim, double base);

/*
 * fp4kv_rope_rel - rotate a [n_tokens][H][D] tensor by cache-relative frame
 * positions (relative RoPE: refft.com, question "How do KV-cache relative
 * RoPE and TriAttention work together ..."; fused RoPE: hysenlabs.com,
 * section "NVFP4, sequence parallel and the async decode path").
 *
 * Token t belongs to frame t / T and is rotated by position pos0 + t / T:
 * each pair (2i, 2i+1), i < rot_dim/2, turns by cos_sin[pos][i], i.e.
 * (a, b) -> (fl(fl(a c) - fl(b s)), fl(fl(a s) + fl(b c))): float32, each
 * product rounded before the sum, no fused multiply-add.  Dimensions past
 * rot_dim are copied.  A bf16 output is rounded to nearest even.
 *   x         device, in_dtype (FP4KV_F32 or FP4KV_BF16), 16-byte aligned.
 *   y         device, out_dtype (FP4KV_F32 or FP4KV_BF16), same shape; may
 *             alias x when in_dtype == out_dtype.
 *   cos_sin   device table from fp4kv_rope_table with n_pos rows;
 *             pos0 + (n_tokens - 1) / T must be < n_pos.  With rot_dim = 0
 *             (a copy) the table is not read and may be NULL.
 * The attention kernel takes float32 rotated queries (bf16 is accepted but
 * rounds the queries once more).
 */
int fp4kv_rope_rel(const void *x, int in_dtype, void *y, int out_dtype, int64_t n_tokens,
                   int32_t n_heads, int32_t head_dim, int32_t tokens_per_frame,
                   int32_t pos0, int32_t rot_dim, const float *cos_sin,
                   int32_t n_pos, void *stream);

/*
 * fp4kv_frame_position - cache-relative position of frame `frame` at the
 * step whose frames end at f1 (KV-cache relative RoPE: refft.com, question
 * "How do KV-cache relative RoPE and TriAttention work together ..."),
 * host only.  With ws = max(S, f1 - W): a sink frame keeps its index from the
 * sink's anchor (frame 0; with sink_per_shot = 1, shot_start, the first frame
 * of its shot: position frame - shot_start when that is below S); a window
 * frame ws <= frame < f1 is at S + (frame - ws).  shot_start is read only
 * when sink_per_shot = 1.  Returns the position (>= 0), or FP4KV_EINVAL for
 * a frame that is neither (or outside [0, f1)); descriptor errors as in
 * fp4kv_cache_nbytes.  Pointer fields of `c` are not read.
 */
int fp4kv_frame_position(const fp4kv_cache *c, int32_t frame, int32_t f1, int32_t shot_start);

/*
 * fp4kv_rope_rel_frames - fp4kv_rope_rel of one chunk's tensor
 * [n_frames * T][H][D] (T, H, D and rot_dim from the cache descriptor) with
 * the positions computed by the library: token t of frame frame0 + j turns by
 * fp4kv_frame_position(c, frame0 + j, frame0 + n_frames, frame_shot_start[j]),
 * so frames need not have consecutive positions (per-shot sinks).  Same
 * arithmetic, dtypes, alignment and aliasing rules as fp4kv_rope_rel.
 *   frame_shot_start  host [n_frames], required when sink_per_shot = 1,
 *               else may be NULL.
 *   cos_sin     device table (fp4kv_rope_table, cache->rot_dim) with n_pos
 *               rows, more than any position; NULL allowed when rot_dim = 0.
 * Errors: FP4KV_EINVAL when a frame is neither a sink frame nor in the
 * window ending at frame0 + n_frames; FP4KV_ESHAPE when a position is past
 * the table.
 */
int fp4kv_rope_rel_frames(const fp4kv_cache *c, const void *x, int in_dtype, void *y,
                          int out_dtype, int32_t frame0, int32_t n_frames,
                          const int32_t *frame_shot_start, const float *cos_sin, int32_t n_pos,
                          void *stream);

/*
 * fp4kv_rope_append - the two codec steps of one chunk in one call: the
 * rotation of the chunk's queries (fp4kv_rope_rel_frames of q into q_rot)
 * and the append of its keys and values (fp4kv_quantize_append with
 * tscale_in = NULL) ("fused RoPE" and "in-place quantized KV-cache
 * updates", hysenlabs.com, section "NVFP4, sequence parallel and the async
 * decode path").  Results are bit for bit those of the two separate calls.
 *   - bf16 keys and values: one kernel over a grid that the device holds
 *     at once.  Every thread reads 4 tokens of one 16-element block of K or
 *     V once and keeps them in registers; the workgroups publish partial
 *     maxima, meet at a grid barrier kept in the workspace (rotating the
 *     queries while they wait), then encode what they hold.  When the
 *     chunk has more such items than that grid has threads, the two-kernel
 *     form below runs instead.
 *   - float32 keys and values: two kernels, the first taking the partial
 *     maxima of K and V and rotating part of the queries, the second
 *     encoding K and V and rotating the rest.
 * Arguments as in those calls; the cache must have format
 * FP4KV_FORMAT_NVFP4_V1 (FP4KV_EINVAL otherwise).  q_rot must not be k or v
 * (q_rot may be q when the dtypes match).
 *   workspace   as for fp4kv_quantize_append (its last 8448 bytes, the
 *               grid barrier, hold zeros before the first use).  If part of
 *               the one-pass grid cannot start (other work on the device,
 *               for instance another one-pass call on a concurrent stream),
 *               a workgroup gives up its wait after about 10^6 polls and
 *               takes the maxima of K and V over all their elements itself:
 *               the bytes are the same, the call only slower.  The 32-bit
 *               word at byte offset fp4kv_append_workspace_bytes() - 128 is
 *               then set to 1 (the library never clears it).  The
 *               environment variable FP4KV_BARRIER_SPINS (a number of
 *               polls, read on every call) lowers the limit, for tests.  The
 *               same holds for fp4kv_quantize_append and its no-alloc
 *               variant.
 */
int fp4kv_rope_append(const fp4kv_cache *c, const void *q, int q_dtype, void *q_rot,
                      int q_rot_dtype, const void *k, const void *v, int kv_dtype, int32_t frame0,
                      int32_t n_frames, const int32_t *frame_shot, const int32_t *frame_shot_start,
                      const float *cos_sin, int32_t n_pos, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * fp4kv_attention_chunk - attention of the query frames
 * q_frame0 .. q_frame0+n_q_frames-1 over the NVFP4 cache, with FP4
 * dequantization fused into the attention loop.
 *
 * With f1 = q_frame0 + n_q_frames and ws = max(S, f1 - W), a cached frame kf
 * is visible to query frame qf iff
 *     0 <= kf < f1,  (kf < S or kf >= ws)                       (sink + window)
 *     kf / C <= qf / C                                          (block-causal)
 *     kf < S or slot_shot(kf) == q_shot[qf - q_frame0]          (multi-shot)
 * The multi-shot rule follows evermx.com, section "Multi-Shot Generation";
 * the sink and window follow heatdrop.ai, section "What it does".
 * Cache-relative position: pos(f) = f if f < S else S + (f - ws), for keys
 * and queries alike.  Scores are softmax_scale * (R(pos(qf)) q) . (R(pos(kf)) k)
 * with k the decoded (pre-rotation) key; for FP4KV_FORMAT_NVFP4_ROT_V1 the
 * stored key is already R(pos(kf)) k and is used as decoded.  The output of
 * a query row is the softmax-weighted sum of the decoded values.
 *
 * Arithmetic: MFMA with f16 operands and float32 accumulation.  Decoded keys
 * and values are exact in f16 (tensor scales are applied in float32); the
 * queries are carried as an f16 high part plus an f16 low part; softmax
 * weights are rounded to f16.  Queries must be below 2^15 in magnitude.
 *
 *   q_rot   device [n_q_frames * T][H][D] of q_dtype (FP4KV_F32 or
 *           FP4KV_BF16): queries ALREADY rotated by their cache-relative
 *           positions (fp4kv_rope_rel with pos0 = pos(q_frame0)),
 *           16-byte aligned.
 *   o       device [n_q_frames * T][H][D] of out_dtype (FP4KV_F32 or
 *           FP4KV_BF16), 16-byte aligned, must not alias q_rot.
 *   q_shot  host [n_q_frames]: shot id of each query frame.
 *   cos_sin device rotary table with n_pos >= S + W rows (fp4kv_rope_table,
 *           cache->rot_dim); not read for FP4KV_FORMAT_NVFP4_ROT_V1 (keys
 *           are stored rotated), where it may be NULL.
 * Rows with no visible key are written as zeros.
 *
 * Work split: the key tiles of all (256-row block, head) pairs are cut into
 * one contiguous range per workgroup.  A row block shared by two or more
 * ranges is merged from partial results (log-sum-exp combine, in a fixed
 * order, so repeated calls give identical bytes) kept in the workspace: by
 * the workgroup that completes the row block, or, when there are at least
 * 3 workgroups per row block, by a second kernel enqueued on the same stream
 * right after the first.
 *   n_workgroups  0: one workgroup per compute unit of the current device
 *                 (each range at least 4 key tiles); n > 0: n workgroups
 *                 (at most FP4KV_MAX_WORKGROUPS).  With workspace == NULL
 *                 the argument is ignored and every row block gets its own
 *                 workgroup (no split, no workspace).
 *   workspace     device, at least fp4kv_attention_workspace_bytes(D, n)
 *                 bytes for the n workgroups used, 16-byte aligned, or NULL.
 *                 It must be zero-filled once before its first use; every
 *                 call leaves it ready for the next one.  Calls that overlap
 *                 in time must use different workspaces.
 * Errors: FP4KV_ESHAPE when the workspace is too small for the workgroups.
 */
int fp4kv_attention_chunk(const fp4kv_cache *c, const void *q_rot, int q_dtype, void *o,
                          int out_dtype, int32_t q_frame0, int32_t n_q_frames,
                          const int32_t *q_shot, const float *cos_sin,
                          int32_t n_pos, float softmax_scale, int32_t n_workgroups,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of attention workspace for n_workgroups workgroups (1 ..
 * FP4KV_MAX_WORKGROUPS) at head dimension head_dim (64 or 128): per
 * workgroup two partial results of 256 rows (head_dim floats plus a (max,
 * sum) pair each), plus FP4KV_MAX_WORKGROUPS counters.  0 for invalid
 * arguments.  About 68 MB for 256 workgroups at head_dim 128.
 */
size_t fp4kv_attention_workspace_bytes(int32_t head_dim, int32_t n_workgroups);

#ifdef __cplusplus
}
#endif

#endif /* FP4KV_H */
