// Chunk attention over the NVFP4 KV cache with the FP4 dequantization fused
// into the attention loop ("faster FP4 KV dequantization", hysenlabs.com,
// "NVFP4, sequence parallel and the async decode path"), sink + window
// visibility (heatdrop.ai, "What it does"), block-causal chunks and shot
// masks (evermx.com, "Multi-Shot Generation"), and cache-relative RoPE
// (refft.com, question "How do KV-cache relative RoPE and TriAttention work
// together ...").
//
// Work layout (gfx950, wave64, MFMA 32x32x16 with f16 operands, f32 accum):
//   * a row block is 256 query rows of one head, held by one workgroup of 8
//     waves x 32 rows (one workgroup per CU, two waves per SIMD);
//   * the keys of all visible frames of a row block are walked as one
//     sequence of 64-key tiles, dequantized into LDS (2 K and 4 V buffers).
//     Dequantization is exact: E2M1 x E4M3 has at most 6 significant bits
//     and lies in [2^-10, 2688], so it fits f16; the hardware converts two
//     FP4 codes to f16 (scale 1) and one packed f16 multiply applies the
//     block scale;
//   * each wave computes S^T = K Q^T so that a lane owns one query row in
//     both the score and the output accumulators: the softmax row max and sum
//     stay inside a lane plus one exchange with the lane 32 away;
//   * O^T += V^T P^T, with P taken straight from the score registers and V
//     read dimension-major, as the cache stores it;
//   * ping-pong schedule: the waves form two groups with one wave of each
//     on every SIMD, and while one group issues MFMAs the other does the
//     softmax and dequantizes its half of a later tile;
//   * split schedule: the key tiles of all row blocks are cut into one
//     contiguous range per workgroup; a row block shared by two or more
//     ranges is finished by a log-sum-exp merge of the pieces, in the
//     workgroup that completes the row block or, when the row blocks are cut
//     into many pieces, in a second kernel (merge_kernel).
//
// Rotation: the cache holds keys before rotation.  Rotating q by pos(qf) and
// k by pos(kf) gives the same score as rotating q by pos(qf) - pos(kf), so
// each wave turns its rotated queries back by -pos(kf) once per key frame and
// the keys need no rotation.  The cos/sin rows of these turns are staged in
// LDS once per workgroup.
//
// Precision: the turned-back queries are split into an f16 high part and an
// f16 low part (two MFMAs on the same exact key operand), so scores carry
// about 22 bits; P is rounded to f16 and the row sum adds the same rounded
// weights, so a row dominated by one key returns that key's value exactly
// (under the lazy rescale the dominant weight is any value up to 2^8, not
// 1).  softmax_scale * log2(e) * g_k (the key
// tensor scale of the frame) multiplies the scores inside the exp2 argument;
// the value tensor scale is folded into the output accumulator when the frame
// changes.
#include "fp4kv_device.hpp"
#include "internal.hpp"

namespace fp4kv {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;               // two groups of 4, one wave of each per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;        // query rows per workgroup
constexpr int kBN = 64;                 // keys per tile
constexpr int kPad = 8;                 // f16 elements of padding per LDS row
constexpr int kXcds = 8;                // accelerator complex dies of MI355X
constexpr int kKBufs = 2, kVBufs = 4;   // dequantized K and V tiles in LDS

// Buffer resource (gfx9 format) over `bytes` bytes at `base`: loads at
// offsets past the end return zero instead of touching memory.
constexpr uint32_t kBufferWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache-policy operand of the buffer intrinsics: sc1, a device-coherent access.
constexpr int kSc1 = 16;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, (int)bytes,
                                           (int)kBufferWord3);
}

__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ uint32_t bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ f32x16 mfma32(const f16x8 &a, const f16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two E2M1 codes (byte `sel` of w) -> f16 values, scale 1 (exact).
template <int SEL>
__device__ __forceinline__ f16x2 fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// Two E4M3 codes (16-bit half `HI` of w) -> f16 values (exact).
template <bool HI>
__device__ __forceinline__ f16x2 fp8x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Lanes i and i + 32 hold two halves of one query row.  gfx950's
// v_permlane32_swap (a VALU exchange of the two 32-lane halves, no LDS trip)
// applied to (x, x) returns the low half's values in every lane and the high
// half's values in every lane; max and sum are symmetric in the two.
__device__ __forceinline__ float halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key (within a 32-key block) that row m of the S^T operand reads.  With
// this order the 8 consecutive score registers 8t'..8t'+7 of a lane hold 8
// consecutive keys, which is what the P^T operand of the PV product needs.
__device__ __forceinline__ int sigma(int m) {
  const int i = m >> 3, hh = (m >> 2) & 1, r = m & 3;
  return 16 * (i >> 1) + 8 * hh + 4 * (i & 1) + r;
}

// Physical LDS row of key k in a K tile: rows 8..15 of every 16 swap their
// halves, so the 8 lanes that read together (keys {0-3, 8-11} + 16j and
// {4-7, 12-15} + 16j under sigma) hit 8 different bank groups.
__device__ __forceinline__ int krow_phys(int k) { return k ^ (((k >> 3) & 1) << 2); }

template <int D>
struct Smem {
  uint16_t kh[kKBufs][kBN][D + kPad];   // dequantized K tiles, f16 bits
  uint16_t vt[kVBufs][D][kBN + kPad];   // dequantized V tiles, dimension-major
  float2 rot[FP4KV_MAX_SLOTS][D / 2];  // (cos, sin) of the turn into each listed frame
  int fl_slot[FP4KV_MAX_SLOTS];
  int fl_kf[FP4KV_MAX_SLOTS];
  int fl_pos[FP4KV_MAX_SLOTS];
  int fl_shot[FP4KV_MAX_SLOTS];
  float fl_gk[FP4KV_MAX_SLOTS];
  float fl_gv[FP4KV_MAX_SLOTS];
  int merge_last;       // this workgroup completes the current row block
};

// Packed codes and scales held by one thread between the load and the
// dequantization: one key's 32 elements, or 16 tokens of two value dimensions.
struct RawK {
  uint4 kc;        // 32 key elements (16 bytes)
  uint32_t ks;     // their two block scales (low 16 bits)
};
struct RawV {
  uint2 vc[2];     // 16 tokens of two value dimensions
  uint4 vs;        // the 16 tokens' scales of that value block
};

// Buffer loads over the (head, slot) ranges of the cache: keys past Tc fall
// outside the K range and read as zero, value tokens past Tv are sent out of
// range.  No branch, so the loads stay in flight until the codes are
// dequantized in the next phase.  lt is the thread's index in its group.
// bf16 baseline format: the same elements as bf16 (two 16-byte words per
// 16 elements).
struct RawKB {
  uint4 kc[4];     // 32 key elements
};
struct RawVB {
  uint4 v[4];      // 16 tokens of two value dimensions: v[2 r], v[2 r + 1] = dimension r
};
template <bool K, bool BF16KV>
struct RawOf {
  using type = RawV;
};
template <>
struct RawOf<true, false> {
  using type = RawK;
};
template <>
struct RawOf<false, true> {
  using type = RawVB;
};
template <>
struct RawOf<true, true> {
  using type = RawKB;
};

// Buffer resources over one (head, slot) range of the four cache arrays.
struct SlotRes {
  __amdgpu_buffer_rsrc_t kc, ks, vc, vs;
};
template <int D, bool BF16KV>
__device__ __forceinline__ SlotRes slot_resources(const AttnParams &p, int head, int slot) {
  const long long hs = (long long)head * p.n_slots + slot;
  SlotRes r;
  if constexpr (BF16KV) {
    r.kc = rsrc(p.k_codes + hs * p.Tc * D * 2, p.Tc * D * 2);
    r.vc = rsrc(p.v_codes + hs * D * p.Tv * 2, D * p.Tv * 2);
    r.ks = r.kc;   // no scales
    r.vs = r.vc;
    return r;
  }
  r.kc = rsrc(p.k_codes + hs * p.Tc * (D / 2), p.Tc * (D / 2));
  r.ks = rsrc(p.k_scales + hs * p.Tc * (D / 16), p.Tc * (D / 16));
  r.vc = rsrc(p.v_codes + hs * D * (p.Tv / 2), D * (p.Tv / 2));
  r.vs = rsrc(p.v_scales + hs * (D / 16) * p.Tv, (D / 16) * p.Tv);
  return r;
}

// K-tile work of group thread lt: key within the tile and 32-dimension part.
// At D = 128 the 8 lanes that store together take 4 keys x 2 parts, so their
// 16-byte stores fall on 8 different groups of 4 LDS banks (stores are
// served 8 lanes at a time); each wave still loads 16 whole keys.
template <int D>
__device__ __forceinline__ int k_key(int lt) {
  if constexpr (D == 128) return (lt & 3) | ((lt >> 1) & 12) | ((lt >> 6) << 4);
  return lt / (D / 32);
}
template <int D>
__device__ __forceinline__ int k_part(int lt) {
  if constexpr (D == 128) return ((lt >> 2) & 1) | ((lt >> 4) & 2);
  return lt % (D / 32);
}

template <int D>
__device__ __forceinline__ void load_k(const SlotRes &sr, int k0, int lt, RawK &r) {
  constexpr int KU = D / 32;
  if (lt < kBN * KU) {   // every thread of the group for D = 128
    const uint32_t key = k0 + k_key<D>(lt), qd = k_part<D>(lt);
    const auto kc = __builtin_amdgcn_raw_buffer_load_b128(sr.kc, key * (D / 2) + 16 * qd, 0, 0);
    r.kc = make_uint4(kc[0], kc[1], kc[2], kc[3]);
    r.ks = __builtin_amdgcn_raw_buffer_load_b16(sr.ks, key * (D / 16) + 2 * qd, 0, 0);
  }
}
template <int D>
__device__ __forceinline__ void load_v(const SlotRes &sr, int Tv, int k0, int lt, RawV &r) {
  if (lt < 2 * D) {
    const int rp = lt >> 2, kg = lt & 3;
    const int tok = k0 + 16 * kg;
    const bool ok = tok < Tv;
    const uint32_t o0 = ok ? (uint32_t)(2 * rp * (Tv / 2) + tok / 2) : kOutOfRange;
    const uint32_t o1 = ok ? o0 + (uint32_t)(Tv / 2) : kOutOfRange;
    const uint32_t os = ok ? (uint32_t)((2 * rp / 16) * Tv + tok) : kOutOfRange;
    const auto c0 = __builtin_amdgcn_raw_buffer_load_b64(sr.vc, o0, 0, 0);
    const auto c1 = __builtin_amdgcn_raw_buffer_load_b64(sr.vc, o1, 0, 0);
    const auto vs = __builtin_amdgcn_raw_buffer_load_b128(sr.vs, os, 0, 0);
    r.vc[0] = make_uint2(c0[0], c0[1]);
    r.vc[1] = make_uint2(c1[0], c1[1]);
    r.vs = make_uint4(vs[0], vs[1], vs[2], vs[3]);
  }
}

template <int D>
__device__ __forceinline__ void load_k(const SlotRes &sr, int k0, int lt, RawKB &r) {
  constexpr int KU = D / 32;
  if (lt < kBN * KU) {
    const uint32_t off = (k0 + k_key<D>(lt)) * (D * 2) + 64 * k_part<D>(lt);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(sr.kc, off + 16 * i, 0, 0);
      r.kc[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}
template <int D>
__device__ __forceinline__ void load_v(const SlotRes &sr, int Tv, int k0, int lt, RawVB &r) {
  if (lt < 2 * D) {
    const int rp = lt >> 2, kg = lt & 3;
    const int tok = k0 + 16 * kg;
    const bool ok = tok < Tv;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const uint32_t o = ok ? (uint32_t)(((2 * rp + rr) * Tv + tok) * 2) : kOutOfRange;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(sr.vc, o + 16 * i, 0, 0);
        r.v[2 * rr + i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

// Largest finite f16: the MFMA operands are f16.
constexpr float kF16Max = 65504.0f;

// Two bf16 values (a 32-bit word) -> f16x2 bits; exact within the f16 range,
// values beyond it saturate to +-65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float a = __builtin_amdgcn_fmed3f(__uint_as_float(w << 16), -kF16Max, kF16Max);
  const float b = __builtin_amdgcn_fmed3f(__uint_as_float(w & 0xFFFF0000u), -kF16Max, kF16Max);
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return bits(h);
}

// K rows past the end of the frame read as zero codes (their scores are
// masked).  V tokens past the end of the frame are the cache's zero padding
// (codes and scales are written as zeros up to Tv) or read as zero, so they
// decode to zero and add nothing to V P.
template <int D>
__device__ __forceinline__ void dequant_k(const RawK &r, int lt, uint16_t (*kt)[D + kPad]) {
  constexpr int KU = D / 32;
  if (lt < kBN * KU) {
    const int key = k_key<D>(lt), qd = k_part<D>(lt);
    const f16x2 s2 = fp8x2<false>(r.ks);
    const f16x2 sa = {s2[0], s2[0]}, sb = {s2[1], s2[1]};
    const uint32_t cw[4] = {r.kc.x, r.kc.y, r.kc.z, r.kc.w};
    uint32_t o[16];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f16x2 sc = w < 2 ? sa : sb;
      o[4 * w + 0] = bits(fp4x2<0>(cw[w]) * sc);
      o[4 * w + 1] = bits(fp4x2<1>(cw[w]) * sc);
      o[4 * w + 2] = bits(fp4x2<2>(cw[w]) * sc);
      o[4 * w + 3] = bits(fp4x2<3>(cw[w]) * sc);
    }
    uint4 *dst = (uint4 *)&kt[krow_phys(key)][32 * qd];
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
}
template <int D>
__device__ __forceinline__ void dequant_v(const RawV &r, int lt, uint16_t (*vt)[kBN + kPad]) {
  if (lt < 2 * D) {
    const int rp = lt >> 2, kg = lt & 3;
    const uint32_t sw[4] = {r.vs.x, r.vs.y, r.vs.z, r.vs.w};
#pragma unroll
    for (int w = 0; w < 2; ++w) {   // tokens 8 w .. 8 w + 7 of both dimensions
      // scales of the token pairs (8 w + 2 j, 8 w + 2 j + 1)
      const f16x2 sc[4] = {fp8x2<false>(sw[2 * w]), fp8x2<true>(sw[2 * w]),
                           fp8x2<false>(sw[2 * w + 1]), fp8x2<true>(sw[2 * w + 1])};
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const uint32_t cw = w == 0 ? r.vc[rr].x : r.vc[rr].y;
        uint4 *dst = (uint4 *)&vt[2 * rp + rr][16 * kg];
        dst[w] = make_uint4(bits(fp4x2<0>(cw) * sc[0]), bits(fp4x2<1>(cw) * sc[1]),
                            bits(fp4x2<2>(cw) * sc[2]), bits(fp4x2<3>(cw) * sc[3]));
      }
    }
  }
}
template <int D>
__device__ __forceinline__ void dequant_k(const RawKB &r, int lt, uint16_t (*kt)[D + kPad]) {
  constexpr int KU = D / 32;
  if (lt < kBN * KU) {
    const int key = k_key<D>(lt), qd = k_part<D>(lt);
    uint4 *dst = (uint4 *)&kt[krow_phys(key)][32 * qd];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = make_uint4(bf16x2_to_f16x2(r.kc[i].x), bf16x2_to_f16x2(r.kc[i].y),
                          bf16x2_to_f16x2(r.kc[i].z), bf16x2_to_f16x2(r.kc[i].w));
  }
}
template <int D>
__device__ __forceinline__ void dequant_v(const RawVB &r, int lt, uint16_t (*vt)[kBN + kPad]) {
  if (lt < 2 * D) {
    const int rp = lt >> 2, kg = lt & 3;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      uint4 *dst = (uint4 *)&vt[2 * rp + rr][16 * kg];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 w = r.v[2 * rr + i];
        dst[i] = make_uint4(bf16x2_to_f16x2(w.x), bf16x2_to_f16x2(w.y), bf16x2_to_f16x2(w.z),
                            bf16x2_to_f16x2(w.w));
      }
    }
  }
}

// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

// S^T (64 keys x the wave's 32 query rows) = K (Q_hi + Q_lo)^T.  The K
// operands are read two k-steps ahead of their MFMAs.
template <int D>
__device__ __forceinline__ void scores(f32x16 (&s)[2], const uint16_t (*kt)[D + kPad], int krow,
                                       int hf, const f16x8 (&qhi)[D / 16],
                                       const f16x8 (&qlo)[D / 16]) {
  constexpr int KS = D / 16;
  f16x8 ka[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int b = 0; b < 2; ++b)
      ka[kk][b] = as_f16x8(*(const uint4 *)&kt[32 * b + krow][16 * kk + 8 * hf]);
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const f16x8 k0 = ka[kk & 1][0], k1 = ka[kk & 1][1];
    if (kk == 0) {   // the first k-step starts from a zero accumulator
      const f32x16 zero = {};
      s[0] = mfma32(k0, qhi[0], zero);
      s[1] = mfma32(k1, qhi[0], zero);
    } else {
      s[0] = mfma32(k0, qhi[kk], s[0]);
      s[1] = mfma32(k1, qhi[kk], s[1]);
    }
    s[0] = mfma32(k0, qlo[kk], s[0]);
    s[1] = mfma32(k1, qlo[kk], s[1]);
    if (kk + 2 < KS) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
        ka[kk & 1][b] = as_f16x8(*(const uint4 *)&kt[32 * b + krow][16 * (kk + 2) + 8 * hf]);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
    if (kk + 2 < KS) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
    if (kk + 2 < KS) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
  }
}

// P = exp2(s * cf - m) rounded to f16 as four P^T operands of 16 keys.
__device__ __forceinline__ void softmax_weights(const f32x16 (&s)[2], float cf, float m,
                                                f16x8 (&pb)[4]) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[b][8 * t2 + 2 * e], cf, -m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[b][8 * t2 + 2 * e + 1], cf, -m));
        const f16x2 ph = {(_Float16)p0, (_Float16)p1};
        w[e] = bits(ph);
      }
      pb[2 * b + t2] = as_f16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
}

// V^T operands of a tile for this wave: slice t4 (16 keys), block db (32
// dimensions) in va[t4 * (D / 32) + db].  They are read in the softmax phase
// before the MFMA phase that uses them.
template <int D>
__device__ __forceinline__ void read_v_operands(f16x8 (&va)[D / 8],
                                                const uint16_t (*vt)[kBN + kPad], int n, int hf) {
  constexpr int DB = D / 32;
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      va[t4 * DB + db] = as_f16x8(*(const uint4 *)&vt[32 * db + n][16 * t4 + 8 * hf]);
}

// O^T += V^T P^T over the four slices of 16 keys of a tile, and this lane's
// share of l += sum of P.  The row sum adds exactly the rounded weights the
// PV product uses (products with 1 are exact, sums in float32).  On the
// VALU it cost about 100 instructions per tile (the compiler rounds each
// weight a second time for it); here it costs eight small MFMAs.
template <int D>
__device__ __forceinline__ void accumulate_pv(f32x16 (&o)[D / 32], f32x4 &lsum,
                                              const f16x8 (&va)[D / 8], const f16x8 (&pb)[4]) {
  constexpr int DB = D / 32;
  const f16x4 ones = {1, 1, 1, 1};
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      o[db] = mfma32(va[t4 * DB + db], pb[t4], o[db]);
    }
    // Row sum on the matrix cores: 16 blocks of 4x4x4 with A all ones give
    // every lane the float32 sum of its own four weights of the operand.
    lsum = __builtin_amdgcn_mfma_f32_4x4x4f16(
        ones, __builtin_shufflevector(pb[t4], pb[t4], 0, 1, 2, 3), lsum, 0, 0, 0);
    lsum = __builtin_amdgcn_mfma_f32_4x4x4f16(
        ones, __builtin_shufflevector(pb[t4], pb[t4], 4, 5, 6, 7), lsum, 0, 0, 0);
  }
}

// Masks the scores of keys at or past nval and of rows that do not see the
// frame, and returns the row maximum times cf (-inf for a fully masked row).
template <bool MASK>
__device__ __forceinline__ float mask_and_max(f32x16 (&s)[2], bool vis, int nval, int hf,
                                              float cf) {
  if (MASK) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = 32 * b + 16 * (j >> 3) + 8 * hf + (j & 7);
        s[b][j] = (vis && key < nval) ? s[b][j] : -INFINITY;
      }
  }
  float part[4];   // four independent chains of 8
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    part[c] = s[c >> 1][8 * (c & 1)];
#pragma unroll
    for (int j = 1; j < 8; ++j) part[c] = fmaxf(part[c], s[c >> 1][8 * (c & 1) + j]);
  }
  const float tmax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  return halves_max(tmax) * cf;
}

template <int D>
__host__ __device__ constexpr size_t smem_bytes() { return sizeof(Smem<D>); }

// Softmax rescaling is lazy: the reference maximum of a row moves only when
// a score exceeds it by more than 2^kTau (log2 units), so weights stay below
// 2^kTau (representable in f16) and the output accumulators are rescaled
// rarely.
constexpr float kTau = 8.0f;

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// Position of a tile in the walk: listed frame fi, tile tt within the frame,
// index i in the walk.
struct Cursor {
  int fi, tt, i;
};

// Workgroup barrier that orders LDS accesses only, so the global loads
// issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier at the end of a VALU phase of a wave that read V operands: its LDS
// writes (the dequantized tile, issued before its D/8 V-operand reads) are
// complete, and up to min(D/8, 15) of the reads stay in flight (15 is the
// largest count the wait takes).  LDS operations of a wave complete in
// order, so at most N outstanding, N no larger than the reads that follow
// the writes, means that every write is done; scalar loads that share the
// counter only add to the operations already complete.  The reads' buffer is
// next written at least three phases later.
template <int D>
__device__ __forceinline__ void barrier_v_reads_in_flight() {
  static_assert(D == 128 || D == 64, "V-operand reads per thread: D / 8");
  if constexpr (D == 128)
    asm volatile("s_waitcnt lgkmcnt(15)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt lgkmcnt(8)\n\ts_barrier" ::: "memory");
}

// The kernel's argument block (a single AttnParams at offset 0), read
// through a pointer the compiler cannot see through.
__device__ __forceinline__ const AttnParams &opaque_params() {
  auto kp = (const __attribute__((address_space(4))) AttnParams *)
      __builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return *(const AttnParams *)kp;
}

// This lane's index within its wave, computed by an instruction the compiler
// cannot move or merge (the count of the wave's lanes below this one), so
// that a value derived from it is derived again where it is needed instead
// of being held across a loop.
__device__ __forceinline__ int fresh_lane() {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return lane;
}

// First virtual tile of workgroup w when n_units tiles are cut into n_wg
// contiguous ranges of (nearly) equal length.
__device__ __forceinline__ long long split_start(int w, long long n_units, int n_wg) {
  return (long long)w * n_units / n_wg;
}

// One log-sum-exp merge step, a_old * acc + a_in * x, with one rounding
// order fixed for both merge paths.
__device__ __forceinline__ float merge_step(float acc, float a_old, float x, float a_in) {
  return fmaf(x, a_in, acc * a_old);
}

// Workgroup whose range holds virtual tile x: the largest w with
// split_start(w) <= x.
__device__ __forceinline__ int split_owner(long long x, long long n_units, int n_wg) {
  return (int)(((x + 1) * n_wg + n_units - 1) / n_units) - 1;
}

// Index in a row block's walk (the tiles of its visible slots, in slot order)
// of the first walked tile at or after virtual tile x = slot * n_tiles + tt.
__device__ __forceinline__ int walk_index(unsigned long long visible, int x, int n_tiles) {
  const int slot = x / n_tiles, tt = x - slot * n_tiles;
  const unsigned long long below = slot >= 64 ? visible : visible & ((1ull << slot) - 1ull);
  const bool here = slot < 64 && ((visible >> slot) & 1ull);
  return __popcll(below) * n_tiles + (here ? tt : 0);
}

// Ping-pong schedule.  The 8 waves form two groups of 4 with one wave of
// each group on every SIMD; both groups walk the same tiles for different
// query rows, offset by one phase.  Phases end at workgroup barriers, and in
// every phase one group issues MFMAs while the other does the softmax:
//   MFMA phase of step t:  O += V(t-1) P(t-1) and l += sum of P(t-1), the
//                          codes of one half of tile t+2 (group 0: V, group
//                          1: K) loaded, then S(t) = K(t) Q'^T;
//   VALU phase of step t:  mask, row max and rescale of S(t), and P(t); the
//                          queries turned into the frame of tile t+1; the
//                          group's half of tile t+2 dequantized; the V
//                          operands of tile t read.
// Group 0 runs MFMA phases on even phases 2t, group 1 on odd phases 2t+1
// after an empty opening phase.  Tiles 0 and 1 are dequantized before phase
// 0.  K(t) is written in phase 2t-2 and read in phases 2t and 2t+1 (2
// buffers); V(t) is written in phase 2t-3 and read in phases 2t+1 and 2t+2,
// where the reads may stay in flight into the next phase (4 buffers: the
// buffer is written again in phase 2t+5).  Every phase ends at a barrier
// after the phase's LDS writes are complete.
template <int D, bool OUT_F32, bool BF16KV>
__global__ __launch_bounds__(kThreads, 1) void attention_kernel(AttnParams p) {
  constexpr int KS = D / 16;   // k-steps of S^T over d
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem<D> &sm = *reinterpret_cast<Smem<D> *>(smem_raw);

  // ---- split schedule.  A row block (kBM query rows of one head, head-major
  // order) has n_v virtual tiles, n_tiles per cache slot; the n_wg
  // workgroups take equal contiguous ranges of the virtual tiles of all row
  // blocks.  Tiles of invisible slots cost nothing, so the ranges are
  // balanced whenever the row blocks see the same frames.  A row block that
  // lies inside one range is finished directly; the pieces of a row block
  // shared by several ranges leave partial results (g_v * acc, m, l) in the
  // workspace, and the workgroup that completes the row block last merges
  // them (with a merge pass, merge_kernel does).  Workgroups are dispatched round-robin over the 8 XCDs (each with
  // its own L2): XCD x takes the contiguous ranges of workgroups
  // [x*per, (x+1)*per), so each head's FP4 KV is read into few L2s.
  const int per = (int)gridDim.x / kXcds;
  const int w = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (w >= p.n_wg) return;
  const long long n_v = (long long)p.n_slots * ((p.Tc + kBN - 1) / kBN);
  const long long n_units = (long long)((p.Nq + kBM - 1) / kBM) * p.H * n_v;
  const long long u0 = split_start(w, n_units, p.n_wg);
  const long long u1 = split_start(w + 1, n_units, p.n_wg);
  if (u0 >= u1) return;
  // The range covers row blocks blk0 .. blk0 + n_blk - 1, from virtual tile
  // lo0 of the first to hi_last of the last.  Row block indices (at most
  // rows x heads / 256 + heads, with rows x heads <= 2^31) and n_v (64 slots
  // of < 2^18 tiles) fit in int, so the segment loop runs on 32-bit scalar
  // arithmetic; only u0, u1 and n_units need 64 bits.
  const int blk0 = (int)(u0 / n_v);
  const int n_blk = (int)((u1 - 1) / n_v) - blk0 + 1;
  const int lo0 = (int)(u0 - blk0 * n_v);
  const int hi_last = (int)(u1 - (blk0 + n_blk - 1) * n_v);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  for (int bi = 0; bi < n_blk; ++bi) {
    const int blk = blk0 + bi;
    // Every wave has finished reading the previous row block's frame list,
    // turn table and tiles once it passes this barrier.  (The first row
    // block needs none; the barrier is unconditional so that the protocol
    // does not depend on the order in which row blocks are visited.)
    __syncthreads();
    // The kernel arguments and the lane index are made opaque in every
    // segment (opaque_params, fresh_lane), so that the compiler derives
    // addresses, divisors and thread indices here instead of holding them
    // (spilled) across the segment loop.
    const AttnParams &p = opaque_params();
    const int lane = fresh_lane();
    const int tid = wave * 64 + lane;
    const int n_qt = (p.Nq + kBM - 1) / kBM;
    const int n_tiles = (p.Tc + kBN - 1) / kBN;
    const int last_nval = p.Tc - (n_tiles - 1) * kBN;
    const int half_rot = p.rot_dim >> 1;
    const int f1 = p.q_frame0 + p.n_q_frames;
    const int ws = max(p.S, f1 - p.W);
    const int n_v = p.n_slots * n_tiles;
    const long long n_units = (long long)n_qt * p.H * n_v;
    const long long vbase = (long long)blk * n_v;
    const int v_lo = bi == 0 ? lo0 : 0, v_hi = bi == n_blk - 1 ? hi_last : n_v;
    const int n = lane & 31, hf = lane >> 5;
    const int grp = __builtin_amdgcn_readfirstlane(tid >> 8);
    const int lt = tid & 255;   // thread index within the group
    const int head = (int)(blk / n_qt);
    const int wg_row0 = (int)(blk - (long long)head * n_qt) * kBM;
    const int my_row = wg_row0 + wave * 32 + n;
    const bool row_ok = my_row < p.Nq;
    const int my_qf = p.q_frame0 + (row_ok ? my_row : p.Nq - 1) / p.T;
    const int my_qshot = p.q_shot[my_qf - p.q_frame0];
    const int my_qchunk = my_qf / p.C;

    // ---- visible key frames of this row block (ballot over the slots).
    // Every wave derives the mask, and from it the segment's walk range, in
    // scalar registers; wave 0 writes the compacted frame list.
    const int qf_lo = p.q_frame0 + wg_row0 / p.T;
    const int qf_hi = p.q_frame0 + (min(p.Nq, wg_row0 + kBM) - 1) / p.T;
    bool ok = false;
    int kf = -1, kshot = 0;
    bool sink = false;
    if (lane < p.n_slots) {
      kf = p.slot_frame[lane];
      kshot = p.slot_shot[lane];
      // a sink slot holds frame kf < S of the stream (seen across shots),
      // or with per-shot sinks one of the first S frames of some shot
      // (seen by that shot only); its position is its slot
      sink = p.sink_per_shot ? lane < p.S : kf < p.S;
      const bool exempt = sink && !p.sink_per_shot;
      ok = kf >= 0 && kf < f1 && (sink || kf >= ws);
      if (ok) {
        bool any = false;
        for (int qf = qf_lo; qf <= qf_hi; ++qf)
          any |= (kf / p.C <= qf / p.C) && (exempt || kshot == p.q_shot[qf - p.q_frame0]);
        ok = any;
      }
    }
    const unsigned long long mask = __ballot(ok);
    if (wave == 0 && ok) {
      const int idx = __popcll(mask & ((1ull << lane) - 1ull));
      sm.fl_slot[idx] = lane;
      sm.fl_kf[idx] = kf;
      sm.fl_pos[idx] = sink ? lane : p.S + (kf - ws);
      sm.fl_shot[idx] = kshot;
      sm.fl_gk[idx] = p.k_tscale[lane];
      sm.fl_gv[idx] = p.v_tscale[lane];
    }
    __syncthreads();

    // The segment walks the tiles [c0, c0 + n_total) of the row block's walk,
    // from tile ta of listed frame fa to tile te of listed frame fe.
    const int c0 = walk_index(mask, v_lo, n_tiles);
    const int n_total = walk_index(mask, v_hi, n_tiles) - c0;
    const int fa = c0 / n_tiles, ta = c0 - fa * n_tiles;
    const int fe = (c0 + max(n_total, 1) - 1) / n_tiles, te = c0 + max(n_total, 1) - 1 - fe * n_tiles;

    // ---- turn into listed frame fi: R(-(pos(fi) - pos(fi - 1))), and
    // R(-pos(fa)) into the segment's first frame; pairs past rot_dim / 2 get
    // the identity (1, 0)
    for (int i = tid; i < (n_total > 0 ? fe - fa + 1 : 0) * (D / 2); i += kThreads) {
      const int fi = fa + i / (D / 2), j = i % (D / 2);
      const int dpos = sm.fl_pos[fi] - (fi > fa ? sm.fl_pos[fi - 1] : 0);
      float2 cs = make_float2(1.0f, 0.0f);
      if (j < half_rot) {
        const float2 t = *(const float2 *)(p.cos_sin + (long long)abs(dpos) * p.rot_dim + 2 * j);
        cs = make_float2(t.x, dpos >= 0 ? -t.y : t.y);
      }
      sm.rot[fi][j] = cs;
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[b][j] = 0.0f;
    float m_run = -1.0e30f, gv_last = 1.0f;
    f32x4 lsum = {};   // element 0: this lane's share of the row sum

    if (n_total > 0) {
      const int krow = krow_phys(sigma(n));   // + 32 b for key block b
      const long long qoff = ((long long)(row_ok ? my_row : 0) * p.H + head) * D + 8 * hf;
      f16x8 qhi[KS], qlo[KS];

      // Turns the queries into listed frame fi: the first frame reads the
      // rotated queries from memory, later frames turn the previous frame's.
      auto turn_queries = [&](int fi, bool from_memory) __attribute__((always_inline)) {
        const float2 *rot = sm.rot[fi];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          float x[8];
          if (from_memory) {
            if (p.q_f32) {
              const float4 a = *(const float4 *)((const float *)p.q + qoff + 16 * kk);
              const float4 b = *(const float4 *)((const float *)p.q + qoff + 16 * kk + 4);
              x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
              x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
            } else {
              const uint4 v = *(const uint4 *)((const uint16_t *)p.q + qoff + 16 * kk);
              const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                x[2 * e] = __uint_as_float(w[e] << 16);
                x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
              }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = row_ok ? x[e] : 0.0f;
            // The f16 range bounds the query operands: a rotary pair whose
            // norm exceeds 65504 is scaled to norm 65504 (turns keep a
            // pair's norm, so no later turn leaves the range), an element
            // past the rotary pairs is clamped to +-65504.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (8 * kk + 4 * hf + e < p.sat_half) {
                // norm taken on values scaled by 2^-66 so that no finite
                // input overflows the square
                const float sa = x[2 * e] * 0x1p-66f, sb = x[2 * e + 1] * 0x1p-66f;
                const float n2 = sa * sa + sb * sb;
                if (n2 > (kF16Max * 0x1p-66f) * (kF16Max * 0x1p-66f)) {
                  const float f = (kF16Max * 0x1p-66f) * __builtin_amdgcn_rsqf(n2);
                  x[2 * e] *= f;
                  x[2 * e + 1] *= f;
                }
              } else {
                x[2 * e] = __builtin_amdgcn_fmed3f(x[2 * e], -kF16Max, kF16Max);
                x[2 * e + 1] = __builtin_amdgcn_fmed3f(x[2 * e + 1], -kF16Max, kF16Max);
              }
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)qhi[kk][e] + (float)qlo[kk][e];
          }
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 cs = rot[8 * kk + 4 * hf + e];
            float ra, rb;
            rotate_pair(x[2 * e], x[2 * e + 1], cs.x, cs.y, ra, rb);
            const f16x2 h2 = {(_Float16)ra, (_Float16)rb};
            const f16x2 l2 = {(_Float16)(ra - (float)h2[0]), (_Float16)(rb - (float)h2[1])};
            hw[e] = bits(h2);
            lw[e] = bits(l2);
          }
          qhi[kk] = as_f16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
          qlo[kk] = as_f16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
      };

      // Next tile of the walk (the segment's last tile stays put).
      auto advance = [&](Cursor c) __attribute__((always_inline)) {
        if (c.fi == fe && c.tt == te) return c;
        ++c.i;
        if (++c.tt == n_tiles) {
          c.tt = 0;
          ++c.fi;
        }
        return c;
      };
      // Per-frame values of the frame of the tile whose softmax comes next:
      // visibility of this lane's row, whether the whole wave sees the frame,
      // the exp2 factor softmax_scale * log2(e) * g_k and the value scale g_v.
      // f_ratio = g_v(previous frame) / g_v(this frame) keeps O = g_v * acc.
      bool f_vis = false, f_all = false;
      float f_cf = 0.0f, f_gv = 1.0f, f_ratio = 1.0f;
      auto load_frame = [&](int fi) __attribute__((always_inline)) {
        const int kf = sm.fl_kf[fi];
        f_vis = row_ok & (kf / p.C <= my_qchunk) &
                ((!p.sink_per_shot & (kf < p.S)) | (sm.fl_shot[fi] == my_qshot));
        f_all = __ballot(f_vis) == ~0ull;
        f_cf = p.scale_log2 * sm.fl_gk[fi];
        const float gv = sm.fl_gv[fi];
        f_ratio = __fdiv_rn(f_gv, gv);
        f_gv = gv;
      };

      // Each group dequantizes one half (group 0: V, group 1: K) of the tiles
      // in walk order; cd is the next tile whose codes are loaded or loading.
      // The two groups run the same walk; group 1 dequantizes K halves and
      // group 0 V halves, so each group's code holds only its own codes.
      // L: the wave has query rows below Nq.  A wave past the last row (in
      // the ragged last row block of a head) skips its MFMAs and softmax and
      // only dequantizes its share of the tiles.
      auto run_group = [&](auto gtag, auto ltag) __attribute__((always_inline)) {
        constexpr bool G = decltype(gtag)::value;
        constexpr bool L = decltype(ltag)::value;
        typename RawOf<G, BF16KV>::type raw;
        Cursor cd = {fa, ta, 0};
        // (the slot index is wave-uniform; read as such, the descriptors sit in
        // scalar registers and the tile loads need no waterfall loop)
        SlotRes res = slot_resources<D, BF16KV>(
            p, head, __builtin_amdgcn_readfirstlane(sm.fl_slot[fa]));   // frame of cd
        auto load_half = [&]() __attribute__((always_inline)) {
          if constexpr (G) load_k<D>(res, cd.tt * kBN, lt, raw);
          else load_v<D>(res, p.Tv, cd.tt * kBN, lt, raw);
        };
        // Dequantizes the half tile cd.i into its buffer (tiles past the end
        // of the walk are never read and are skipped).
        auto dequant_tile = [&]() __attribute__((always_inline)) {
          if (cd.i < n_total) {
            if constexpr (G) dequant_k<D>(raw, lt, sm.kh[cd.i % kKBufs]);
            else dequant_v<D>(raw, lt, sm.vt[cd.i % kVBufs]);
          }
        };
        // Moves cd to the next tile and loads its codes (past the end of the
        // walk the loads repeat the last tile).
        auto next_codes = [&]() __attribute__((always_inline)) {
          Cursor nx = advance(cd);
          nx.i = cd.i + 1;
          if (nx.fi != cd.fi)
            res = slot_resources<D, BF16KV>(p, head, __builtin_amdgcn_readfirstlane(sm.fl_slot[nx.fi]));
          cd = nx;
          load_half();
        };

        // ---- prologue: tiles 0 and 1 dequantized
        load_half();
        dequant_tile();
        next_codes();
        dequant_tile();
        lds_barrier();   // tiles 0 and 1, the turn table and the frame list are in LDS

        if constexpr (L) turn_queries(fa, true);
        load_frame(fa);
        Cursor ct = {fa, ta, 0};   // tile of this group's next S and softmax
        f32x16 s[2];
        f16x8 pb[4];
        f16x8 va[D / 8];   // V operands of the tile whose PV comes next

        // Softmax of tile t (ct): mask, row max, lazy rescale of O and l
        // together with the g_v ratio on the first tile of a frame, then P and l.
        auto softmax_tile = [&](auto masked) __attribute__((always_inline)) {
          const int nval = ct.tt == n_tiles - 1 ? last_nval : kBN;
          const float tmax = mask_and_max<decltype(masked)::value>(s, f_vis, nval, hf, f_cf);
          const bool first = ct.i > 0 && ct.tt == 0;
          float factor = first ? f_ratio : 1.0f;
          bool scale_o = first;
          if (__ballot(tmax > m_run + kTau) != 0ull) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            lsum[0] *= alpha;
            factor *= alpha;
            scale_o = true;
          }
          if (scale_o) {
    #pragma unroll
            for (int b = 0; b < DB; ++b)
    #pragma unroll
              for (int j = 0; j < 16; ++j) oacc[b][j] *= factor;
          }
          softmax_weights(s, f_cf, m_run, pb);
        };

        // VALU phase of step t: softmax of tile t, the queries turned into the
        // frame of tile t+1, the group's half of tile t+2 dequantized, and the
        // V operands of tile t read
        auto valu_phase = [&](int t) __attribute__((always_inline)) {
          if constexpr (L) {
            if (t < n_total) {
              if (!f_all || (ct.tt == n_tiles - 1 && last_nval < kBN))
                softmax_tile(BoolC<true>());
              else
                softmax_tile(BoolC<false>());
            }
          }
          if (t + 1 < n_total) {
            const Cursor cn = advance(ct);
            if (cn.fi != ct.fi) {
              if constexpr (L) turn_queries(cn.fi, false);
              load_frame(cn.fi);
            }
            ct = cn;
          }
          // The group's half of tile t + 2 (its codes were loaded in the MFMA
          // phase), then the V operands of tile t for the next MFMA phase
          dequant_tile();
          // the tile stores stay ahead of the V reads (the barrier after this
          // phase waits for all but the last 8 LDS operations)
          asm volatile("" ::: "memory");
          if constexpr (L) read_v_operands<D>(va, sm.vt[t % kVBufs], n, hf);
        };

        // MFMA phase of step t: PV of tile t - 1, then S of tile t.  It issues
        // matrix work only, at raised priority; the dequantization runs in the
        // VALU phase, where the other group's MFMAs leave issue cycles free.
        auto mfma_phase = [&](int t, auto has_pv, auto has_s) __attribute__((always_inline)) {
          __builtin_amdgcn_s_setprio(1);
          if constexpr (L && decltype(has_pv)::value) accumulate_pv<D>(oacc, lsum, va, pb);
          next_codes();   // of tile t + 2
          if constexpr (L && decltype(has_s)::value)
            scores<D>(s, sm.kh[t % kKBufs], krow, hf, qhi, qlo);
          __builtin_amdgcn_s_setprio(0);
          lds_barrier();
        };

        if (G) lds_barrier();   // group 1's opening phase
        auto valu_barrier = [&]() __attribute__((always_inline)) {
          if constexpr (L) barrier_v_reads_in_flight<D>();
          else lds_barrier();   // no V reads follow the LDS writes
        };
        mfma_phase(0, BoolC<false>(), BoolC<true>());
        valu_phase(0);
        valu_barrier();
        for (int t = 1; t < n_total; ++t) {
          mfma_phase(t, BoolC<true>(), BoolC<true>());
          valu_phase(t);
          valu_barrier();
        }
        mfma_phase(n_total, BoolC<true>(), BoolC<false>());
        if (!G) lds_barrier();   // group 0's closing phase
        gv_last = f_gv;
      };
      const bool live = wg_row0 + wave * 32 < p.Nq;   // wave-uniform
      if (grp) {
        if (live) run_group(BoolC<true>(), BoolC<true>());
        else run_group(BoolC<true>(), BoolC<false>());
      } else {
        if (live) run_group(BoolC<false>(), BoolC<true>());
        else run_group(BoolC<false>(), BoolC<false>());
      }
    }

    // ---- epilogue: O = g_v * acc / l, g_v of the last frame walked.  The
    // lane's rows are derived again, so that nothing per lane is held across
    // the tile loop.
    const int e_lane = fresh_lane();
    const int e_n = e_lane & 31, e_hf = e_lane >> 5;
    const int e_row = wave * 32 + e_n, e_my_row = wg_row0 + e_row;
    const float l = halves_sum(lsum[0]);
    auto store_out = [&](float inv) __attribute__((always_inline)) {
      if (e_my_row >= p.Nq) return;
      const long long obase = ((long long)e_my_row * p.H + head) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 32 * db + 8 * i + 4 * e_hf;
          const float v0 = oacc[db][4 * i] * inv, v1 = oacc[db][4 * i + 1] * inv;
          const float v2 = oacc[db][4 * i + 2] * inv, v3 = oacc[db][4 * i + 3] * inv;
          if (OUT_F32) {
            *(float4 *)((float *)p.o + obase + d) = make_float4(v0, v1, v2, v3);
          } else {
            const uint32_t w0 = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
            const uint32_t w1 = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
            *(uint2 *)((uint16_t *)p.o + obase + d) = make_uint2(w0, w1);
          }
        }
    };
    if (v_lo == 0 && v_hi == n_v) {   // the whole row block
      store_out(l > 0.0f ? __fdiv_rn(gv_last, l) : 0.0f);
      continue;
    }

    // ---- a piece of a shared row block: publish (g_v * acc, m, l) in the
    // workgroup's first or second partial slot, then count the piece in.
    // Pieces are written and read with device-coherent (sc1) accesses, which
    // do not stop in an XCD's L2, so no L2 writeback or invalidation is
    // needed between workgroups on different XCDs.
    const __amdgpu_buffer_rsrc_t ws_o =
        rsrc((const uint8_t *)p.ws_o, (uint32_t)(2 * p.n_wg * kBM * D * 4));
    const __amdgpu_buffer_rsrc_t ws_ml =
        rsrc((const uint8_t *)p.ws_ml, (uint32_t)(2 * p.n_wg * kBM * 8));
    {
      const int slot = bi == 0 ? 2 * w : 2 * w + 1;
      const int ob = ((slot * kBM + e_row) * D + 4 * e_hf) * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            oacc[db][4 * i + e] *= gv_last;
            x[e] = __float_as_uint(oacc[db][4 * i + e]);
          }
          __builtin_amdgcn_raw_buffer_store_b128(x, ws_o, ob + (32 * db + 8 * i) * 4, 0, kSc1);
        }
      if (e_hf == 0) {
        const u32x2 ml = {__float_as_uint(m_run), __float_as_uint(l)};
        __builtin_amdgcn_raw_buffer_store_b64(ml, ws_ml, (slot * kBM + e_row) * 8, 0, kSc1);
      }
    }
    if (p.merge_pass) continue;   // merge_kernel combines the pieces
    const int w_first = split_owner(vbase, n_units, p.n_wg);
    const int w_last = split_owner(vbase + n_v - 1, n_units, p.n_wg);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the piece is written
    __syncthreads();
    if (wave == 0 && e_lane == 0)
      sm.merge_last = __hip_atomic_fetch_add(p.ws_cnt + w_first, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == w_last - w_first;
    __syncthreads();
    if (!sm.merge_last) continue;
    if (wave == 0 && e_lane == 0)   // ready for the next launch
      __hip_atomic_store(p.ws_cnt + w_first, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- the last piece in: log-sum-exp merge of all pieces of the row
    // block, its own included, in workgroup order (so the result does not
    // depend on which workgroup came last)
    float m_all = -1.0e30f, l_all = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[db][j] = 0.0f;
    for (int wc = w_first; wc <= w_last; ++wc) {
      const int slot = 2 * wc + (split_start(wc, n_units, p.n_wg) < vbase ? 1 : 0);
      const u32x2 ml = __builtin_amdgcn_raw_buffer_load_b64(ws_ml, (slot * kBM + e_row) * 8, 0, kSc1);
      const float m_in = __uint_as_float(ml[0]), l_in = __uint_as_float(ml[1]);
      const float m_new = fmaxf(m_all, m_in);
      const float a_old = __builtin_amdgcn_exp2f(m_all - m_new);
      const float a_in = __builtin_amdgcn_exp2f(m_in - m_new);
      m_all = m_new;
      l_all = merge_step(l_all, a_old, l_in, a_in);
      const int ib = ((slot * kBM + e_row) * D + 4 * e_hf) * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 x =
              __builtin_amdgcn_raw_buffer_load_b128(ws_o, ib + (32 * db + 8 * i) * 4, 0, kSc1);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            oacc[db][4 * i + e] =
                merge_step(oacc[db][4 * i + e], a_old, __uint_as_float(x[e]), a_in);
        }
    }
    store_out(l_all > 0.0f ? __fdiv_rn(1.0f, l_all) : 0.0f);
  }
}

// Merge pass of the split schedule, for calls whose row blocks are cut into
// many pieces: the pieces of a row block are combined by 8 workgroups (one
// per 32-row slice, one wave per 32-dimension block) instead of by the one
// workgroup that finishes last.  The arithmetic per output element is the
// in-kernel merge's, in the same workgroup order; up to 8 pieces' loads are
// in flight at once.  Row blocks finished inside one range are skipped.
constexpr int kMergeSlices = kBM / 32;
constexpr int kMergeBatch = 8;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(64 * (D / 32)) void merge_kernel(AttnParams p) {
  const int n_qt = (p.Nq + kBM - 1) / kBM;
  const int n_tiles = (p.Tc + kBN - 1) / kBN;
  const long long n_v = (long long)p.n_slots * n_tiles;
  const long long n_units = (long long)n_qt * p.H * n_v;
  const int rb = (int)blockIdx.x / kMergeSlices, slice = (int)blockIdx.x % kMergeSlices;
  const long long vbase = (long long)rb * n_v;
  const int w_first = split_owner(vbase, n_units, p.n_wg);
  const int w_last = split_owner(vbase + n_v - 1, n_units, p.n_wg);
  if (w_first == w_last) return;   // finished by its one workgroup
  const int db = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int n = lane & 31, hf = lane >> 5;
  const int row = slice * 32 + n;   // row within the row block
  const int head = rb / n_qt;
  const int my_row = (rb - head * n_qt) * kBM + row;
  if (my_row >= p.Nq) return;
  const __amdgpu_buffer_rsrc_t ws_o =
      rsrc((const uint8_t *)p.ws_o, (uint32_t)(2 * p.n_wg * kBM * D * 4));
  const __amdgpu_buffer_rsrc_t ws_ml =
      rsrc((const uint8_t *)p.ws_ml, (uint32_t)(2 * p.n_wg * kBM * 8));
  float m_all = -1.0e30f, l_all = 0.0f;
  float acc[16] = {};
  for (int w0 = w_first; w0 <= w_last; w0 += kMergeBatch) {
    u32x2 ml[kMergeBatch];
    u32x4 x[kMergeBatch][4];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int wc = w0 + k;
      if (wc <= w_last) {
        const int slot = 2 * wc + (split_start(wc, n_units, p.n_wg) < vbase ? 1 : 0);
        ml[k] = __builtin_amdgcn_raw_buffer_load_b64(ws_ml, (slot * kBM + row) * 8, 0, kSc1);
        const int ib = ((slot * kBM + row) * D + 4 * hf) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[k][i] =
              __builtin_amdgcn_raw_buffer_load_b128(ws_o, ib + (32 * db + 8 * i) * 4, 0, kSc1);
      }
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (w0 + k <= w_last) {
        const float m_in = __uint_as_float(ml[k][0]), l_in = __uint_as_float(ml[k][1]);
        const float m_new = fmaxf(m_all, m_in);
        const float a_old = __builtin_amdgcn_exp2f(m_all - m_new);
        const float a_in = __builtin_amdgcn_exp2f(m_in - m_new);
        m_all = m_new;
        l_all = merge_step(l_all, a_old, l_in, a_in);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[4 * i + e] = merge_step(acc[4 * i + e], a_old, __uint_as_float(x[k][i][e]), a_in);
      }
    }
  }
  const float inv = l_all > 0.0f ? __fdiv_rn(1.0f, l_all) : 0.0f;
  const long long obase = ((long long)my_row * p.H + head) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = 32 * db + 8 * i + 4 * hf;
    const float v0 = acc[4 * i] * inv, v1 = acc[4 * i + 1] * inv;
    const float v2 = acc[4 * i + 2] * inv, v3 = acc[4 * i + 3] * inv;
    if (OUT_F32) {
      *(float4 *)((float *)p.o + obase + d) = make_float4(v0, v1, v2, v3);
    } else {
      const uint32_t w0 = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
      const uint32_t w1 = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
      *(uint2 *)((uint16_t *)p.o + obase + d) = make_uint2(w0, w1);
    }
  }
}

template <int D, bool OUT_F32, bool BF16KV>
hipError_t launch_one(const AttnParams &p, hipStream_t s) {
  constexpr size_t bytes = smem_bytes<D>();
  static const hipError_t attr = hipFuncSetAttribute(
      (const void *)attention_kernel<D, OUT_F32, BF16KV>,
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)((p.n_wg + kXcds - 1) / kXcds * kXcds));
  hipLaunchKernelGGL((attention_kernel<D, OUT_F32, BF16KV>), grid, dim3(kThreads), bytes, s, p);
  if (!p.merge_pass) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n_rb = (long long)(p.Nq + kBM - 1) / kBM * p.H;
  hipLaunchKernelGGL((merge_kernel<D, OUT_F32>), dim3((unsigned)(n_rb * kMergeSlices)),
                     dim3(64 * (D / 32)), 0, s, p);
  return hipGetLastError();
}

template <bool BF16KV>
hipError_t launch_kv(const AttnParams &p, int head_dim, int out_f32, hipStream_t s) {
  if (head_dim == 128)
    return out_f32 ? launch_one<128, true, BF16KV>(p, s) : launch_one<128, false, BF16KV>(p, s);
  return out_f32 ? launch_one<64, true, BF16KV>(p, s) : launch_one<64, false, BF16KV>(p, s);
}

}  // namespace

hipError_t launch_attention(const AttnParams &p, int head_dim, int out_f32, hipStream_t s) {
  return p.bf16_cache ? launch_kv<true>(p, head_dim, out_f32, s)
                      : launch_kv<false>(p, head_dim, out_f32, s);
}

}  // namespace fp4kv
