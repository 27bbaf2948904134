// Chunk attention over the NVFP4 KV cache with the FP4 dequantization fused
// into the attention loop ("faster FP4 KV dequantization", hysenlabs.com,
// "NVFP4, sequence parallel and the async decode path"), sink + window
// visibility (heatdrop.ai, "What it does"), block-causal chunks and shot
// masks (evermx.com, "Multi-Shot Generation"), and cache-relative RoPE
// (refft.com, question "How do KV-cache relative RoPE and TriAttention work
// together ...").
//
// Work layout (gfx950, wave64, MFMA 32x32x16 with f16 operands, f32 accum):
//   * one workgroup = 128 query rows of one head, 4 waves x 32 rows;
//   * the keys of every visible frame are walked in tiles of 64.  The packed
//     FP4 codes and E4M3 scales of tile i+1 are loaded into registers while
//     tile i is computed, then dequantized once per workgroup into a second
//     LDS buffer (one barrier per tile).  Dequantization is exact: E2M1 x E4M3
//     has at most 6 significant bits and lies in [2^-10, 2688], so it fits
//     f16; the hardware converts two FP4 codes to f16 (scale 1) and one packed
//     f16 multiply applies the block scale;
//   * each wave computes S^T = K Q^T so that a lane owns one query row in
//     both the score and the output accumulators: the softmax row max and sum
//     stay inside a lane plus one exchange with the lane 32 away;
//   * O^T += V^T P^T, with P taken straight from the score registers and V
//     read dimension-major, as the cache stores it.
//
// Rotation: the cache holds keys before rotation.  Rotating q by pos(qf) and
// k by pos(kf) gives the same score as rotating q by pos(qf) - pos(kf), so
// each wave turns its rotated queries back by -pos(kf) once per key frame and
// the keys need no rotation.
//
// Precision: the turned-back queries are split into an f16 high part and an
// f16 low part (two MFMAs on the same exact key operand), so scores carry
// about 22 bits; P is rounded to f16.  softmax_scale * log2(e) * g_k (the key
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

constexpr int kBM = 128;   // query rows per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPad = 8;    // f16 elements of padding per LDS row
constexpr int kXcds = 8;   // accelerator complex dies of MI355X

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

template <int D>
struct Smem {
  uint16_t kh[2][kBN][D + kPad];   // dequantized K tiles, f16 bits
  uint16_t vt[2][D][kBN + kPad];   // dequantized V tiles, dimension-major
  int fl_slot[FP4KV_MAX_SLOTS];
  int fl_kf[FP4KV_MAX_SLOTS];
  int fl_pos[FP4KV_MAX_SLOTS];
  int fl_shot[FP4KV_MAX_SLOTS];
  float fl_gk[FP4KV_MAX_SLOTS];
  float fl_gv[FP4KV_MAX_SLOTS];
  int n_fl;
};

// Packed codes and scales of one tile held by one thread between the load
// and the dequantization.
struct Raw {
  uint4 kc;        // 32 key elements (16 bytes) of one key
  uint32_t ks;     // their two block scales (low 16 bits)
  uint2 vc[2];     // 16 tokens of two value dimensions
  uint4 vs;        // the 16 tokens' scales of that value block
};

// Loads are unconditional (addresses clamped into the frame, results
// zeroed afterwards) so the compiler keeps them in flight across the compute
// of the current tile instead of waiting at a branch.
template <int D>
__device__ __forceinline__ void load_tile(const AttnParams &p, int head, int slot, int k0,
                                          int nval, Raw &r) {
  const int tid = threadIdx.x;
  constexpr int KU = D / 32;
  if (tid < kBN * KU) {   // all threads for D = 128
    const int key = tid / KU, qd = tid % KU;
    const bool ok = key < nval;
    const long long row = ((long long)head * p.n_slots + slot) * p.Tc + k0 + (ok ? key : 0);
    const uint4 kc = *(const uint4 *)(p.k_codes + row * (D / 2) + 16 * qd);
    const uint32_t ks = *(const uint16_t *)(p.k_scales + row * (D / 16) + 2 * qd);
    r.kc = ok ? kc : make_uint4(0, 0, 0, 0);
    r.ks = ok ? ks : 0u;
  }
  if (tid < 2 * D) {
    const int rp = tid >> 2, kg = tid & 3;
    const int tok = k0 + 16 * kg;
    const bool ok = tok < p.Tv;
    const int tk = ok ? tok : 0;
    const long long drow = ((long long)head * p.n_slots + slot) * D + 2 * rp;
    const uint2 c0 = *(const uint2 *)(p.v_codes + drow * (p.Tv / 2) + tk / 2);
    const uint2 c1 = *(const uint2 *)(p.v_codes + (drow + 1) * (p.Tv / 2) + tk / 2);
    const long long srow = ((long long)head * p.n_slots + slot) * (D / 16) + (2 * rp) / 16;
    const uint4 vs = *(const uint4 *)(p.v_scales + srow * p.Tv + tk);
    r.vc[0] = ok ? c0 : make_uint2(0, 0);
    r.vc[1] = ok ? c1 : make_uint2(0, 0);
    r.vs = ok ? vs : make_uint4(0, 0, 0, 0);
  }
}

// Physical LDS row of key k in a K tile: rows 8..15 of every 16 swap their
// halves, so the 8 lanes that read together (keys {0-3, 8-11} + 16j and
// {4-7, 12-15} + 16j under sigma) hit 8 different bank groups.
__device__ __forceinline__ int krow_phys(int k) { return k ^ (((k >> 3) & 1) << 2); }

template <int D>
__device__ __forceinline__ void dequant_tile(const Raw &r, int nval, Smem<D> &sm, int buf) {
  const int tid = threadIdx.x;
  constexpr int KU = D / 32;
  if (tid < kBN * KU) {
    const int key = tid / KU, qd = tid % KU;
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
    // rows past the end of the frame were not loaded: they hold zeros, and
    // zero codes decode to zero
    uint4 *dst = (uint4 *)&sm.kh[buf][krow_phys(key)][32 * qd];
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
  if (tid < 2 * D) {
    const int rp = tid >> 2, kg = tid & 3;
    const uint32_t sw[4] = {r.vs.x, r.vs.y, r.vs.z, r.vs.w};
    f16x2 sc[8];   // scales of token pairs (2j, 2j+1)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc[2 * w] = fp8x2<false>(sw[w]);
      sc[2 * w + 1] = fp8x2<true>(sw[w]);
    }
    const int valid = nval - 16 * kg;   // tokens of this unit inside the frame
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const uint32_t cw[2] = {r.vc[rr].x, r.vc[rr].y};
      uint32_t o[8];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        o[4 * w + 0] = bits(fp4x2<0>(cw[w]) * sc[4 * w + 0]);
        o[4 * w + 1] = bits(fp4x2<1>(cw[w]) * sc[4 * w + 1]);
        o[4 * w + 2] = bits(fp4x2<2>(cw[w]) * sc[4 * w + 2]);
        o[4 * w + 3] = bits(fp4x2<3>(cw[w]) * sc[4 * w + 3]);
      }
      if (valid < 16) {   // tail of the frame: padding tokens contribute zero
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t keep = (2 * j + 1 < valid) ? 0xFFFFFFFFu : (2 * j < valid ? 0xFFFFu : 0u);
          o[j] &= keep;
        }
      }
      uint4 *dst = (uint4 *)&sm.vt[buf][2 * rp + rr][16 * kg];
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

template <int D>
__host__ __device__ constexpr size_t smem_bytes() { return sizeof(Smem<D>); }

// Softmax rescaling is lazy: the reference maximum of a row moves only when
// a score exceeds it by more than 2^kTau (log2 units), so weights stay below
// 2^kTau (representable in f16) and the output accumulators are rescaled
// rarely.
constexpr float kTau = 8.0f;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(AttnParams p) {
  constexpr int KS = D / 16;   // k-steps of S^T over d
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem<D> &sm = *reinterpret_cast<Smem<D> *>(smem_raw);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hf = lane >> 5;
  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2).  Give XCD x the contiguous work items [x*per, (x+1)*per) in
  // head-major order, so each head's FP4 KV is read into few L2s.
  const int n_qt = (p.Nq + kBM - 1) / kBM;
  const int n_work = n_qt * p.H;
  const int per = (n_work + kXcds - 1) / kXcds;
  const int work = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (work >= n_work) return;
  const int head = work / n_qt;
  const int f1 = p.q_frame0 + p.n_q_frames;
  const int ws = max(p.S, f1 - p.W);

  const int wg_row0 = (work - head * n_qt) * kBM;
  const int my_row = wg_row0 + wave * 32 + n;
  const bool row_ok = my_row < p.Nq;
  const int my_qf = p.q_frame0 + (row_ok ? my_row : p.Nq - 1) / p.T;
  const int my_qshot = p.q_shot[my_qf - p.q_frame0];
  const int my_qchunk = my_qf / p.C;

  // ---- visible key frames of this workgroup (one wave, ballot compaction)
  if (wave == 0) {
    const int qf_lo = p.q_frame0 + wg_row0 / p.T;
    const int qf_hi = p.q_frame0 + (min(p.Nq, wg_row0 + kBM) - 1) / p.T;
    bool ok = false;
    int kf = -1, kshot = 0;
    if (lane < p.n_slots) {
      kf = p.slot_frame[lane];
      kshot = p.slot_shot[lane];
      ok = kf >= 0 && kf < f1 && (kf < p.S || kf >= ws);
      if (ok) {
        bool any = false;
        for (int qf = qf_lo; qf <= qf_hi; ++qf)
          any |= (kf / p.C <= qf / p.C) && (kf < p.S || kshot == p.q_shot[qf - p.q_frame0]);
        ok = any;
      }
    }
    const unsigned long long mask = __ballot(ok);
    const int idx = __popcll(mask & ((1ull << lane) - 1ull));
    if (ok) {
      sm.fl_slot[idx] = lane;
      sm.fl_kf[idx] = kf;
      sm.fl_pos[idx] = kf < p.S ? kf : p.S + (kf - ws);
      sm.fl_shot[idx] = kshot;
      sm.fl_gk[idx] = p.k_tscale[lane];
      sm.fl_gv[idx] = p.v_tscale[lane];
    }
    if (lane == 0) sm.n_fl = __popcll(mask);
  }
  __syncthreads();

  const int n_fl = sm.n_fl;
  const int n_tiles = (p.Tc + kBN - 1) / kBN;
  const int last_nval = p.Tc - (n_tiles - 1) * kBN;

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[b][j] = 0.0f;
  float m_run = -1.0e30f, l_part = 0.0f, gv_cur = 1.0f;
  const int half_rot = p.rot_dim >> 1;
  const int krow = krow_phys(sigma(n));   // + 32 b for key block b
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  const long long qoff = ((long long)(row_ok ? my_row : 0) * p.H + head) * D + 8 * hf;
  f16x8 qhi[KS], qlo[KS];
  int prev_pos = 0;

  Raw raw;
  int buf = 0;
  if (n_fl > 0) {
    const int nv0 = n_tiles == 1 ? last_nval : kBN;
    load_tile<D>(p, head, sm.fl_slot[0], 0, nv0, raw);
    dequant_tile<D>(raw, nv0, sm, 0);
  }
  __syncthreads();

  for (int fi = 0; fi < n_fl; ++fi) {
    // ---- new key frame: visibility, tensor scales, turned-back queries
    const int kf = sm.fl_kf[fi], pos = sm.fl_pos[fi];
    const float gv = sm.fl_gv[fi];
    const bool lane_vis =
        row_ok && (kf / p.C <= my_qchunk) && (kf < p.S || sm.fl_shot[fi] == my_qshot);
    const bool wave_any = __ballot(lane_vis) != 0ull;
    const bool wave_all = __ballot(lane_vis) == ~0ull;
    if (fi > 0) {   // keep O = g_v * acc across the change of tensor scale
      const float ratio = __fdiv_rn(gv_cur, gv);
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[b][j] *= ratio;
    }
    gv_cur = gv;
    const float cf = p.scale_log2 * sm.fl_gk[fi];
    // Queries turned back by -pos(kf) as f16 hi + lo.  The first frame reads
    // the rotated queries; later frames turn the previous frame's queries by
    // -(pos(kf) - pos(prev)), so the queries are read from memory once.
    {
      const int dpos = fi == 0 ? pos : pos - prev_pos;
      const float sgn = dpos >= 0 ? -1.0f : 1.0f;   // R(-dpos) = (c, -s) of |dpos|
      const float *tab = p.cos_sin + (long long)abs(dpos) * p.rot_dim;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        float x[8];
        if (fi == 0) {
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
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (float)qhi[kk][e] + (float)qlo[kk][e];
        }
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pair = 8 * kk + 4 * hf + e;
          float ra = x[2 * e], rb = x[2 * e + 1];
          if (pair < half_rot) {
            const float2 cs = *(const float2 *)(tab + 2 * pair);
            rotate_pair(x[2 * e], x[2 * e + 1], cs.x, sgn * cs.y, ra, rb);
          }
          const f16x2 h2 = {(_Float16)ra, (_Float16)rb};
          const f16x2 l2 = {(_Float16)(ra - (float)h2[0]), (_Float16)(rb - (float)h2[1])};
          hw[e] = bits(h2);
          lw[e] = bits(l2);
        }
        qhi[kk] = as_f16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
        qlo[kk] = as_f16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
    }
    prev_pos = pos;

    for (int t = 0; t < n_tiles; ++t) {
      const int nval = t == n_tiles - 1 ? last_nval : kBN;
      // ---- prefetch the next tile's packed codes and scales
      const bool has_next = t + 1 < n_tiles || fi + 1 < n_fl;
      int nval_next = 0;
      if (has_next) {
        const bool same = t + 1 < n_tiles;
        const int tn = same ? t + 1 : 0;
        nval_next = tn == n_tiles - 1 ? last_nval : kBN;
        load_tile<D>(p, head, sm.fl_slot[same ? fi : fi + 1], tn * kBN, nval_next, raw);
      }

      if (wave_any) {
        // ---- S^T = K (Q_hi + Q_lo)^T for 2 blocks of 32 keys
        // all 16 K operands are read first; the MFMAs then alternate between
        // the two key blocks so consecutive MFMAs never share an accumulator
        f32x16 sacc[2];
        f16x8 ka[2][KS];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int kk = 0; kk < KS; ++kk)
            ka[b][kk] = as_f16x8(*(const uint4 *)&sm.kh[buf][32 * b + krow][16 * kk + 8 * hf]);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) sacc[b][j] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          sacc[0] = mfma32(ka[0][kk], qhi[kk], sacc[0]);
          sacc[1] = mfma32(ka[1][kk], qhi[kk], sacc[1]);
          sacc[0] = mfma32(ka[0][kk], qlo[kk], sacc[0]);
          sacc[1] = mfma32(ka[1][kk], qlo[kk], sacc[1]);
        }
        __builtin_amdgcn_s_setprio(0);
        // ---- mask (tail tiles and rows that do not see this frame)
        if (!(wave_all && nval == kBN)) {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int key = 32 * b + 16 * (j >> 3) + 8 * hf + (j & 7);
              sacc[b][j] = (lane_vis && key < nval) ? sacc[b][j] : -INFINITY;
            }
        }
        // ---- online softmax, exp2 argument = s * cf - m
        float tmax = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, sacc[b][j]);
        tmax = halves_max(tmax) * cf;
        const bool grow = tmax > m_run + kTau;
        if (__ballot(grow) != 0ull) {
          const float m_new = fmaxf(m_run, tmax);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_part *= alpha;
#pragma unroll
          for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[b][j] *= alpha;
        }
        f16x8 pb[4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[b][8 * t2 + 2 * e], cf, -m_run));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[b][8 * t2 + 2 * e + 1], cf, -m_run));
              const f16x2 ph = {(_Float16)p0, (_Float16)p1};
              l_part = __builtin_amdgcn_fdot2(ph, ones, l_part, false);
              w[e] = bits(ph);
            }
            pb[2 * b + t2] = as_f16x8(make_uint4(w[0], w[1], w[2], w[3]));
          }
        // ---- O^T += V^T P^T, 4 slices of 16 keys
        // V operands are read DB ahead of their MFMA
        __builtin_amdgcn_s_setprio(1);
        f16x8 va[4][DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
          va[0][db] = as_f16x8(*(const uint4 *)&sm.vt[buf][32 * db + n][8 * hf]);
        __builtin_amdgcn_sched_group_barrier(0x100, DB, 0);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            if (t4 + 1 < 4)
              va[t4 + 1][db] =
                  as_f16x8(*(const uint4 *)&sm.vt[buf][32 * db + n][16 * (t4 + 1) + 8 * hf]);
            oacc[db] = mfma32(va[t4][db], pb[t4], oacc[db]);
            if (t4 + 1 < 4) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            } else {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }

      if (has_next) dequant_tile<D>(raw, nval_next, sm, buf ^ 1);
      buf ^= 1;
      __syncthreads();
    }
  }

  // ---- epilogue: O = g_v * acc / l
  const float l = halves_sum(l_part);
  const float inv = l > 0.0f ? __fdiv_rn(gv_cur, l) : 0.0f;
  if (!row_ok) return;
  const long long obase = ((long long)my_row * p.H + head) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * hf;
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
}

template <int D, bool OUT_F32>
hipError_t launch_one(const AttnParams &p, hipStream_t s) {
  constexpr size_t bytes = smem_bytes<D>();
  static const hipError_t attr = hipFuncSetAttribute(
      (const void *)attention_kernel<D, OUT_F32>, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)bytes);
  if (attr != hipSuccess) return attr;
  const int n_work = (p.Nq + kBM - 1) / kBM * p.H;
  const dim3 grid((n_work + kXcds - 1) / kXcds * kXcds);
  hipLaunchKernelGGL((attention_kernel<D, OUT_F32>), grid, dim3(kThreads), bytes, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnParams &p, int head_dim, int out_f32, hipStream_t s) {
  if (head_dim == 128) return out_f32 ? launch_one<128, true>(p, s) : launch_one<128, false>(p, s);
  return out_f32 ? launch_one<64, true>(p, s) : launch_one<64, false>(p, s);
}

}  // namespace fp4kv
