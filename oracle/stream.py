"""The FP4 KV cache as a stream of chunk steps, in the library's layout.

TEST INFRASTRUCTURE (CPU oracle); see oracle/__init__.py.

Chains the oracle's parts into the three operations of the path:
  * append: quantize a new chunk's K and V to NVFP4 and write them in place
    into the ring of sink + window slots ("in-place quantized KV-cache
    updates", hysenlabs.com, "NVFP4, sequence parallel and the async decode
    path");
  * rope: rotate queries (or keys) by cache-relative position (refft.com,
    relative RoPE and TriAttention question);
  * attention: decode the cache and attend with block-causal, window and
    shot masks (evermx.com, "Multi-Shot Generation").

Cache layout (the byte layout the GPU library must reproduce bit for bit).
Keys are stored token-major, values dimension-major; both keep NVFP4 blocks
of 16 consecutive elements along D.  Tv = Tc rounded up to a multiple of 32;
value entries of the padding tokens Tc..Tv-1 are zero.
  k_codes   uint8 [H][S+W][Tc][D/2]   key codes; element 2j of a row in the
                                      low nibble, 2j+1 in the high nibble
  k_scales  uint8 [H][S+W][Tc][D/16]  E4M3 scale of each key block
  v_codes   uint8 [H][S+W][D][Tv/2]   value codes of one dimension d across
                                      tokens; token 2j low nibble, 2j+1 high
  v_scales  uint8 [H][S+W][D/16][Tv]  E4M3 scale of value block b of each token
  k_tscale, v_tscale float32 [S+W]    tensor scale g of the frame
  slot_frame         int32 [S+W]      frame held, -1 when empty
  slot_shot          int32 [S+W]      shot id of that frame
OracleCache holds keys before rotation; keys are rotated after decoding
with the positions of the current step, so codes are written once and never
re-quantized when the window slides (reading of "KV-cache relative RoPE").
OracleCacheRot is the other reading: keys stored rotated and turned in place
when the window slides.

Keeping every token_stride-th token of each cached frame stands in for the
pages' KV compression (refft.com, "TriAttention compression"); queries are
never decimated.  The per-tensor scale is computed over the kept tokens of
one appended tensor (K or V of one call, all heads).
"""
from __future__ import annotations

import copy

import numpy as np

from . import attention as att
from . import nvfp4
from . import ring
from . import rope


class OracleCache:
    def __init__(self, H, D, T, C, S, W, token_stride=1, rot_dim=None,
                 base=10000.0, sink_per_shot=False):
        assert T % token_stride == 0 and D % nvfp4.BLOCK == 0
        self.H, self.D, self.T, self.C, self.S, self.W = H, D, T, C, S, W
        self.stride = token_stride
        self.Tc = T // token_stride
        self.rot_dim = D if rot_dim is None else rot_dim
        self.base = base
        self.sink_per_shot = sink_per_shot   # see ring.slot_of_shot
        n = S + W
        self.Tv = -(-self.Tc // 32) * 32
        self.k_codes = np.zeros((H, n, self.Tc, D // 2), np.uint8)
        self.v_codes = np.zeros((H, n, D, self.Tv // 2), np.uint8)
        self.k_scales = np.zeros((H, n, self.Tc, D // 16), np.uint8)
        self.v_scales = np.zeros((H, n, D // 16, self.Tv), np.uint8)
        self.k_tscale = np.ones(n, np.float32)
        self.v_tscale = np.ones(n, np.float32)
        self.slot_frame = np.full(n, -1, np.int32)
        self.slot_shot = np.zeros(n, np.int32)

    @classmethod
    def for_workload(cls, w, rot_dim=None, sink_per_shot=False):
        return cls(w.H, w.D, w.T, w.C, w.S, w.W, w.token_stride, rot_dim,
                   sink_per_shot=sink_per_shot)

    def slot(self, f, fs=0):
        """Slot of frame f (fs: first frame of its shot, per-shot sinks)."""
        if self.sink_per_shot:
            return ring.slot_of_shot(f, fs, self.S, self.W)
        return ring.slot_of(f, self.S, self.W)

    def snapshot(self):
        return copy.deepcopy(self)

    # ---------------------------------------------------------------- append
    def kept(self, x, n_frames):
        """[n_frames*T][H][D] -> kept tokens [n_frames][Tc][H][D]."""
        x = np.asarray(x, dtype=np.float32).reshape(n_frames, self.T, self.H, self.D)
        return x[:, ::self.stride]

    def append(self, k, v, frame0, n_frames, shots, tscale=None, shot_starts=None):
        """Quantize K, V ([n_frames*T][H][D], float32 values) into the slots of
        frames frame0 .. frame0+n_frames-1 (shot_starts: first frame of each
        frame's shot, per-shot sinks only).  Returns (g_k, g_v)."""
        fss = [0] * n_frames if shot_starts is None else list(shot_starts)
        gs = []
        for idx, (x, tsc) in enumerate(((k, self.k_tscale), (v, self.v_tscale))):
            xk = self.kept(x, n_frames)                        # [n][Tc][H][D]
            g = nvfp4.tensor_scale(xk) if tscale is None else self.caller_scale(tscale[idx])
            c, s8 = nvfp4.encode_blocks(xk, g)                 # codes per element
            for j in range(n_frames):
                slot = self.slot(frame0 + j, fss[j])
                cj = c[j].transpose(1, 0, 2)                   # [H][Tc][D]
                sj = s8[j].transpose(1, 0, 2)                  # [H][Tc][D/16]
                if idx == 0:
                    self.k_codes[:, slot] = nvfp4.pack_nibbles(cj)
                    self.k_scales[:, slot] = sj
                else:
                    pad = self.Tv - self.Tc
                    ct = np.pad(cj.transpose(0, 2, 1), ((0, 0), (0, 0), (0, pad)))
                    self.v_codes[:, slot] = nvfp4.pack_nibbles(ct)      # [H][D][Tv/2]
                    self.v_scales[:, slot] = np.pad(sj.transpose(0, 2, 1),
                                                    ((0, 0), (0, 0), (0, pad)))
                tsc[slot] = g
            gs.append(g)
        for j in range(n_frames):
            slot = self.slot(frame0 + j, fss[j])
            self.slot_frame[slot] = frame0 + j
            self.slot_shot[slot] = shots[j]
        return tuple(gs)

    @staticmethod
    def caller_scale(g):
        """Reading (the pages fix none): a caller-supplied tensor scale is used
        when it is finite and positive; zero, negative, infinite or NaN
        scales are replaced by 1, so no cached scale makes decoding
        undefined."""
        g = np.float32(g)
        return g if (np.isfinite(g) and g > 0) else np.float32(1.0)

    def decode_slot(self, slot):
        """(k_hat, v_hat) float32 [H][Tc][D] of one slot."""
        kh = nvfp4.decode_blocks(nvfp4.unpack_nibbles(self.k_codes[:, slot]),
                                 self.k_scales[:, slot], self.k_tscale[slot])
        cv = nvfp4.unpack_nibbles(self.v_codes[:, slot])[:, :, :self.Tc]   # [H][D][Tc]
        sv = self.v_scales[:, slot][:, :, :self.Tc]                        # [H][D/16][Tc]
        vh = nvfp4.decode_blocks(cv.transpose(0, 2, 1), sv.transpose(0, 2, 1),
                                 self.v_tscale[slot])
        return kh, vh

    def operands(self, kh, vh):
        """Decoded keys and values as attention uses them (NVFP4 values are
        at most 6 * 448 * g in magnitude, so nothing changes here)."""
        return kh, vh

    # ------------------------------------------------------------ positions
    def positions(self, frames, f1, shot_starts=None):
        if self.sink_per_shot:
            return np.array([ring.pos_shot(f, fs, f1, self.S, self.W)
                             for f, fs in zip(frames, shot_starts)])
        return np.array([ring.rel_pos(f, f1, self.S, self.W) for f in frames])

    # Largest finite f16.  Reading (the pages fix no operand format): the
    # attention operands are f16, so a query whose rotary pair (2i, 2i+1),
    # i < rot_dim/2, has a norm above F16_MAX is scaled to norm F16_MAX (a
    # turn keeps the norm, so the scaling commutes with the rotation), and a
    # query element past rot_dim is clamped to +-F16_MAX.  Inputs within the
    # f16 range are unchanged.
    F16_MAX = 65504.0

    def rope_queries(self, q, q_frame0, n_q_frames, q_shot_starts=None):
        """Rotate q[n_q_frames*T][H][D] by the cache-relative positions of its
        frames, then saturate it to the f16 range (F16_MAX); float64 result."""
        f1 = q_frame0 + n_q_frames
        pos = self.positions(range(q_frame0, f1), f1, q_shot_starts)
        pos_tok = np.repeat(pos, self.T)[:, None]           # [Nq, 1] over heads
        y = rope.rotate(q, pos_tok, self.rot_dim, self.base)
        rd = self.rot_dim
        a, b = y[..., 0:rd:2], y[..., 1:rd:2]
        norm = np.sqrt(a * a + b * b)
        f = np.where(norm > self.F16_MAX, self.F16_MAX / np.maximum(norm, 1.0), 1.0)
        y[..., 0:rd:2] = a * f
        y[..., 1:rd:2] = b * f
        y[..., rd:] = np.clip(y[..., rd:], -self.F16_MAX, self.F16_MAX)
        return y

    # ------------------------------------------------------------ attention
    def rotate_keys(self, k, kpos):
        """Decoded keys [Nk][D] turned by their cache-relative positions
        (float64): this cache stores keys before rotation."""
        return rope.rotate(k, kpos, self.rot_dim, self.base)

    def visible_slots(self, f1):
        ws = ring.window_start(f1, self.S, self.W)
        out = []
        for slot in range(self.S + self.W):
            kf = int(self.slot_frame[slot])
            sink = slot < self.S if self.sink_per_shot else kf < self.S
            if 0 <= kf < f1 and (sink or kf >= ws):
                out.append((slot, kf))
        return out

    def attention(self, q, q_frame0, n_q_frames, q_shots, scale=None,
                  return_probs=False, rows=None, heads=None, q_shot_starts=None):
        """Chunk attention for query frames q_frame0 .. +n_q_frames-1.

        q: float32 values [n_q_frames*T][H][D] before rotation.
        rows / heads: optional subsets of query tokens / heads to compute
        (each output element depends only on its own query row and head).
        Returns float64 o[len(rows)][len(heads)][D] (all rows and heads by
        default)."""
        H, D, T, S, W, C = self.H, self.D, self.T, self.S, self.W, self.C
        f1 = q_frame0 + n_q_frames
        rows = np.arange(n_q_frames * T) if rows is None else np.asarray(rows)
        heads = list(range(H)) if heads is None else list(heads)
        qr = self.rope_queries(q, q_frame0, n_q_frames, q_shot_starts)[rows]  # [Nr][H][D]
        ws = ring.window_start(f1, S, W)
        slots = self.visible_slots(f1)
        keys, vals, kpos = [], [], []
        for slot, kf in slots:
            kh, vh = self.operands(*self.decode_slot(slot))    # [H][Tc][D]
            keys.append(kh)
            vals.append(vh)
            if self.sink_per_shot:
                kpos.append(np.full(self.Tc, slot if slot < S else S + (kf - ws)))
            else:
                kpos.append(np.full(self.Tc, ring.rel_pos(kf, f1, S, W)))
        K = np.concatenate(keys, axis=1)                       # [H][Nk][D]
        V = np.concatenate(vals, axis=1)
        kpos = np.concatenate(kpos)
        frame_rows = {}
        for a, qf in enumerate(range(q_frame0, f1)):
            if self.sink_per_shot:
                per_slot = [ring.key_visible_shot(kf, slot, qf, f1, S, W, C,
                                                  int(self.slot_shot[slot]), int(q_shots[a]))
                            for slot, kf in slots]
            else:
                per_slot = [ring.key_visible(kf, qf, f1, S, W, C,
                                             int(self.slot_shot[slot]), int(q_shots[a]))
                            for slot, kf in slots]
            frame_rows[a] = np.repeat(np.array(per_slot, dtype=bool), self.Tc)
        mask = np.stack([frame_rows[int(r) // T] for r in rows])
        out = np.empty((len(rows), len(heads), D), np.float64)
        probs = []
        for hi, h in enumerate(heads):
            kr = self.rotate_keys(K[h], kpos)
            if return_probs:
                s = (qr[:, h] @ kr.T) * (1.0 / np.sqrt(D) if scale is None else scale)
                probs.append(att.softmax_rows(s, mask))
            out[:, hi] = att.attend(qr[:, h], kr, V[h], mask, scale)
        if return_probs:
            return out, probs
        return out


# ------------------------------------------------------------ bf16 baseline
def bf16_round(x):
    """float32 -> the nearest bf16 value (ties to even), kept as float32.
    Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


class OracleCacheBF16(OracleCache):
    """The unquantized baseline the NVFP4 cache is measured against: the same
    ring of sink + window slots, keys and values kept as bf16 (rounded to
    nearest even at append), tensor scales 1.

    Layout (the library's FP4KV_FORMAT_BF16_V1), as float32 values here:
      k_vals  [H][S+W][Tc][D]   keys, token-major
      v_vals  [H][S+W][D][Tv]   values, dimension-major; padding tokens zero
    """

    def __init__(self, *a, **kw):
        super().__init__(*a, **kw)
        n = self.S + self.W
        self.k_vals = np.zeros((self.H, n, self.Tc, self.D), np.float32)
        self.v_vals = np.zeros((self.H, n, self.D, self.Tv), np.float32)

    def append(self, k, v, frame0, n_frames, shots, tscale=None, shot_starts=None):
        fss = [0] * n_frames if shot_starts is None else list(shot_starts)
        for idx, x in enumerate((k, v)):
            xk = bf16_round(self.kept(x, n_frames))             # [n][Tc][H][D]
            for j in range(n_frames):
                slot = self.slot(frame0 + j, fss[j])
                if idx == 0:
                    self.k_vals[:, slot] = xk[j].transpose(1, 0, 2)
                else:
                    self.v_vals[:, slot] = 0.0
                    self.v_vals[:, slot, :, :self.Tc] = xk[j].transpose(1, 2, 0)
        for j in range(n_frames):
            slot = self.slot(frame0 + j, fss[j])
            self.k_tscale[slot] = self.v_tscale[slot] = 1.0
            self.slot_frame[slot] = frame0 + j
            self.slot_shot[slot] = shots[j]
        return (np.float32(1.0), np.float32(1.0))

    def decode_slot(self, slot):
        return (self.k_vals[:, slot].copy(),
                self.v_vals[:, slot, :, :self.Tc].transpose(0, 2, 1).copy())

    def operands(self, kh, vh):
        """Reading (the pages fix no operand format): attention takes f16
        operands, so stored bf16 keys and values beyond the f16 range
        saturate to +-F16_MAX when attention reads them; the stored bf16
        values themselves are unchanged."""
        return (np.clip(kh, -self.F16_MAX, self.F16_MAX),
                np.clip(vh, -self.F16_MAX, self.F16_MAX))


# ------------------------------------------------- rotate-at-write variant
class OracleCacheRot(OracleCache):
    """The other reading of "KV-cache relative RoPE" (refft.com, relative RoPE
    and TriAttention question; aiany.app, "What Sets It Apart"): keys are
    stored already rotated by their cache-relative position, and when the
    window start moves the surviving window keys are turned back in place.

    Reading, step by step:
      * a key frame is written rotated by its position at the step that
        appends it (window end f1 = the end of that step's frames): rotate in
        float32 (rope.rotate_f32 with the float32 table), then NVFP4-encode
        as any append (one tensor scale over the call's kept tokens);
      * when the window end moves from f1_from to f1_to the window start
        moves by delta = ws(f1_to) - ws(f1_from); every window slot (slot
        >= S) whose frame f satisfies ws(f1_to) <= f < f1_from survives and
        is turned by -delta: decode (float32), rotate_f32 inverse with table
        row delta, encode again with a fresh tensor scale amax / 2688 over
        that frame's kept keys (all heads); values and sink slots never
        move (a sink frame's position is fixed);
      * attention decodes keys and uses them as stored (no key rotation);
        queries are rotated by their positions as before.
    Each window key is re-encoded once per step it survives, up to
    ceil(W / C) - 1 times in steady state: the re-quantization error is the
    price of this reading.
    """

    def __init__(self, *a, table=None, **kw):
        super().__init__(*a, **kw)
        n = self.S + self.W
        self.table = (rope.table_f32(n, self.rot_dim, self.base) if table is None
                      else np.asarray(table, np.float32))

    def rotate_keys(self, k, kpos):
        return np.asarray(k, np.float64)

    def append_rotated(self, k, v, frame0, n_frames, shots, tscale=None, shot_starts=None,
                       f1=None):
        """Rotate the keys of frames frame0 .. +n_frames-1 by their positions at
        the window ending at f1 (default frame0 + n_frames), then append."""
        f1 = frame0 + n_frames if f1 is None else f1
        fss = [0] * n_frames if shot_starts is None else list(shot_starts)
        pos = self.positions(range(frame0, frame0 + n_frames), f1, fss)
        rows = np.repeat(pos, self.T)                               # per token
        kk = np.asarray(k, np.float32).reshape(n_frames * self.T, self.H, self.D)
        kr = rope.rotate_f32(kk, self.table[rows][:, None])         # same turn for all heads
        return self.append(kr, v, frame0, n_frames, shots, tscale=tscale,
                           shot_starts=shot_starts)

    def rerotate(self, f1_from, f1_to):
        """Move the stored key rotations from the window ending at f1_from to
        the one ending at f1_to.  Returns the slots re-encoded."""
        S, W = self.S, self.W
        ws0, ws1 = ring.window_start(f1_from, S, W), ring.window_start(f1_to, S, W)
        delta = ws1 - ws0
        done = []
        if delta == 0:
            return done
        for slot in range(S, S + W):
            f = int(self.slot_frame[slot])
            if not (ws1 <= f < f1_from):
                continue
            kh = nvfp4.decode_blocks(nvfp4.unpack_nibbles(self.k_codes[:, slot]),
                                     self.k_scales[:, slot], self.k_tscale[slot])  # [H][Tc][D]
            kr = rope.rotate_f32(kh, self.table[delta], inverse=True)
            g = nvfp4.tensor_scale(kr)
            codes, s8 = nvfp4.encode_blocks(kr, g)
            self.k_codes[:, slot] = nvfp4.pack_nibbles(codes)
            self.k_scales[:, slot] = s8
            self.k_tscale[slot] = g
            done.append(slot)
        return done
