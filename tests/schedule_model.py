"""CPU model of the attention kernel's workgroup protocol: the barrier
sequence of its 8 waves and every LDS access, plus the split schedule's
piece slots and merge counters.  Test infrastructure: it restates the
schedule that csrc/attention.hip describes in its comments (phases, buffers,
which barrier waits for what) and checks that schedule for races; it shares
no code with the kernel.

Waves 0..3 form group 0 (dequantizes the V half of each tile), waves 4..7
group 1 (the K half).  A wave's events are barriers and LDS accesses
(kind 'R' or 'W', a location, and a lifetime: 0 = complete before the wave's
next barrier, 1 = may stay in flight across that barrier).  Two accesses to
one location by different waves, at least one a write, race when their
barrier intervals overlap."""
from __future__ import annotations

import itertools


def split_start(w, n_units, n_wg):
    return w * n_units // n_wg


def split_owner(x, n_units, n_wg):
    """Workgroup whose range holds virtual tile x."""
    return ((x + 1) * n_wg + n_units - 1) // n_units - 1


def segments(n_qt, H, n_v, n_wg):
    """Per workgroup: the (row block, v_lo, v_hi) pieces of its range."""
    n_units = n_qt * H * n_v
    out = []
    for w in range(n_wg):
        u0, u1 = split_start(w, n_units, n_wg), split_start(w + 1, n_units, n_wg)
        segs = []
        blk = u0 // n_v if u0 < u1 else None
        while blk is not None and blk * n_v < u1:
            vb = blk * n_v
            segs.append((blk, max(u0, vb) - vb, min(u1, vb + n_v) - vb))
            blk += 1
        out.append(segs)
    return out, n_units


def check_pieces(n_qt, H, n_v, n_wg, reverse=False):
    """The slot a workgroup writes for a cut row block is the slot the merger
    reads for it, and no counter serves two row blocks."""
    segs, n_units = segments(n_qt, H, n_v, n_wg)
    written, counters = {}, {}
    for w, lst in enumerate(segs):
        if not lst:
            continue
        blk0 = lst[0][0]
        for blk, vlo, vhi in (reversed(lst) if reverse else lst):
            if vlo == 0 and vhi == n_v:
                continue
            slot = 2 * w if blk == blk0 else 2 * w + 1
            assert slot not in written, ("slot written twice", w, slot)
            written[slot] = blk
            counters.setdefault(split_owner(blk * n_v, n_units, n_wg), set()).add(blk)
    for wf, s in counters.items():
        assert len(s) == 1, ("counter shared", wf, s)
    for blk in range(n_qt * H):
        vb = blk * n_v
        wf, wl = split_owner(vb, n_units, n_wg), split_owner(vb + n_v - 1, n_units, n_wg)
        for wc in range(wf, wl + 1) if wf != wl else ():
            slot = 2 * wc + (1 if split_start(wc, n_units, n_wg) < vb else 0)
            assert written.get(slot) == blk, ("merger reads a slot not written for it", blk, wc)


def segment_events(n_total, frames, lists, merge, live, kbufs, vbufs):
    """Events of the 8 waves for one segment of n_total tiles (frames[i] is
    the listed frame of tile i).  The segment opens with the unconditional
    workgroup barrier of the kernel."""
    waves = []
    for wave in range(8):
        G, L = wave >> 2, live[wave]
        ev = [('B',)]
        if wave == 0:                                   # frame list (every wave
            ev += [('W', loc, 0) for loc in lists]      # derives the walk range)
        ev += [('B',)]
        if n_total == 0:
            if merge:
                ev += [('B',)] + ([('W', 'merge', 0)] if wave == 0 else []) + [('B',), ('R', 'merge', 0)]
            waves.append(ev)
            continue
        fa, fe = frames[0], frames[-1]
        for fi in range(fa, fe + 1):                    # turn table
            ev.append(('R', ('fl_pos', fi), 0))
            ev.append(('W', ('rot', fi), 0))
        buf, nbuf = ('kh', kbufs) if G else ('vt', vbufs)
        ev.append(('R', ('fl_slot', fa), 0))
        cd = 0

        def dequant_tile():
            if cd < n_total:
                ev.append(('W', (buf, cd % nbuf), 0))

        def next_codes():
            nonlocal cd
            cur, nx = min(cd, n_total - 1), min(cd + 1, n_total - 1)
            if frames[nx] != frames[cur]:
                ev.append(('R', ('fl_slot', frames[nx]), 0))
            cd += 1

        dequant_tile()                                  # prologue: tiles 0 and 1
        next_codes()
        dequant_tile()
        ev.append(('B',))
        if L:
            ev.append(('R', ('rot', fa), 0))
        ev += [('R', (f, fa), 0) for f in ('fl_kf', 'fl_shot', 'fl_gk', 'fl_gv')]
        if G:
            ev.append(('B',))                           # group 1's opening phase

        def mfma_phase(t, has_s):
            next_codes()                                # codes of tile t + 2
            if L and has_s:
                ev.append(('R', ('kh', t % kbufs), 0))  # K operands of S(t)
            ev.append(('B',))

        def valu_phase(t):
            if t + 1 < n_total and frames[t + 1] != frames[t]:
                if L:
                    ev.append(('R', ('rot', frames[t + 1]), 0))
                ev.extend(('R', (f, frames[t + 1]), 0) for f in ('fl_kf', 'fl_shot', 'fl_gk', 'fl_gv'))
            dequant_tile()                              # tile t + 2
            if L:                                       # V operands, left in flight
                ev.append(('R', ('vt', t % vbufs), 1))
            ev.append(('B',))

        for t in range(n_total):
            mfma_phase(t, True)
            valu_phase(t)
        mfma_phase(n_total, False)
        if not G:
            ev.append(('B',))                           # group 0's closing phase
        if merge:
            ev += [('B',)] + ([('W', 'merge', 0)] if wave == 0 else []) + [('B',), ('R', 'merge', 0)]
        waves.append(ev)
    return waves


def races(waves):
    """Conflicting accesses of different waves with overlapping intervals."""
    acc = {}
    n_bar = None
    for w, ev in enumerate(waves):
        k = 0
        for e in ev:
            if e[0] == 'B':
                k += 1
                continue
            kind, loc, life = e
            acc.setdefault(loc, []).append((w, kind, k, k + life))
        assert n_bar is None or n_bar == k, "barrier counts differ between waves"
        n_bar = k
    out = []
    for loc, lst in acc.items():
        for a, b in itertools.combinations(lst, 2):
            if a[0] == b[0] or (a[1] == 'R' and b[1] == 'R'):
                continue
            if a[1] == 'W' and b[1] == 'W' and isinstance(loc, tuple) and loc[0] in ('rot', 'kh', 'vt'):
                continue   # the threads of a group write disjoint entries
            if not (a[3] < b[2] or b[3] < a[2]):
                out.append((loc, a, b))
    return out


def random_workgroups(rng, cases, kbufs, vbufs, reverse=False):
    """Runs random split schedules (row blocks, tiles per frame, visible
    frames, dead waves, workgroup counts) and returns the races found."""
    found = []
    for _ in range(cases):
        n_qt, H = rng.randint(1, 4), rng.randint(1, 3)
        n_tiles, n_slots = rng.randint(1, 3), rng.randint(1, 6)
        n_v = n_slots * n_tiles
        n_wg = rng.randint(1, min(40, n_qt * H * n_v))
        check_pieces(n_qt, H, n_v, n_wg, reverse)
        segs, _ = segments(n_qt, H, n_v, n_wg)
        for lst in segs:
            waves = [[] for _ in range(8)]
            for blk, vlo, vhi in (reversed(lst) if reverse else lst):
                vis = sorted(rng.sample(range(n_slots), rng.randint(1, n_slots)))

                def widx(x):
                    s, tt = divmod(x, n_tiles)
                    return sum(1 for v in vis if v < s) * n_tiles + (tt if s in vis else 0)

                c0, c1 = widx(vlo), widx(vhi)
                n_total = max(c1 - c0, 0)
                frames = [(c0 + i) // n_tiles for i in range(n_total)]
                lists = [(f, i) for f in ('fl_slot', 'fl_kf', 'fl_pos', 'fl_shot', 'fl_gk', 'fl_gv')
                         for i in range(len(vis))]
                live = [rng.random() < 0.8 for _ in range(8)]
                ev = segment_events(n_total, frames, lists, not (vlo == 0 and vhi == n_v), live,
                                    kbufs, vbufs)
                for i in range(8):
                    waves[i] += ev[i]
            found += races(waves)
    return found
