"""Host model of the decode stream kernel's work split (the balanced shares).

Test infrastructure.  It replays, with Python integers, what every wave of
``decode_stream_kernel`` (``paged_kv_cache_75_amd/csrc/pa_kernels.hip``)
works out before it reads the pools: the units of each (sequence, kv head)
pair (its attended 16-token tiles plus one for the pair's fixed cost), the
equal share bounds, the runs of
segments the lanes find in parallel (at most ``seg_cap`` per run, at most 64
candidate sequences per search), each segment's tiles and piece flags, and the
piece headers the merge kernel reads.  It holds no attention arithmetic and is
not the oracle: CPU tests use it to check that the split covers every attended
tile exactly once and that the piece bookkeeping is consistent, on batches the
full-size workloads never produce (empty sequences, one-tile sequences, a huge
sequence among tiny ones, windows).
"""

from __future__ import annotations

import dataclasses

TILE = 16
PAIR_COST = 1
WAVE = 64
PIECE_FIRST, PIECE_LAST, SHARE_FIRST = 1, 2, 4


def window_first(T: int, window: int) -> int:
    return max(0, T - window) if window > 0 else 0


def attended_tiles(T: int, window: int) -> int:
    return (T + TILE - 1) // TILE - window_first(T, window) // TILE if T > 0 else 0


def pair_units(T: int, window: int) -> int:
    t = attended_tiles(T, window)
    return t + PAIR_COST if t else 0


def share_lo(total: int, w: int, nsh: int) -> int:
    return total * w // nsh


def share_of(total: int, u: int, nsh: int) -> int:
    """The largest w with share_lo(w) <= u, in closed form."""
    return ((u + 1) * nsh + total - 1) // total - 1


@dataclasses.dataclass
class Segment:
    seq: int
    g: int
    tile0: int        # absolute tile index (from position 0) of the first tile
    n: int            # tiles
    start: int        # index in the run's tile list
    flags: int        # PIECE_FIRST | PIECE_LAST | SHARE_FIRST
    pieces: int       # shares the pair spans (for a piece that starts its pair)


@dataclasses.dataclass
class Split:
    total: int
    nsh: int
    runs: list        # per wave: list of runs, each a list of Segment
    headers: list     # per wave: [slot0, slot1], each None or (seq, g, flags, pieces)


def model(lens, num_kv_heads: int, max_context_len: int, num_waves: int, seg_cap: int,
          window: int = 0, min_split_tiles: int = 8) -> Split:
    """The split every wave of a launch with ``num_waves`` workgroups computes."""
    N, Hkv = len(lens), num_kv_heads
    T = [min(max(int(t), 0), max_context_len) for t in lens]
    u = [pair_units(t, window) for t in T]
    P = [0]
    for x in u:
        P.append(P[-1] + x)
    total = Hkv * P[N]
    want = (total + min_split_tiles - 1) // min_split_tiles
    nsh = max(1, min(num_waves, want))
    runs, headers = [], []
    for w in range(num_waves):
        lo, hi = ((share_lo(total, w, nsh), share_lo(total, w + 1, nsh))
                  if w < nsh and total > 0 else (0, 0))
        first_seq = sum(1 for s in range(N) if Hkv * P[s] <= lo) - 1
        pos, s_cur = lo, max(first_seq, 0)
        wave_runs = []
        hdr = [None, None]
        while pos < hi:
            # every lane's segments, in lane order
            found = []            # (seq, g, t0, t1, pair start unit)
            for j in range(WAVE):
                s = s_cur + j
                if s >= N:
                    break
                beg, us = Hkv * P[s], u[s]
                a0, a1 = max(pos, beg), min(hi, beg + Hkv * us)
                if us == 0 or a0 >= a1:
                    continue
                g_first = (a0 - beg) // us
                g_last = (a1 - 1 - beg) // us
                if a1 - (beg + g_last * us) <= PAIR_COST:
                    g_last -= 1
                for g in range(g_first, g_last + 1):
                    ps = beg + g * us
                    t0 = max(0, pos - ps - PAIR_COST)
                    t1 = min(hi, ps + us) - ps - PAIR_COST
                    found.append((s, g, t0, t1, ps))
            nseg = min(len(found), seg_cap)
            if nseg == 0:
                s_next = s_cur + WAVE
                if s_next >= N:
                    break
                pos = max(pos, Hkv * P[s_next])
                s_cur = s_next
                continue
            run, start = [], 0
            for slot, (s, g, t0, t1, ps) in enumerate(found[:nseg]):
                flags = (PIECE_FIRST if t0 == 0 else 0) | (PIECE_LAST if t1 == u[s] - PAIR_COST else 0)
                if slot == 0 and pos == lo:
                    flags |= SHARE_FIRST
                pieces = (share_of(total, ps + u[s] - 1, nsh) - w + 1
                          if flags & 3 == PIECE_FIRST else 1)
                run.append(Segment(s, g, window_first(T[s], window) // TILE + t0, t1 - t0, start,
                                   flags, pieces))
                start += t1 - t0
            if len(found) > nseg:
                s_last, _, _, t1_last, ps_last = found[nseg - 1]
                run_end, run_seq = ps_last + PAIR_COST + t1_last, s_last
            else:
                run_end = min(hi, Hkv * P[s_cur + WAVE]) if s_cur + WAVE < N else hi
                run_seq = None
            share_done = run_end >= hi
            # pieces: the share's first segment goes to slot 0, its last to slot 1
            ntot = start
            for seg in run:
                if seg.flags & 3 == 3:
                    continue
                last_tile = seg.start + seg.n == ntot
                slot = 0 if (seg.flags & SHARE_FIRST) else 1
                if not (seg.flags & SHARE_FIRST) and not (share_done and last_tile):
                    raise AssertionError(f"wave {w}: a piece in the middle of a share")
                assert hdr[slot] is None, f"wave {w}: slot {slot} written twice"
                hdr[slot] = (seg.seq, seg.g, seg.flags & 3, seg.pieces)
            wave_runs.append(run)
            pos = run_end
            s_cur = run_seq if len(found) > nseg else min(N, s_cur + WAVE)
        runs.append(wave_runs)
        headers.append(hdr)
    return Split(total, nsh, runs, headers)
