"""The decode stream kernel's work split, replayed on the CPU.

tests/split_model.py restates the kernel's integer planning (equal shares,
lane-parallel segment search, runs of at most seg_cap segments, piece flags
and headers).  These tests check on many batches that:

* every attended tile of every (sequence, kv head) pair is handled exactly
  once, and no segment reaches a tile outside [first attended tile, ceil(T/16)),
  so no block-table index is negative or past the sequence's blocks;
* every run the kernel streams holds at least one segment with at least one
  tile (the kernel never builds descriptors for an empty run);
* a pair cut by share boundaries leaves exactly the pieces the merge kernel
  reads: its first piece (slot 0 or 1) in the share holding its first tile,
  recording how many shares it spans, then slot 0 of each following share,
  with the first/last flags at the ends;
* the share bounds cover [0, total) in order, and share_of inverts them.
"""
import bisect

import numpy as np
import pytest

import split_model as M


def check(lens, hkv, max_len, waves, cap, window=0):
    sp = M.model(lens, hkv, max_len, waves, cap, window)
    T = [min(max(int(t), 0), max_len) for t in lens]
    ranges = {}
    for w, runs in enumerate(sp.runs):
        for run in runs:
            assert run and all(seg.n >= 1 for seg in run), f"wave {w}: empty run"
            ntot = 0
            for seg in run:
                assert seg.start == ntot
                ntot += seg.n
                t = T[seg.seq]
                lo_tile = M.window_first(t, window) // M.TILE
                hi_tile = (t + M.TILE - 1) // M.TILE
                assert lo_tile <= seg.tile0 and seg.tile0 + seg.n <= hi_tile, (w, seg, t)
                ranges.setdefault((seg.seq, seg.g), []).append((seg.tile0, seg.n, w, seg.flags,
                                                                seg.pieces))
    for s, t in enumerate(T):
        tiles = M.attended_tiles(t, window)
        for g in range(hkv):
            got = sorted(ranges.get((s, g), []))
            if tiles == 0:
                assert not got
                continue
            pos = M.window_first(t, window) // M.TILE
            for (t0, n, _, _, _) in got:
                assert t0 == pos, (s, g, got)
                pos += n
            assert pos == (t + M.TILE - 1) // M.TILE
            if len(got) == 1:
                assert got[0][3] & 3 == 3
                continue
            # pieces: consecutive shares, first/last flags at the ends
            waves_of = [r[2] for r in got]
            assert waves_of == list(range(waves_of[0], waves_of[0] + len(got)))
            assert got[0][3] & 3 == M.PIECE_FIRST and got[-1][3] & 3 == M.PIECE_LAST
            assert all(r[3] & 3 == 0 for r in got[1:-1])
            assert got[0][4] == len(got)
            w0 = waves_of[0]
            first_hdr = [h for h in sp.headers[w0] if h and h[:2] == (s, g)]
            assert first_hdr == [(s, g, M.PIECE_FIRST, len(got))]
            for w in waves_of[1:]:
                h0 = sp.headers[w][0]
                assert h0 is not None and h0[:2] == (s, g), (s, g, w, sp.headers[w])
    bounds = [M.share_lo(sp.total, w, sp.nsh) for w in range(sp.nsh + 1)]
    assert bounds[0] == 0 and bounds[-1] == sp.total and bounds == sorted(bounds)
    return sp


def lognormal_lens(n, seed):
    rng = np.random.default_rng(seed)
    sigma = np.log(735 / 260) / 1.645
    mu = np.log(400) - sigma ** 2 / 2
    return np.clip(np.rint(rng.lognormal(mu, sigma, n)), 1, 4096).astype(int).tolist()


CASES = {
    "llama3-8b": (lambda: lognormal_lens(256, 3), 8, 4096, 2048, 4),
    "llama3-8b-cap1": (lambda: lognormal_lens(256, 4), 8, 4096, 2048, 1),
    "llama2-7b": (lambda: [4096] * 64, 32, 4096, 2048, 6),
    "qwen2-0.5b": (lambda: np.random.default_rng(2).integers(1, 4097, 32).tolist(), 2, 4096, 2048, 6),
    "prefix-70b": (lambda: (1801 + np.random.default_rng(5).integers(0, 513, 12)).tolist(), 8, 2400, 2048, 2),
    # short contexts: many segments per share (the case a run could end with none)
    "short-251": (lambda: np.random.default_rng(251).integers(1, 33, 251).tolist(), 8, 32, 2048, 4),
    "short-251-cap2": (lambda: np.random.default_rng(252).integers(1, 33, 251).tolist(), 8, 32, 2048, 2),
    "short-1024": (lambda: np.random.default_rng(9).integers(0, 20, 1024).tolist(), 4, 32, 1792, 6),
    "zeros-and-ones": (lambda: [0, 1, 0, 0, 17, 0, 1, 16, 0, 33] * 20, 2, 64, 512, 3),
    "all-zero": (lambda: [0] * 70, 8, 16, 2048, 4),
    # one huge sequence among 1000 tiny ones: shares hold over 64 sequences
    "huge-and-tiny": (lambda: [200_000] + [1, 2, 3] * 333, 1, 200_000, 2048, 6),
    "odd-wave-count": (lambda: lognormal_lens(97, 7), 8, 4096, 13, 4),
    "one-wave": (lambda: lognormal_lens(20, 8), 4, 4096, 1, 4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_split_covers_every_tile_once(name):
    make, hkv, max_len, waves, cap = CASES[name]
    check(make(), hkv, max_len, waves, cap)


@pytest.mark.parametrize("window", [1, 17, 256, 4096])
def test_split_with_sliding_window(window):
    check(lognormal_lens(256, 30 + window), 8, 4096, 2048, 4, window=window)
    check(np.random.default_rng(window).integers(0, 700, 200).tolist(), 2, 700, 333, 2,
          window=window)


def test_share_of_inverts_the_bounds():
    for total, nsh in [(1000, 7), (55_400, 2048), (1 << 30, 4096), (17, 1)]:
        bounds = [M.share_lo(total, w, nsh) for w in range(nsh + 1)]
        for u in list(range(0, min(total, 2000))) + [total - 1, total // 2]:
            w = M.share_of(total, u, nsh)
            assert bounds[w] <= u < bounds[w + 1]
            assert w == bisect.bisect_right(bounds, u) - 1


def test_shares_differ_by_at_most_one_unit():
    for total, nsh in [(55_400, 2048), (1000, 7), (2048 * 5 + 3, 2048)]:
        sizes = np.diff([M.share_lo(total, w, nsh) for w in range(nsh + 1)])
        assert sizes.max() - sizes.min() <= 1 and sizes.sum() == total
