"""The attention kernels' key-tile order (kvc_tiles.hpp), built for the host (CPU only).

Attention over a set of keys does not depend on the order they are visited in,
so the dense kernels visit each visible range's whole tiles first and its edge
tiles (a range's first tile when the range starts inside it, its last when it
ends inside it) last, and run the steps before the edges without mask code.
That is only correct if the order visits every tile of the logical sequence
exactly once, if the tiles it reports as whole really are whole, and if the
whole-tile lookup the pipelined steps use agrees with the general one wherever
those steps reach -- also for every part of a split-key launch.  The
block-causal kernels keep the logical order and count their mask-free steps in
closed form, checked here against the definition.  The key-part count of a
split launch (same header) is checked against its rule and against the split
buffers' size.
"""
import ctypes
import os

import numpy as np
import pytest

BN = 64


@pytest.fixture(scope="module")
def tiles():
    from rolling_kv_cache_amd import build as b
    if not os.path.exists(b.RING_LIB):
        b.build()
    lib = ctypes.CDLL(b.RING_LIB)
    i32 = ctypes.c_int32
    p32 = ctypes.POINTER(ctypes.c_int32)
    lib.kvr_tile_count.restype = i32
    lib.kvr_tile_count.argtypes = [i32, i32, i32, i32]
    lib.kvr_tile_order.restype = i32
    lib.kvr_tile_order.argtypes = [i32, i32, i32, i32, i32, i32, i32, p32, p32]
    lib.kvr_causal_clean_steps.restype = i32
    lib.kvr_causal_clean_steps.argtypes = [i32, i32, i32, i32, i32]
    return lib


def _order(lib, ranges, edges_last, first, count):
    out = np.zeros(max(count, 1), np.int32)
    whole = np.zeros(max(count, 1), np.int32)
    p32 = ctypes.POINTER(ctypes.c_int32)
    w = lib.kvr_tile_order(*ranges, edges_last, first, count, out.ctypes.data_as(p32), whole.ctypes.data_as(p32))
    assert w >= 0
    return out[:count], whole[:count], w


def _logical(lo0, n0, lo1, n1):
    """The logical tile sequence, with an empty range 0 replaced by range 1 (as the launch does)."""
    def tiles_of(lo, n):
        return list(range(lo // BN, (n + BN - 1) // BN)) if n > lo else []
    t0, t1 = tiles_of(lo0, n0), tiles_of(lo1, n1)
    if not t0:
        return [(0, t) for t in t1], ((lo1, n1), (0, 0))
    return [(0, t) for t in t0] + [(1, t) for t in t1], ((lo0, n0), (lo1, n1))


def _shapes(seed, n):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        lo0 = int(rng.choice([0, 0, rng.integers(0, 400)]))
        n0 = lo0 + int(rng.choice([0, rng.integers(1, 400), 64 * rng.integers(1, 6)]))
        lo1 = int(rng.choice([0, 0, rng.integers(0, 400)]))
        n1 = lo1 + int(rng.choice([0, rng.integers(1, 400), 64 * rng.integers(1, 6)]))
        yield lo0, n0, lo1, n1


def test_orders_are_permutations_with_whole_tiles_first(tiles):
    checked = 0
    for ranges in _shapes(1, 4000):
        nt = tiles.kvr_tile_count(*ranges)
        logical, rr = _logical(*ranges)
        assert nt == len(logical)
        if nt == 0:
            continue
        seq, whole, _ = _order(tiles, ranges, 0, 0, nt)
        assert [(x & 1, x >> 1) for x in seq] == logical, ranges            # logical order
        assert np.array_equal(seq, whole)                                     # no edges in logical order
        seq, whole, w = _order(tiles, ranges, 1, 0, nt)
        got = [(x & 1, x >> 1) for x in seq]
        assert sorted(got) == sorted(logical), ranges                         # every tile exactly once
        for k, (r, tile) in enumerate(got):
            lo, n = rr[r]
            valid, lead = n - tile * BN, lo - tile * BN
            assert valid > max(lead, 0), (ranges, k)                         # at least one visible key
            if k < w:
                assert valid >= BN and lead <= 0, (ranges, k)                # whole, no mask needed
                assert whole[k] == seq[k], (ranges, k)
        assert w >= nt - 4                                                    # at most two edges per range
        checked += 1
    assert checked > 3000


@pytest.mark.parametrize("kparts", [2, 3, 5, 8])
def test_split_parts_cover_the_sequence_and_keep_their_clean_steps_whole(tiles, kparts):
    """Part p of a split launch visits tiles [p*nt/k, (p+1)*nt/k) of the edges-last order; its mask-free
    steps (t = 0 .. clean - 1, clean = whole prefix - 2) read tiles t + 1 and t + 2 with the whole-tile
    lookup, which must name whole tiles."""
    for ranges in _shapes(2, 1500):
        nt = tiles.kvr_tile_count(*ranges)
        if nt < 4 * kparts:
            continue
        full, _, _ = _order(tiles, ranges, 1, 0, nt)
        _, rr = _logical(*ranges)
        seen = []
        for p in range(kparts):
            first, end = p * nt // kparts, (p + 1) * nt // kparts
            seq, whole, w = _order(tiles, ranges, 1, first, end - first)
            assert np.array_equal(seq, full[first:end])
            seen += list(seq)
            clean = max(0, w - 2)
            last = end - first - 1
            for t in range(0, clean - 1, 2):
                for s in (t, t + 1):
                    for it in (min(s + 1, last), min(s + 2, last)):
                        r, tile = int(whole[it]) & 1, int(whole[it]) >> 1
                        lo, n = rr[r]
                        assert whole[it] == seq[it] and n - tile * BN >= BN and lo - tile * BN <= 0
        assert sorted(seen) == sorted(full)


def test_causal_clean_steps_closed_form(tiles):
    """Block-causal: the tiles from tile 1 on that are whole and end before lim_lo, capped at nt - 1,
    against the definition walked tile by tile."""
    rng = np.random.default_rng(3)
    for _ in range(20000):
        n0 = int(rng.choice([rng.integers(1, 700), 64 * rng.integers(1, 10)]))
        n1 = int(rng.choice([0, rng.integers(1, 700), 64 * rng.integers(1, 10)]))
        nt0 = (n0 + BN - 1) // BN
        lim_lo = int(rng.integers(1, n0 + n1 + 1))
        hi = int(rng.integers(lim_lo, n0 + n1 + 1))
        nt = (hi + BN - 1) // BN if hi <= n0 else nt0 + (hi - n0 + BN - 1) // BN

        def qualifies(tt):
            lb, valid = (tt * BN, n0 - tt * BN) if tt < nt0 else (n0 + (tt - nt0) * BN, n1 - (tt - nt0) * BN)
            return valid >= BN and lb + BN <= lim_lo
        c = 0
        while c + 1 < nt and qualifies(c + 1):
            c += 1
        assert tiles.kvr_causal_clean_steps(n0, n1, nt0, nt, lim_lo) == c, (n0, n1, nt, lim_lo)


def test_split_parts(tiles):
    """The key-part count of a split launch: 2..8 parts only when that fills the last round of 256 CUs
    better than the unsplit launch (by more than 2 %), each part holding at least four tiles, and never
    more partial rows (parts x workgroups x 256) than the split buffers hold (512 x 256)."""
    tiles.kvr_split_parts.restype = ctypes.c_int32
    tiles.kvr_split_parts.argtypes = [ctypes.c_int32, ctypes.c_int32]

    def fill(w):
        return w / (256.0 * ((w + 255) // 256))
    for total in range(1, 256):
        for ntiles in (1, 4, 7, 8, 16, 31, 32, 100, 439, 561):
            k = tiles.kvr_split_parts(total, ntiles)
            assert 1 <= k <= 8
            if k == 1:
                continue
            assert k * 4 <= ntiles and k * total * 256 <= 512 * 256, (total, ntiles, k)
            assert fill(k * total) > fill(total) + 0.02, (total, ntiles, k)
            allowed = [kp for kp in range(2, 9) if kp * 4 <= ntiles and kp * total * 256 <= 512 * 256]
            assert fill(k * total) >= max(fill(kp * total) for kp in allowed) - 0.02, (total, ntiles, k)
    assert tiles.kvr_split_parts(95, 439) == 5        # one GPU's 5-head share of the C3 layer
    assert tiles.kvr_split_parts(228, 561) == 1       # 12 heads x 19 blocks: as full unsplit as split
