"""Host-only build of the ring planner fuzzed against the oracle's cache state machine (CPU only).

The GPU library's index arithmetic (sink/window rings, FIFO eviction by head
advance, replace-newest, retime ranges, compaction, Rolling-Sink push) must
yield, in logical order, exactly the (t, g) sequence the oracle gets with
explicit concatenation and a physical left shift, and reject exactly the
same calls.
"""
import ctypes
import os

import numpy as np
import pytest

from oracle import OracleCache, OracleError


@pytest.fixture(scope="module")
def ring():
    from rolling_kv_cache_amd import build as b
    if not os.path.exists(b.RING_LIB):
        b.build()
    lib = ctypes.CDLL(b.RING_LIB)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    p32 = ctypes.POINTER(ctypes.c_int32)
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.kvr_new.restype = vp
    lib.kvr_new.argtypes = [i32, i32, i32]
    lib.kvr_free.argtypes = [vp]
    lib.kvr_append.restype = i32
    lib.kvr_append.argtypes = [vp, i32, i32, i32, p32, i32]
    lib.kvr_sink_push.restype = i32
    lib.kvr_sink_push.argtypes = [vp, i32, i32, i32]
    lib.kvr_retime.restype = i32
    lib.kvr_retime.argtypes = [vp, i32, i32, i32, i32]
    lib.kvr_compact.restype = i32
    lib.kvr_compact.argtypes = [vp, p32, i32]
    lib.kvr_counters.argtypes = [vp, p64]
    lib.kvr_logical.argtypes = [vp, p32, p64]
    lib.kvr_physical.argtypes = [vp, p32, p32]
    return lib


class Ring:
    def __init__(self, lib, S, sink_tok, win_tok):
        self.lib = lib
        self.p = lib.kvr_new(S, sink_tok, win_tok)
        self.W = win_tok
        self.Stok = sink_tok

    def counters(self):
        c = np.zeros(9, np.int64)
        self.lib.kvr_counters(self.p, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return c

    def logical(self):
        n = int(self.counters()[0])
        t = np.zeros(max(n, 1), np.int32)
        g = np.zeros(max(n, 1), np.int64)
        self.lib.kvr_logical(self.p, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                             g.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return t[:n], g[:n]

    def append(self, F, t0, replace):
        segs = np.zeros(64, np.int32)
        r = self.lib.kvr_append(self.p, F, t0, int(replace), segs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 16)
        return r, segs[:4 * max(r, 0)].reshape(-1, 4)


def _both(fn_oracle, fn_ring):
    try:
        fn_oracle()
        ok_o = True
    except OracleError:
        ok_o = False
    ok_r = fn_ring() >= 0
    assert ok_o == ok_r
    return ok_o


@pytest.mark.parametrize("seed", range(12))
def test_ring_matches_oracle_state_machine(ring, seed):
    rng = np.random.default_rng(seed)
    S = int(rng.choice([2, 3, 4]))
    sink_f = int(rng.integers(0, 3))
    win_f = int(rng.integers(3, 7))
    oc = OracleCache(sink_f, win_f, S, 1, 64, 1 if S < 2 else S // (2 if S % 2 == 0 else 1), "f32",
                     bank_frames=sink_f)
    rr = Ring(ring, S, sink_f * S, win_f * S)
    try:
        for step in range(120):
            op = rng.choice(["append", "append", "append", "replace", "retime", "compact", "push"])
            if op in ("append", "replace"):
                F = int(rng.integers(1, win_f + 2))
                t0 = int(rng.integers(0, 300))
                z = np.zeros((F * S, 1, 64), np.float32)
                _both(lambda: oc.append(z, z, F, t0, replace_newest=(op == "replace")),
                      lambda: rr.append(F, t0, op == "replace")[0])
            elif op == "retime" and oc.n > 0:
                lo = int(rng.integers(0, oc.n + 1))
                hi = int(rng.integers(lo, oc.n + 1)) if rng.random() < 0.9 else oc.n + 1
                d = int(rng.integers(-40, 41))
                cl = bool(rng.integers(0, 2))
                _both(lambda: oc.retime(d, cl, lo, hi), lambda: ring.kvr_retime(rr.p, d, int(cl), lo, hi))
            elif op == "compact" and oc.n > 0:
                keep = np.arange(oc.n_sink)
                rest = np.arange(oc.n_sink, oc.n)
                sel = rest[rng.random(rest.shape[0]) < 0.6]
                keep = np.concatenate([keep, sel]).astype(np.int32)
                if rng.random() < 0.15 and keep.shape[0] > 1:
                    keep = keep[1:]                           # drops a sink entry (or is empty of it)
                if keep.shape[0] == 0:
                    continue
                _both(lambda: oc.compact(keep),
                      lambda: ring.kvr_compact(rr.p, keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                               keep.shape[0]))
            elif op == "push" and sink_f > 0 and oc.global_end >= oc.bank_tok:
                F = int(rng.integers(1, sink_f + 1))
                bf = int(rng.integers(0, sink_f - F + 1))
                t0 = int(rng.integers(0, 300))
                _both(lambda: oc.sink_push(bf, F, t0), lambda: ring.kvr_sink_push(rr.p, F, bf * S, t0))
            t, g = rr.logical()
            assert np.array_equal(t, oc.t), (step, op)
            assert np.array_equal(g, oc.g), (step, op)
            c = rr.counters()
            assert c[0] == oc.n and c[1] == oc.n_sink and c[8] == oc.global_end
            # invariants: a partly filled region is a prefix of its physical slots
            if c[1] < sink_f * S:
                assert c[2] == 0 and c[3] == 0
            if c[3] < win_f * S:
                assert c[4] == 0
    finally:
        ring.kvr_free(rr.p)


def test_append_segments_wrap_and_straddle(ring):
    # sink 2 frames of 4 tokens, window 5 frames: a 3-frame chunk straddles sink/window,
    # and eviction wraps the window ring
    rr = Ring(ring, 4, 8, 20)
    r, segs = rr.append(3, 0, False)
    assert r == 2 and segs.tolist() == [[0, 0, 0, 8], [1, 0, 8, 4]]
    r, segs = rr.append(3, 3, False)
    assert segs.tolist() == [[1, 4, 0, 12]]
    r, segs = rr.append(3, 6, False)                    # window 16 + 12 > 20: evict 8, head 8
    assert segs.tolist() == [[1, 16, 0, 4], [1, 0, 4, 8]]
    c = rr.counters()
    assert c[3] == 20 and c[4] == 8
    r, segs = rr.append(3, 6, True)                     # replace newest: same slots, no eviction
    assert segs.tolist() == [[1, 16, 0, 4], [1, 0, 4, 8]] and rr.counters()[4] == 8
    assert rr.append(6, 9, False)[0] == -1              # chunk larger than the window
    ring.kvr_free(rr.p)
