"""The product's policy drivers (rolling_kv_cache_amd/policies.py) against the oracle's policy runs, on the CPU.

The drivers only decide which library calls to make (append times, retime deltas and ranges, flush and
keep sets, sink pushes).  Here they drive a stand-in cache whose index state is the host-only build of the
library's ring planner (the same C++ as libkvc) and whose scores come from an oracle cache fed the same
calls; the oracle's own runs (oracle/policies.py, written separately) step beside them.  After every
chunk the planner's logical (t, g) sequence must equal the oracle run's, and where entries are scored the
two keep sets must be the same.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import OracleCache, make_run
from workloads import WORKLOADS, Workload, chunk_inputs


@pytest.fixture(scope="module")
def ring():
    from rolling_kv_cache_amd import build as b
    if not os.path.exists(b.RING_LIB):
        b.build()
    lib = ctypes.CDLL(b.RING_LIB)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    p32, p64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
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
    lib.kvr_error.restype = ctypes.c_char_p
    return lib


class PlannerCache:
    """The subset of KVCache the policy drivers use: index state from the ring planner, scores from an
    oracle cache that receives the same calls, attention a no-op."""

    def __init__(self, lib, w):
        self.lib, self.w = lib, w
        self.S, self.H, self.D = w.frame_seqlen, w.heads, w.head_dim
        self.device = torch.device("cpu")
        self.S_tok, self.W_tok = w.sink_frames * self.S, w.window_frames * self.S
        self.p = lib.kvr_new(self.S, self.S_tok, self.W_tok)
        self.oc = OracleCache(w.sink_frames, w.window_frames, self.S, w.heads, w.head_dim, w.grid_w, w.dtype,
                              w.bank_frames)

    def close(self):
        self.lib.kvr_free(self.p)

    def _ok(self, r, what):
        assert r >= 0, f"{what}: {self.lib.kvr_error().decode()}"

    def counters(self):
        c = np.zeros(9, np.int64)
        self.lib.kvr_counters(self.p, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return c

    def info(self):
        c = self.counters()
        return {"n_valid": int(c[0]), "capacity": self.S_tok + self.W_tok, "sink_tokens": self.S_tok,
                "sink_filled": int(c[1]), "newest_frames": int(c[7]), "global_end": int(c[8])}

    def slot_times(self):
        n = int(self.counters()[0])
        t = np.zeros(max(n, 1), np.int32)
        g = np.zeros(max(n, 1), np.int64)
        self.lib.kvr_logical(self.p, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                             g.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return t[:n], g[:n]

    def append(self, k, v, t_index, replace_newest=False):
        F = k.shape[0] // self.S
        segs = np.zeros(64, np.int32)
        self._ok(self.lib.kvr_append(self.p, F, int(t_index), int(replace_newest),
                                     segs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 16), "append")
        self.oc.append(k.numpy(), v.numpy(), F, int(t_index), replace_newest=replace_newest)

    def attend(self, q, t_index=None, out=None, row_stats=None):
        return None

    def retime(self, delta, clamp0=False, lo=0, hi=None):
        hi = self.info()["n_valid"] if hi is None else hi
        self._ok(self.lib.kvr_retime(self.p, int(delta), int(clamp0), int(lo), int(hi)), "retime")
        self.oc.retime(int(delta), bool(clamp0), int(lo), int(hi))

    def compact(self, keep):
        keep = np.ascontiguousarray(np.asarray(keep, np.int32))
        self._ok(self.lib.kvr_compact(self.p, keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      keep.shape[0]), "compact")
        self.oc.compact(keep.astype(np.int64))

    def sink_push(self, bank_frame, n_frames, t_index):
        self._ok(self.lib.kvr_sink_push(self.p, int(n_frames), int(bank_frame) * self.S, int(t_index)), "sink push")
        self.oc.sink_push(int(bank_frame), int(n_frames), int(t_index))

    def score(self, q_win, q_t, out=None, row_stats=None):
        F = q_win.shape[0] // self.S
        return torch.from_numpy(np.asarray(self.oc.score(q_win.numpy(), F, list(q_t)), np.float64))

    def relax_scores(self, tail_frames, weight=0.5, out=None):
        return torch.from_numpy(np.asarray(self.oc.relax_scores(tail_frames, weight), np.float64))


def _small(name, cfg_id, n_chunks, **kw):
    base = WORKLOADS[name]
    return Workload(f"{name}_host", cfg_id, 2, 64, "bf16", 4, 8, base.sink_frames, base.window_frames,
                    (3,) * n_chunks, kw.get("bank_frames", base.bank_frames), kw.get("cut_chunks", ()))


CASES = {
    "c3": _small("c3", 401, 12),
    "c4": _small("c4", 402, 16),
    "c5a": _small("c5a", 403, 14, cut_chunks=(5, 9)),
    "c5b": _small("c5b", 404, 16),
    "c5c": _small("c5c", 405, 16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_policy_driver_matches_oracle_run(ring, name):
    from rolling_kv_cache_amd.policies import driver_for
    w = CASES[name]
    fake = PlannerCache(ring, w)
    drv = driver_for(w.name)(fake, w)
    run = make_run(w)
    q_prev = q_prev_t = None
    scored = 0
    try:
        for i in range(w.n_chunks):
            q, k, v = chunk_inputs(w, i)
            qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
            drv.step(i, qt, kt, vt, q_prev=q_prev_t)
            run.step(i, q, k, v, q_prev=q_prev, rows=np.arange(1)) if name == "c5b" else \
                run.step(i, q, k, v, rows=np.arange(1))
            t, g = fake.slot_times()
            assert np.array_equal(g, run.cache.g), f"{name} chunk {i}: g"
            assert np.array_equal(t, run.cache.t), f"{name} chunk {i}: t"
            assert fake.info()["sink_filled"] == run.cache.n_sink
            if getattr(run, "last", None) and "keep" in run.last:
                assert np.array_equal(np.asarray(drv.last["keep"], np.int64), np.asarray(run.last["keep"], np.int64))
                assert (drv.last["d_c"], drv.last["d_s"]) == (run.last["d_c"], run.last["d_s"])
                scored += 1
            q_prev, q_prev_t = q, qt
    finally:
        fake.close()
    if name in ("c5b", "c5c"):
        assert scored >= 2, "the stream should compact at least twice"
