"""Pins for the oracle's raw-key mode (the MemRoPE variant of the rCM length-extrapolation article: keys kept
un-rotated and placed at attention time).  CPU only.

What the mode must satisfy, checked against independent constructions: the stored key keeps the raw time band
and the same height/width bands as a fully rotated cache; before any retime its attention keys equal the rotated
cache's stored keys bit for bit; after any sequence of retimes they equal a cache built from scratch at the new
times (no accumulated rounding, unlike the in-place storage model); a retime never touches the stored keys."""
import numpy as np

from oracle import InfinityRopeRun, OracleCache, band_split, round_to_bf16
from workloads import Workload, chunk_inputs


def _pair(raw, n_chunks=5, F=2, S=6, H=2, D=64, sink=1, window=6, t0=0, dtype="bf16"):
    caches = [OracleCache(sink, window, S, H, D, 3, dtype, raw_keys=r) for r in (raw, False)]
    rng = np.random.default_rng(11)
    for j in range(n_chunks):
        k = rng.standard_normal((F * S, H, D)).astype(np.float32)
        v = rng.standard_normal((F * S, H, D)).astype(np.float32)
        if dtype == "bf16":
            k, v = round_to_bf16(k), round_to_bf16(v)
        for c in caches:
            c.append(k, v, F, t0 + j * F)
    return caches


def test_stored_form():
    raw, rot = _pair(True)
    (ts, tw), hb, wb = band_split(raw.D)
    assert np.array_equal(raw.K[:, :, ts:ts + tw], raw.Kraw[:, :, ts:ts + tw])          # time band raw
    assert np.array_equal(raw.K[:, :, tw:], rot.K[:, :, tw:])                            # h/w bands rotated
    assert not np.array_equal(raw.K[:, :, :tw], rot.K[:, :, :tw])


def test_attention_keys_equal_rotated_cache_before_retime():
    for dtype in ("bf16", "f32"):
        raw, rot = _pair(True, dtype=dtype)
        assert np.array_equal(raw.attention_keys(), rot.K)


def test_retime_is_index_only_and_exact():
    """Shift by +5, clamp-shift by -9, shift a sub-range by +3: the raw cache's attention keys equal a cache
    whose every entry was rotated once, from scratch, at its final time."""
    raw, _ = _pair(True, n_chunks=4)
    K0 = raw.K.copy()
    raw.retime(5, False)
    raw.retime(-9, True)
    raw.retime(3, False, 2, 10)
    assert np.array_equal(raw.K, K0)                       # stored keys untouched
    fresh = OracleCache(raw.S_tok // raw.S, raw.W_tok // raw.S, raw.S, raw.H, raw.D, raw.grid_w, raw.dtype)
    ref = fresh._rotate(raw.Kraw, raw.t, raw.tok)
    assert np.array_equal(raw.attention_keys(), ref)
    # the same schedule on the in-place storage model drifts by rounding but stays within a few ulp
    _, rot = _pair(True, n_chunks=4)
    rot.retime(5, False)
    rot.retime(-9, True)
    rot.retime(3, False, 2, 10)
    assert np.array_equal(rot.t, raw.t)
    assert np.max(np.abs(rot.K - ref)) > 0


def test_infinity_rope_raw_equals_absolute_time_rotation():
    """Infinity-RoPE (shift, clamp, flush, cut) on a raw cache: at every chunk the attention keys are the raw
    keys rotated once at their current times."""
    w = Workload("c5a_small", 104, 2, 64, "bf16", 2, 3, 3, 18, (3,) * 12, cut_chunks=(7,), raw_keys=True)
    run = InfinityRopeRun(w)
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        run.step(i, q, k, v)
        c = run.cache
        fresh = OracleCache(c.S_tok // c.S, c.W_tok // c.S, c.S, c.H, c.D, c.grid_w, c.dtype)
        assert np.array_equal(c.attention_keys(), fresh._rotate(c.Kraw, c.t, c.tok)), i
        assert np.array_equal(c.K[:, :, :band_split(c.D)[0][1]], c.Kraw[:, :, :band_split(c.D)[0][1]])


def test_time_band_rotation_of_stored_keys_is_the_full_rotation():
    """The identity the GPU path relies on: rotating only the stored time band (the height/width bands are
    already rotated) at the current time gives the full rotation of the raw key, bit for bit -- after
    arbitrary retimes, including clamps and times below zero."""
    from oracle import rotate_f32
    for dtype in ("bf16", "f32"):
        raw, _ = _pair(True, n_chunks=4, dtype=dtype)
        raw.retime(-3, False)
        raw.retime(-4, True, 0, 7)
        zero = np.zeros_like(raw.t)
        staged = raw._store(rotate_f32(raw.K, raw.t, zero, zero, bands=(True, False, False)))
        assert np.array_equal(staged, raw.attention_keys())
        assert np.min(raw.t) < 0                     # some entries sit before time 0
