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


# ---------------------------------------------------------------- MemRoPE memory tokens
def _mem_cache(alphas, n_chunks, F=1, S=6, H=2, D=64, sink=1, window=3, seed=5, raw_keys=True):
    c = OracleCache(sink, window, S, H, D, 3, "bf16", raw_keys=raw_keys, memory=alphas)
    rng = np.random.default_rng(seed)
    ks, vs = [], []
    for j in range(n_chunks):
        k = round_to_bf16(rng.standard_normal((F * S, H, D)).astype(np.float32))
        v = round_to_bf16(rng.standard_normal((F * S, H, D)).astype(np.float32))
        c.append(k, v, F, j * F)
        ks.append(k)
        vs.append(v)
    return c, ks, vs


def test_memory_ema_closed_form():
    """After folding frames E_1..E_n: M = a^(n-1) E_1 + sum_{i>=2} (1-a) a^(n-i) E_i (fp64), within the
    rounding of n fp32 multiply-adds; memory exists only from the first eviction on."""
    c, _, _ = _mem_cache((0.9, 0.5), 4)               # capacity 4 frames: nothing evicted yet
    assert c.mem_frames == 0 and c.memory_entries() is None
    c, _, _ = _mem_cache((0.9, 0.5), 9)
    assert c.mem_frames == 5
    # the evicted frames are the window's frames 1..5 in order (frame 0 is the sink); their stored keys
    ref = OracleCache(1, 8, 6, 2, 64, 3, "bf16", raw_keys=True)
    rng = np.random.default_rng(5)
    for j in range(9):
        k = round_to_bf16(rng.standard_normal((6, 2, 64)).astype(np.float32))
        v = round_to_bf16(rng.standard_normal((6, 2, 64)).astype(np.float32))
        ref.append(k, v, 1, j)
    Ek = [ref.K[6 * f:6 * (f + 1)].astype(np.float64) for f in range(1, 6)]
    Ev = [ref.V[6 * f:6 * (f + 1)].astype(np.float64) for f in range(1, 6)]
    for m, a in enumerate((0.9, 0.5)):
        n = len(Ek)
        mk = a ** (n - 1) * Ek[0] + sum((1 - a) * a ** (n - i) * Ek[i - 1] for i in range(2, n + 1))
        mv = a ** (n - 1) * Ev[0] + sum((1 - a) * a ** (n - i) * Ev[i - 1] for i in range(2, n + 1))
        scale = max(np.max(np.abs(mk)), 1.0)
        assert np.max(np.abs(c.mem_k[m] - mk)) < 8 * n * 2.0 ** -24 * scale * 4
        assert np.max(np.abs(c.mem_v[m] - mv)) < 8 * n * 2.0 ** -24 * scale * 4
    assert not np.array_equal(c.mem_k[0], c.mem_k[1])


def test_memory_extreme_rates_are_exact():
    """alpha = 1 keeps the first evicted frame, alpha = 0 the last one, bit for bit."""
    c, _, _ = _mem_cache((1.0, 0.0), 9)
    ref = OracleCache(1, 8, 6, 2, 64, 3, "bf16", raw_keys=True)
    rng = np.random.default_rng(5)
    for j in range(9):
        k = round_to_bf16(rng.standard_normal((6, 2, 64)).astype(np.float32))
        v = round_to_bf16(rng.standard_normal((6, 2, 64)).astype(np.float32))
        ref.append(k, v, 1, j)
    assert np.array_equal(c.mem_k[0], ref.K[6:12]) and np.array_equal(c.mem_v[0], ref.V[6:12])
    assert np.array_equal(c.mem_k[1], ref.K[30:36]) and np.array_equal(c.mem_v[1], ref.V[30:36])


def test_memory_placement():
    """With alpha_short = 0 the short memory is the last evicted frame, and it is placed at t_w - 1, the time
    that frame had: its attended keys equal that frame's keys in a plain rotated cache with a larger window.
    With alpha_long = 1 the long memory is the first evicted frame, placed at t_w - 2: its keys equal that raw
    frame rotated freshly at t_w - 2."""
    c, ks, vs = _mem_cache((1.0, 0.0), 9)
    big = OracleCache(1, 8, 6, 2, 64, 3, "bf16")
    for j in range(9):
        big.append(ks[j], vs[j], 1, j)
    K, V, T = c.memory_entries()
    t_w = int(c.t[c.n_sink])
    assert t_w == 6 and np.all(T[:6] == 4) and np.all(T[6:] == 5)
    assert np.array_equal(K[6:], big.K[30:36]) and np.array_equal(V[6:], big.V[30:36])
    at = OracleCache(0, 1, 6, 2, 64, 3, "bf16")
    at.append(ks[1], vs[1], 1, t_w - 2)
    assert np.array_equal(K[:6], at.K) and np.array_equal(V[:6], at.V)


def test_memory_follows_uniform_shift():
    """A uniform retime of every entry moves the memory with the window (it is placed relative to the oldest
    window entry), so attention with queries shifted alike changes only by rounding."""
    c, _, _ = _mem_cache((0.9, 0.5), 9)
    rng = np.random.default_rng(9)
    q = round_to_bf16(rng.standard_normal((6, 2, 64)).astype(np.float32))
    a = c.attend(q, 1, 8, f64=True)
    c.retime(37, False)
    b = c.attend(q, 1, 45, f64=True)
    assert np.max(np.abs(a - b)) < 2e-2 and np.sqrt(np.mean((a - b) ** 2)) < 3e-3


def test_memory_needs_raw_keys_and_refuses_compaction():
    """MemRoPE memory is defined on a raw-key cache only, and not together with compaction, a
    Rolling-Sink push or block-causal attention (none of those pages combine them with memory)."""
    from oracle import OracleError
    import pytest as _pt
    with _pt.raises(OracleError):
        OracleCache(1, 3, 6, 2, 64, 3, "bf16", memory=(0.9, 0.5))
    c, _, _ = _mem_cache((0.9, 0.5), 6)
    with _pt.raises(OracleError):
        c.compact(np.arange(c.n))
    with _pt.raises(OracleError):
        c.sink_push(0, 1, 0)
    q = np.zeros((c.S, c.H, c.D), np.float32)
    with _pt.raises(OracleError):
        c.attend_block_causal(q, 1, 0, 1)
