"""Pins for the oracle's in-place retime, Rolling Sink, Infinity-RoPE and Deep-Forcing drivers (CPU only)."""
import math

import numpy as np
import pytest

from oracle import (DeepForcingRun, InfinityRopeRun, OracleCache, RollingSinkRun, SlidingWindowRun,
                    attention_f32, attention_f64, attention_loops_f64, attention_mass_scores, bf16_ulp,
                    roll_index, rotate_f64, round_to_bf16, row_normalisers)
from workloads import WORKLOADS, Workload, chunk_inputs


def _pair_ulp(x):
    """bf16 ulp of each (2p, 2p+1) pair's norm, broadcast to both components: a rotation mixes the
    pair, so its rounding error scales with the pair magnitude, not with each component."""
    x = np.asarray(x, np.float64)
    r = np.sqrt(x[..., 0::2] ** 2 + x[..., 1::2] ** 2)
    u = bf16_ulp(r)
    return np.repeat(u, 2, axis=-1)


def _rel_rms(a, b):
    return float(np.sqrt(np.sum((a - b) ** 2) / np.sum(b ** 2)))


def _fill(c, n_chunks, F=1, seed=0, t_start=0):
    rng = np.random.default_rng(seed)
    for j in range(n_chunks):
        N = F * c.S
        k = rng.standard_normal((N, c.H, c.D)).astype(np.float32)
        v = rng.standard_normal((N, c.H, c.D)).astype(np.float32)
        if c.dtype == "bf16":
            k, v = round_to_bf16(k), round_to_bf16(v)
        c.append(k, v, F, t_start + j * F)


# ---------------------------------------------------------------- retime (storage model)
def test_retime_zero_is_identity():
    c = OracleCache(1, 4, 6, 2, 128, 3, "bf16")
    _fill(c, 5)
    K0 = c.K.copy()
    c.retime(0, False)
    assert np.array_equal(c.K.view(np.uint32), K0.view(np.uint32))
    c.retime(-3, True, 0, 6)      # t = 0 there: the clamp leaves these entries unchanged
    assert np.array_equal(c.K[:6].view(np.uint32), K0[:6].view(np.uint32))


def test_retime_roundtrip_within_two_ulp():
    c = OracleCache(1, 4, 6, 2, 128, 3, "bf16")
    _fill(c, 5, t_start=40)
    K0 = c.K.copy()
    c.retime(17, False)
    c.retime(-17, False)
    err = np.abs(c.K[:, :, :44].astype(np.float64) - K0[:, :, :44])
    assert np.all(err <= 2 * _pair_ulp(K0[:, :, :44]))
    assert np.array_equal(c.K[:, :, 44:], K0[:, :, 44:])
    assert np.array_equal(c.t, np.repeat(np.arange(40, 45), 6))


def test_retime_equals_fresh_rotation_within_rounding_bound():
    # semantic reference: the raw key rotated from scratch at the new time, in fp64
    for dtype in ("f32", "bf16"):
        c = OracleCache(1, 4, 6, 2, 128, 3, dtype)
        _fill(c, 5, t_start=10)
        r = 0
        for d in (-3, 5, -11):
            c.retime(d, False)
            r += 1
        tok = c.tok
        fresh = rotate_f64(c.Kraw, c.t, tok // 3, tok % 3)
        err = np.abs(c.K.astype(np.float64) - fresh)
        if dtype == "f32":
            assert err.max() < 1e-2 and err.max() < 1e-5
        else:
            assert np.all(err <= (r + 1) * _pair_ulp(fresh) + 1e-6)


def test_clamp_composes_for_negative_deltas():
    rng = np.random.default_rng(0)
    t = rng.integers(0, 40, 1000)
    for d1, d2 in [(-3, -5), (-24, -3), (0, -7), (-40, -1)]:
        a = np.maximum(0, np.maximum(0, t + d1) + d2)
        b = np.maximum(0, t + d1 + d2)
        assert np.array_equal(a, b)
    # the oracle's t state follows the same composition
    c1 = OracleCache(1, 4, 6, 1, 64, 3, "f32")
    c2 = OracleCache(1, 4, 6, 1, 64, 3, "f32")
    _fill(c1, 5, t_start=2)
    _fill(c2, 5, t_start=2)
    c1.retime(-3, True)
    c1.retime(-2, True)
    c2.retime(-5, True)
    assert np.array_equal(c1.t, c2.t)


def test_uniform_retime_leaves_attention_unchanged():
    # relative invariance: shifting every key and the queries by the same delta
    c = OracleCache(1, 4, 6, 2, 64, 3, "f32")
    _fill(c, 5, t_start=3)
    q = np.random.default_rng(9).standard_normal((6, 2, 64)).astype(np.float32)
    a = c.attend(q, 1, 7, f64=True)
    c.retime(11, False)
    b = c.attend(q, 1, 18, f64=True)
    assert np.max(np.abs(a - b)) < 1e-5


# ---------------------------------------------------------------- Rolling Sink
def test_roll_order_forward_then_reverse():
    # "even cycles forward, odd cycles reverse" over K = 6 blocks
    seq = [roll_index(n, 6) for n in range(18)]
    assert seq == [0, 1, 2, 3, 4, 5, 5, 4, 3, 2, 1, 0, 0, 1, 2, 3, 4, 5]


def _rs_small(n_chunks=16):
    base = WORKLOADS["c4"]
    return Workload("c4_small", 103, 2, 64, "bf16", 2, 3, base.sink_frames, base.window_frames,
                    (3,) * n_chunks, base.bank_frames)


def test_rolling_sink_context_and_sliding_indices():
    w = _rs_small(16)
    run = RollingSinkRun(w)
    S = w.frame_seqlen
    raw = {}
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        raw[i] = (k, v)
        run.step(i, q, k, v)
        c = run.cache
        if i >= 6:
            assert c.n == 21 * S                              # K + 1 blocks of 3 frames every step
            # sink time indices slide: [3(i-6), 3(i-1))
            assert np.array_equal(np.unique(c.t[:15 * S]), np.arange(3 * (i - 6), 3 * (i - 1)))
            # explicit-concatenation rebuild: Cat(Roll(bank)[i-6 .. i-2] at 3(i-6).., block i-1, block i)
            parts_k, parts_v, parts_t = [], [], []
            for n in range(i - 6, i - 1):
                b = roll_index(n, 6) if i >= 7 else n
                kb, vb = raw[b]
                parts_k.append((kb, 3 * n)), parts_v.append(vb)
            for b in (i - 1, i):
                kb, vb = raw[b]
                parts_k.append((kb, 3 * b)), parts_v.append(vb)
            Kexp = []
            for kb, t0 in parts_k:
                tok = np.arange(kb.shape[0]) % S
                Kexp.append(round_to_bf16(
                    __import__("oracle").rotate_f32(kb, t0 + np.arange(kb.shape[0]) // S, tok // w.grid_w,
                                                    tok % w.grid_w)))
            assert np.array_equal(c.K.view(np.uint32), np.concatenate(Kexp).view(np.uint32))
            assert np.array_equal(c.V, np.concatenate(parts_v))


def test_rolling_sink_equals_plain_window_at_bank_fill():
    # at i = K and i = K + 1 the Rolling Sink context is a plain cache of the last 7 blocks
    w = _rs_small(8)
    rs = RollingSinkRun(w)
    plain_w = Workload("plain", 103, 2, 64, "bf16", 2, 3, 0, 21, (3,) * 8)
    plain = SlidingWindowRun(plain_w)
    for i in range(8):
        q, k, v = chunk_inputs(w, i)
        rs.step(i, q, k, v)
        plain.step(i, q, k, v)
        if i in (6, 7):
            a, b = rs.cache, plain.cache
            m = 21 * w.frame_seqlen
            assert np.array_equal(a.K.view(np.uint32), b.K[-m:].view(np.uint32))
            assert np.array_equal(a.t, b.t[-m:])


# ---------------------------------------------------------------- Infinity-RoPE
def _ir_small():
    base = WORKLOADS["c5a"]
    return Workload("c5a_small", 104, 2, 64, "bf16", 2, 3, base.sink_frames, base.window_frames,
                    (3,) * 12 + (2,), cut_chunks=(7, 10))


def test_infinity_rope_horizon_flush_and_cut():
    w = _ir_small()
    run = InfinityRopeRun(w)
    S = w.frame_seqlen
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        run.step(i, q, k, v)
        c = run.cache
        F = w.chunk_frames[i]
        assert c.t.min() >= 0 and c.t.max() < 21                 # inside the trained horizon
        assert np.array_equal(c.t[-F * S:], np.repeat(np.arange(21 - F, 21), S))
        if i in w.cut_chunks:
            assert c.n == 3 * S + 3 * S + F * S                   # sink + last block, then the new block
            assert np.all(c.t[:-F * S] == 0)                       # cut: old content clamps to 0
        assert c.n <= c.C_tok


def test_infinity_rope_matches_absolute_time_before_first_clamp():
    # before any clamp, Infinity-RoPE is a uniform time shift of the absolute-time run
    w = _ir_small()
    ir = InfinityRopeRun(w)
    ab = SlidingWindowRun(w)
    for i in range(6):
        q, k, v = chunk_inputs(w, i)
        a = ir.step(i, q, k, v, f64=True)
        b = ab.step(i, q, k, v, f64=True)
        assert np.array_equal(ir.cache.t - ir.cache.t[0], ab.cache.t - ab.cache.t[0])
        assert np.max(np.abs(a - b)) < 2e-2 and _rel_rms(a, b) < 5e-3


# ---------------------------------------------------------------- Deep Forcing
def test_scores_sum_and_brute_force():
    rng = np.random.default_rng(4)
    qh = rng.standard_normal((7, 2, 64))
    K = rng.standard_normal((19, 2, 64))
    s = attention_mass_scores(qh, K)
    assert abs(s.sum() - 2 * 7) < 1e-10
    # brute force: column sums of the explicit softmax
    ref = np.zeros(19)
    for h in range(2):
        for i in range(7):
            e = [math.exp(float(np.dot(qh[i, h], K[j, h])) / 8.0) for j in range(19)]
            z = sum(e)
            for j in range(19):
                ref[j] += e[j] / z
    assert np.max(np.abs(s - ref)) < 1e-12


def test_row_normalisers_brute_force_and_scores():
    """log2 softmax normalisers against explicit sums of powers of two; with them, every row's
    probabilities sum to one and their column sums are the attention-mass scores."""
    rng = np.random.default_rng(5)
    qh = rng.standard_normal((7, 2, 64)) * 3.0
    K = rng.standard_normal((19, 2, 64)) * 3.0
    M = row_normalisers(qh, K)
    assert M.shape == (2, 7)
    c = math.log2(math.e) / 8.0
    for h in range(2):
        for i in range(7):
            z = sum(2.0 ** (c * float(np.dot(qh[i, h], K[j, h]))) for j in range(19))
            assert abs(M[h, i] - math.log2(z)) < 1e-10
    s = attention_mass_scores(qh, K)
    cols = np.zeros(19)
    for h in range(2):
        e = np.exp2(c * (qh[:, h, :] @ K[:, h, :].T) - M[h][:, None])
        assert np.allclose(e.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        cols += e.sum(axis=0)
    assert np.max(np.abs(cols - s)) < 1e-12


def _df_small(n=16):
    base = WORKLOADS["c5b"]
    return Workload("c5b_small", 105, 2, 64, "bf16", 2, 3, base.sink_frames, base.window_frames, (3,) * n)


def test_deep_forcing_keep_set_and_gap_closing():
    w = _df_small()
    run = DeepForcingRun(w)
    S = w.frame_seqlen
    prev_q = None
    compactions = 0
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        before = {n: getattr(run.cache, n).copy() for n in ("K", "V", "t", "g")}
        run.step(i, q, k, v, q_prev=prev_q)
        prev_q = q
        c = run.cache
        if run.last:
            compactions += 1
            keep, scores = run.last["keep"], run.last["scores"]
            n_old = before["t"].shape[0]
            assert abs(scores.sum() - w.heads * 3 * S) < 1e-4 * w.heads * 3 * S
            assert keep.shape[0] == 3 * S + 4 * S + 2 * S
            # top-C: every kept candidate scores at least as high as every dropped one
            cand = np.arange(3 * S, n_old - 2 * S)
            kept = np.intersect1d(cand, keep)
            dropped = np.setdiff1d(cand, keep)
            assert scores[kept].min() >= scores[dropped].max()
            # compaction is a gather of the kept entries (values and global ids)
            n_keep = keep.shape[0]
            assert np.array_equal(c.V[:n_keep], before["V"][keep])
            assert np.array_equal(c.g[:n_keep], before["g"][keep])
            # gaps closed: sink | compressed | tail are contiguous in time
            comp_t = c.t[3 * S:7 * S]
            tail_t = c.t[7 * S:9 * S]
            assert comp_t.max() == tail_t.min() - 1
            assert c.t[:3 * S].max() == comp_t.min() - 1
        assert c.n <= c.C_tok
    assert compactions == 3        # chunks 7, 11, 15


# ---------------------------------------------------------------- denoise loop over layers
def test_denoise_loop_state_equals_commit_only_run():
    """After each chunk's four sampling passes and the commit, a layer's cache equals a plain sliding-window
    cache that received only the commit passes (the re-writes leave no trace but the last one), and the
    layers stay independent."""
    from oracle import DenoiseLoopRun
    from workloads import denoise_inputs
    w = Workload("dn_small", 107, 2, 64, "bf16", 2, 3, 1, 4, (1, 2, 2, 2, 1, 2))
    run = DenoiseLoopRun(w, layers=2)
    plain = [OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
             for _ in range(2)]
    for i in range(w.n_chunks):
        for s in range(5):
            for layer in range(2):
                q, k, v = denoise_inputs(w, i, s, layer)
                run.step(i, layer, s, q, k, v)
        for layer in range(2):
            _, k, v = denoise_inputs(w, i, 4, layer)
            plain[layer].append(k, v, w.chunk_frames[i], w.chunk_start_frame(i))
            a, b = run.caches[layer], plain[layer]
            for name in ("K", "V", "t", "g"):
                assert np.array_equal(getattr(a, name), getattr(b, name)), (i, layer, name)
    assert not np.array_equal(run.caches[0].K, run.caches[1].K)
