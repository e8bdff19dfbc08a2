"""Pins for the Relax Forcing frame scores and policy of the oracle (rCM article, strategy 5).  CPU only.

The article fixes only the form score = w * alignment + (1 - w) * complement and the Top-K frame choice;
the pins below check the readings (frame vector = mean stored key, cosine, complement = 1 - mean cosine
to the other candidates) against hand-computed closed forms and invariants that a dropped term, a wrong
sign or a swapped operand would break."""
import math

import numpy as np
import pytest

from oracle import OracleCache, RelaxForcingRun, relax_frame_scores, top_frames, round_to_bf16
from workloads import WORKLOADS, Workload, chunk_inputs


def _cache(frames, S=4, H=2, D=64, sink=1, dtype="bf16", seed=3):
    c = OracleCache(sink, frames - sink, S, H, D, 2, dtype)
    rng = np.random.default_rng(seed)
    for f in range(frames):
        k = rng.standard_normal((S, H, D)).astype(np.float32)
        v = rng.standard_normal((S, H, D)).astype(np.float32)
        if dtype == "bf16":
            k, v = round_to_bf16(k), round_to_bf16(v)
        c.append(k, v, 1, f)
    return c


def test_hand_example():
    """One head of 8 dims, 2 tokens per frame; frame means A = e0, B = e1, C = e0 + e1 and a Tail whose two
    frames average to e0.  By hand: alignment (1, 0, 1/sqrt2); pairwise cosines AB = 0, AC = BC = 1/sqrt2,
    so complement (1 - 1/(2 sqrt2), 1 - 1/(2 sqrt2), 1 - 1/sqrt2)."""
    c = OracleCache(1, 5, 2, 1, 8, 2, "f32")
    for f in range(6):
        c.append(np.zeros((2, 1, 8), np.float32), np.zeros((2, 1, 8), np.float32), 1, f)
    e = np.eye(8)
    means = [e[5], e[0], e[1], e[0] + e[1], e[0] + e[2], e[0] - e[2]]   # sink, A, B, C, tail 1, tail 2
    K = np.zeros((12, 1, 8))
    for f, m in enumerate(means):
        K[2 * f, 0] = m + 0.5 * e[3]
        K[2 * f + 1, 0] = m - 0.5 * e[3]
    c.K = K.astype(np.float32)
    r = 1 / math.sqrt(2)
    align = np.array([1.0, 0.0, r])
    comp = np.array([1 - r / 2, 1 - r / 2, 1 - r])
    for w in (0.5, 0.25, 1.0, 0.0):
        assert np.allclose(c.relax_scores(2, w), w * align + (1 - w) * comp, rtol=0, atol=1e-15)


def test_gram_identity():
    """The same scores from inner products alone: <x, tail mean> is the mean of <x, tail frame t>, and
    |tail mean|^2 the mean of all <t, t'> -- a different computation of the same cosines."""
    c = _cache(9)
    S, n_cand, T = c.S, 6, 2
    X = np.asarray(c.K, np.float64).reshape(9, S, -1).sum(axis=1)        # frame sums
    G = X @ X.T
    cand = np.arange(1, 1 + n_cand)
    tail = np.arange(1 + n_cand, 9)
    tn = math.sqrt(G[np.ix_(tail, tail)].sum())
    ref = []
    for i in cand:
        align = G[i, tail].sum() / (math.sqrt(G[i, i]) * tn)
        cos = [G[i, j] / math.sqrt(G[i, i] * G[j, j]) for j in cand if j != i]
        ref.append(0.3 * align + 0.7 * (1 - sum(cos) / len(cos)))
    assert np.allclose(c.relax_scores(T, 0.3), ref, rtol=0, atol=1e-13)


def test_invariants():
    c = _cache(9)
    S = c.S
    base = c.relax_scores(2, 0.5)
    K0 = c.K.copy()
    # scaling a candidate frame, or the whole Tail, by a power of two (exact in bf16) changes no cosine
    c.K = K0.copy()
    c.K[3 * S:4 * S] *= 2.0
    c.K[7 * S:9 * S] *= 0.5
    assert np.allclose(c.relax_scores(2, 0.5), base, rtol=0, atol=1e-13)
    # w = 1: alignment only, in [-1, 1]; negating the Tail flips it
    c.K = K0.copy()
    a = c.relax_scores(2, 1.0)
    assert np.all(np.abs(a) <= 1 + 1e-12)
    c.K[7 * S:] *= -1.0
    assert np.allclose(c.relax_scores(2, 1.0), -a, rtol=0, atol=1e-13)
    # a Tail made of copies of candidate 2: its alignment is exactly 1
    c.K = K0.copy()
    c.K[7 * S:8 * S] = K0[3 * S:4 * S]
    c.K[8 * S:9 * S] = K0[3 * S:4 * S]
    assert abs(c.relax_scores(2, 1.0)[2] - 1.0) < 1e-13
    # identical candidates: complement 0; w = 0 leaves complement alone, in [0, 2]
    c.K = K0.copy()
    comp = c.relax_scores(2, 0.0)
    assert np.all((comp >= -1e-12) & (comp <= 2 + 1e-12))
    for f in range(2, 7):
        c.K[f * S:(f + 1) * S] = K0[S:2 * S]
    assert np.allclose(c.relax_scores(2, 0.0), 0.0, atol=1e-13)
    # a zero frame: cosine 0 with everything (alignment 0, complement 1), and 0 in the others' means
    c.K = K0.copy()
    c.K[2 * S:3 * S] = 0.0
    s = c.relax_scores(2, 0.5)
    assert abs(s[1] - 0.5) < 1e-15
    # swapping two candidate frames swaps their scores and leaves the rest
    c.K = K0.copy()
    c.K[2 * S:3 * S], c.K[5 * S:6 * S] = K0[5 * S:6 * S], K0[2 * S:3 * S]
    s = c.relax_scores(2, 0.5)
    perm = base.copy()
    perm[1], perm[4] = base[4], base[1]
    assert np.allclose(s, perm, rtol=0, atol=1e-13)


def test_one_candidate_and_errors():
    c = _cache(4)
    s = c.relax_scores(2, 0.5)                      # candidate frame 1 only: complement 1
    from oracle.relax import cosine, frame_vector
    K = c.K
    assert abs(s[0] - (0.5 * cosine(frame_vector(K, 4, 1, 2), frame_vector(K, 4, 2, 4)) + 0.5)) < 1e-15
    from oracle import OracleError
    with pytest.raises(OracleError):
        c.relax_scores(3, 0.5)                      # no candidate left
    with pytest.raises(OracleError):
        c.relax_scores(0, 0.5)                      # no tail


def test_top_frames_ties_keep_lower_index():
    assert list(top_frames([0.5, 0.7, 0.7, 0.1, 0.7], 2)) == [1, 2]
    assert list(top_frames([0.2, 0.9, 0.4], 3)) == [0, 1, 2]


def _rf_small(n=16):
    base = WORKLOADS["c5c"]
    return Workload("c5c_small", 106, 2, 64, "bf16", 2, 3, base.sink_frames, base.window_frames, (3,) * n)


def test_relax_forcing_keep_set_and_gap_closing():
    w = _rf_small()
    run = RelaxForcingRun(w)
    S = w.frame_seqlen
    compactions = 0
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        before = {n: getattr(run.cache, n).copy() for n in ("K", "V", "t", "g")}
        run.step(i, q, k, v)
        c = run.cache
        if run.last:
            compactions += 1
            keep, scores = run.last["keep"], run.last["scores"]
            n_old = before["t"].shape[0]
            n_cand = n_old // S - 3 - 2
            assert scores.shape == (n_cand,)
            assert keep.shape[0] == 3 * S + 4 * S + 2 * S
            # whole frames: the kept History is 4 runs of S consecutive entries starting on frame edges
            hist = keep[3 * S:7 * S].reshape(4, S)
            assert np.all(hist[:, 0] % S == 0) and np.all(np.diff(hist, axis=1) == 1)
            kept_f = hist[:, 0] // S - 3
            dropped_f = np.setdiff1d(np.arange(n_cand), kept_f)
            assert scores[kept_f].min() >= scores[dropped_f].max()
            # sink and tail kept whole
            assert np.array_equal(keep[:3 * S], np.arange(3 * S))
            assert np.array_equal(keep[7 * S:], np.arange(n_old - 2 * S, n_old))
            n_keep = keep.shape[0]
            assert np.array_equal(c.V[:n_keep], before["V"][keep])
            assert np.array_equal(c.g[:n_keep], before["g"][keep])
            comp_t = c.t[3 * S:7 * S]
            tail_t = c.t[7 * S:9 * S]
            assert comp_t.max() == tail_t.min() - 1
            assert c.t[:3 * S].max() == comp_t.min() - 1
        assert c.n <= c.C_tok
    assert compactions == 3        # chunks 7, 11, 15, as for Deep Forcing on the same shape
