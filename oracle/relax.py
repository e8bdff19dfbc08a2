"""Relax Forcing frame scores (rCM length-extrapolation article, strategy 5).  Test infrastructure only.

The article organises the cache as Sink + History + Tail and chooses History frames by cosine
similarity instead of attention mass: a candidate frame scores its alignment with the Tail plus a
complementarity bonus that favours diversity, mixed as  score = w * alignment + (1 - w) * complement,
and the Top-K frames are kept.  It gives no constants and no definition of a frame's vector or of the
complement; the readings taken here are:

* a frame's vector is the mean of its cached (stored, rotated) keys over the frame's S tokens,
  flattened over heads and head dims (length H*D); the Tail's vector is the mean over all Tail tokens;
* alignment(f) = cos(frame f, Tail);
* complement(f) = 1 - mean over the other candidates g of cos(f, g)  (1 when f is the only candidate):
  a candidate unlike the rest of the History scores high;
* cos(x, y) = 0 when either vector is zero;
* w = 0.5 unless given.

Everything is fp64 on the bf16-valued keys.
"""
from __future__ import annotations

import numpy as np


def frame_vector(K, S, f0, f1):
    """Mean key over the tokens of logical frames [f0, f1) of K [n, H, D], flattened to length H*D."""
    K = np.asarray(K, np.float64)
    return K[f0 * S:f1 * S].reshape(-1, K.shape[1] * K.shape[2]).mean(axis=0)


def cosine(x, y):
    nx, ny = float(np.linalg.norm(x)), float(np.linalg.norm(y))
    if nx == 0.0 or ny == 0.0:
        return 0.0
    return float(np.dot(x, y)) / (nx * ny)


def relax_frame_scores(K, S, first, n_cand, tail_frames, weight=0.5):
    """Scores of candidate frames [first, first + n_cand) against the Tail, the tail_frames frames that
    follow them (K in logical order)."""
    cand = [frame_vector(K, S, f, f + 1) for f in range(first, first + n_cand)]
    tail = frame_vector(K, S, first + n_cand, first + n_cand + tail_frames)
    out = np.empty(n_cand, np.float64)
    for i in range(n_cand):
        align = cosine(cand[i], tail)
        others = [cosine(cand[i], cand[j]) for j in range(n_cand) if j != i]
        comp = 1.0 - (sum(others) / len(others) if others else 0.0)
        out[i] = weight * align + (1.0 - weight) * comp
    return out


def top_frames(scores, k):
    """Indices (into scores) of the k best frames, ascending; equal scores keep the lower index."""
    order = np.argsort(-np.asarray(scores), kind="stable")
    return np.sort(order[:k])
