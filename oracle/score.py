"""Deep-Forcing style per-token importance: attention mass received by each cached entry.

The rCM length-extrapolation article (strategy 4, Deep Forcing) scores every
cached token with Q.K^T attention scores collected per layer over a rolling
query window.  Reading taken: the score of entry j is the softmax probability
mass it receives, summed over heads and query rows,
    score_j = sum_h sum_i softmax_j(q_hat_i . k_j / sqrt(D)),
so that sum_j score_j = H * N_q exactly in real arithmetic.
"""
from __future__ import annotations

import math

import numpy as np


def attention_mass_scores(qh, K, dtype=np.float64, block=512):
    """qh [Nq, H, D] (rotated, storage-rounded queries), K [n, H, D] -> scores [n] (float64)."""
    qh = np.asarray(qh, dtype)
    K = np.asarray(K, dtype)
    Nq, H, D = qh.shape
    n = K.shape[0]
    scores = np.zeros(n, np.float64)
    for h in range(H):
        Kh = np.ascontiguousarray(K[:, h, :])
        for r0 in range(0, Nq, block):
            s = (qh[r0:r0 + block, h, :] @ Kh.T) * dtype(1.0 / math.sqrt(D))
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            scores += p.sum(axis=0, dtype=np.float64)
    return scores


def row_normalisers(qh, K, dtype=np.float64, block=512):
    """qh [Nq, H, D], K [n, H, D] -> M [H, Nq] (float64): each query row's softmax normaliser in log2 units,
        M[h, i] = log2 sum_j exp2(c * q_hat_i . k_j),  c = log2(e) / sqrt(D),
    so that softmax_j(q_hat_i . k_j / sqrt(D)) = exp2(c * q_hat_i . k_j - M[h, i]).  This is the quantity
    the scoring's first pass (the row sums of the softmax above) reduces each row to; computed here as the
    natural-log log-sum-exp of the scaled scores, divided by ln 2."""
    qh = np.asarray(qh, dtype)
    K = np.asarray(K, dtype)
    Nq, H, D = qh.shape
    M = np.zeros((H, Nq), np.float64)
    for h in range(H):
        Kh = np.ascontiguousarray(K[:, h, :])
        for r0 in range(0, Nq, block):
            s = (qh[r0:r0 + block, h, :] @ Kh.T) * dtype(1.0 / math.sqrt(D))
            mx = s.max(axis=1)
            lse = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
            M[h, r0:r0 + block] = lse / math.log(2.0)
    return M
