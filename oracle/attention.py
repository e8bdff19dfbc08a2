"""Chunk-wise attention of the current chunk's queries over every cached entry.

o_i = sum_j p_ij v_j,  p_ij = exp(s_ij - m_i) / sum_j exp(s_ij - m_i),
s_ij = q_i . k_j / sqrt(D), over all valid entries with no mask: the new
block is written before attention and the queries read the whole window up to
local_end, which includes it (LingBot-World 2.0 article, "how the window rolls
when full"; Causal-Forcing article, section 3: only the current block's queries
are computed, against cached history concatenated with the current block).
"""
from __future__ import annotations

import math

import numpy as np


def attention_f32(qh, K, V, block=512):
    """fp32 BLAS attention; qh [Lq, H, D], K/V [n, H, D] (bf16-valued float32). Returns [Lq, H, D] float32."""
    qh = np.asarray(qh, np.float32)
    K = np.asarray(K, np.float32)
    V = np.asarray(V, np.float32)
    Lq, H, D = qh.shape
    scale = np.float32(1.0 / math.sqrt(D))
    out = np.empty((Lq, H, D), np.float32)
    for h in range(H):
        Kh = np.ascontiguousarray(K[:, h, :])
        Vh = np.ascontiguousarray(V[:, h, :])
        for r0 in range(0, Lq, block):
            q = qh[r0:r0 + block, h, :]
            s = (q @ Kh.T) * scale
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[r0:r0 + block, h, :] = (p @ Vh) / p.sum(axis=1, keepdims=True)
    return out


def attention_f64(qh, K, V, block=256):
    """Same definition evaluated in float64."""
    qh = np.asarray(qh, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Lq, H, D = qh.shape
    out = np.empty((Lq, H, D), np.float64)
    for h in range(H):
        Kh, Vh = K[:, h, :], V[:, h, :]
        for r0 in range(0, Lq, block):
            s = (qh[r0:r0 + block, h, :] @ Kh.T) / math.sqrt(D)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[r0:r0 + block, h, :] = (p @ Vh) / p.sum(axis=1, keepdims=True)
    return out


def attention_loops_f64(qh, K, V):
    """Brute force with explicit Python loops (tiny inputs only)."""
    Lq, H, D = len(qh), len(qh[0]), len(qh[0][0])
    n = len(K)
    out = [[[0.0] * D for _ in range(H)] for _ in range(Lq)]
    for i in range(Lq):
        for h in range(H):
            s = []
            for j in range(n):
                acc = 0.0
                for d in range(D):
                    acc += float(qh[i][h][d]) * float(K[j][h][d])
                s.append(acc / math.sqrt(D))
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for d in range(D):
                out[i][h][d] = sum(e[j] * float(V[j][h][d]) for j in range(n)) / z
    return np.array(out, dtype=np.float64)
