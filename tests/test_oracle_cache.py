"""Pins for the oracle cache state machine, attention and page constants (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (OracleCache, OracleError, attention_f32, attention_f64, attention_loops_f64, rotate_f32,
                    round_to_bf16, token_positions)
from workloads import WORKLOADS, chunk_inputs, gen

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


# ---------------------------------------------------------------- page constants
def test_page_constants():
    g = GOLD["latent_tokens_per_frame"]
    assert g["latent_h"] * 8 == g["height_px"] and g["latent_w"] * 8 == g["width_px"]
    assert g["latent_h"] * g["latent_w"] // g["patch_tokens"] == g["value"] == 1560
    for name in ("c2", "c3", "c4", "c5a", "c5b"):
        w = WORKLOADS[name]
        assert w.frame_seqlen == 1560 and (w.grid_h, w.grid_w) == (30, 52)
    c3 = WORKLOADS["c3"]
    assert (c3.sink_frames + c3.window_frames) * c3.frame_seqlen == GOLD["window_tokens"]["value"] == 28080
    assert c3.sink_frames * c3.frame_seqlen == GOLD["sink_tokens"]["value"] == 9360
    assert 3 * 1560 == GOLD["chunk_tokens"]["value"]
    # pixel <-> latent frames: (n - 1) / 4 + 1, pinned by f_limit 21 = 81 pixel frames
    lat = lambda n: (n - 1) // 4 + 1
    assert lat(GOLD["f_limit"]["pixel"]) == GOLD["f_limit"]["latent"]
    assert lat(1025) == 257 == WORKLOADS["c4"].total_frames
    assert lat(361) == 91 == c3.total_frames
    assert GOLD["window_pixel_frames_approx"]["value"] == 4 * 18
    rs = GOLD["rolling_sink_K_S"]
    assert round(100 * rs["S"] / rs["K"]) == rs["sink_ratio_percent"]
    assert round(GOLD["long_run_pixel_frames"]["value"] / 16) == GOLD["long_run_pixel_frames"]["seconds_approx"]


# ---------------------------------------------------------------- state machine
def _small_cache(sink=2, window=4, S=6, H=2, D=64, gw=3, dtype="bf16", bank=0):
    return OracleCache(sink, window, S, H, D, gw, dtype, bank)


def _chunk(seed, N, H, D):
    rng = np.random.default_rng(seed)
    k = round_to_bf16(rng.standard_normal((N, H, D)).astype(np.float32))
    v = round_to_bf16(rng.standard_normal((N, H, D)).astype(np.float32))
    return k, v


@pytest.mark.parametrize("frames", [[1] * 15, [2] * 9, [1, 2, 2, 1, 2, 2, 2, 1, 2], [3, 3, 3, 3, 3]])
def test_fifo_eviction_against_full_history(frames):
    c = _small_cache(sink=2, window=4)
    S, H, D = 6, 2, 64
    hist_k, hist_t = [], []
    t0 = 0
    sink_bits = None
    for i, F in enumerate(frames):
        N = F * S
        k, v = _chunk(i, N, H, D)
        before = c.n
        c.append(k, v, F, t0)
        tt, _, _ = token_positions(N, S, 3, t0)
        hist_k.append(k)
        hist_t.append(tt)
        t0 += F
        total = sum(len(x) for x in hist_t)
        # memory constant: n_valid == min(total, capacity)
        assert c.n == min(total, c.C_tok)
        # once full, each chunk evicts exactly as many tokens as it brings
        if before + N > c.C_tok:
            assert c.n == c.C_tok
        # logical g: the sink (first S_tok ever) then the most recent C - S_tok tokens
        exp_g = np.arange(total) if total <= c.C_tok else np.concatenate(
            [np.arange(c.S_tok), np.arange(total - (c.C_tok - c.S_tok), total)])
        assert np.array_equal(c.g, exp_g)
        # each entry's stored key is a fresh rotation of its raw key at its time (no drift)
        allk = np.concatenate(hist_k)
        allt = np.concatenate(hist_t)
        tok = exp_g % S
        fresh = round_to_bf16(rotate_f32(allk[exp_g], allt[exp_g], tok // 3, tok % 3))
        assert np.array_equal(c.K.view(np.uint32), fresh.view(np.uint32))
        assert np.array_equal(c.t, allt[exp_g])
        if c.n_sink == c.S_tok:
            if sink_bits is None:
                sink_bits = c.K[:c.S_tok].copy()
            assert np.array_equal(c.K[:c.S_tok].view(np.uint32), sink_bits.view(np.uint32))


def test_replace_newest_rewrites_in_place():
    c = _small_cache()
    k0, v0 = _chunk(0, 12, 2, 64)
    k1, v1 = _chunk(1, 12, 2, 64)
    for j in range(4):
        c.append(*_chunk(10 + j, 12, 2, 64), 2, 2 * j)
    g_before, n_before = c.g.copy(), c.n
    c.append(k0, v0, 2, 8)
    g_after = c.g.copy()
    c.append(k1, v1, 2, 8, replace_newest=True)
    assert np.array_equal(c.g, g_after) and c.n == min(n_before + 12, c.C_tok)
    assert np.array_equal(c.V[-12:], v1)
    with pytest.raises(OracleError):
        c.append(*_chunk(2, 6, 2, 64), 1, 9, replace_newest=True)


def test_argument_errors():
    c = _small_cache()
    with pytest.raises(OracleError):
        c.append(*_chunk(0, 30, 2, 64), 5, 0)           # chunk larger than the window
    c.append(*_chunk(0, 12, 2, 64), 2, 0)
    with pytest.raises(OracleError):
        c.retime(1, False, 0, 13)
    with pytest.raises(OracleError):
        c.compact([0, 2, 1])
    with pytest.raises(OracleError):
        c.compact([1, 2])                               # drops a sink entry


def test_compact_is_a_gather():
    c = _small_cache()
    for j in range(6):
        c.append(*_chunk(j, 6, 2, 64), 1, j)
    st = {k: v.copy() for k, v in c.state().items() if isinstance(v, np.ndarray)}
    keep = np.array(list(range(12)) + [15, 20, 21, 35])
    c.compact(keep)
    for k in ("K", "V", "t", "g"):
        assert np.array_equal(getattr(c, k), np.stack([st[k][i] for i in keep]))


def test_sliding_window_c3_shape_counts():
    # the 14B-shaped run at reduced heads/dim, integer state only
    w = WORKLOADS["c3"]
    c = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, 1, 64, w.grid_w, "f32")
    z = np.zeros((4680, 1, 64), np.float32)
    for i in range(10):
        before = c.n
        c.append(z, z, 3, 3 * i)
        assert c.n == min(4680 * (i + 1), 28080)
        if i >= 6:
            assert before + 4680 - 28080 == 4680       # num_evicted == new tokens
        m = min(c.n, 9360)
        assert np.array_equal(c.g[:m], np.arange(m))
    assert c.n_sink == 9360 and c.global_end == 46800


# ---------------------------------------------------------------- attention
def _tiny_state(seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((5, 2, 64)).astype(np.float32)
    K = rng.standard_normal((23, 2, 64)).astype(np.float32)
    V = rng.standard_normal((23, 2, 64)).astype(np.float32)
    return q, K, V


def test_attention_brute_force_loops():
    q, K, V = _tiny_state()
    ref = attention_loops_f64(q.tolist(), K.tolist(), V.tolist())
    assert np.max(np.abs(attention_f64(q, K, V) - ref)) < 1e-12
    assert np.max(np.abs(attention_f32(q, K, V) - ref)) < 2e-6


def test_attention_equals_torch_sdpa_fp64():
    q, K, V = _tiny_state(1)
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2)
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).permute(1, 0, 2).numpy()
    assert np.max(np.abs(attention_f64(q, K, V) - ref)) < 1e-12


def test_attention_special_cases():
    q, K, V = _tiny_state(2)
    assert np.max(np.abs(attention_f64(q, K[:1], V[:1]) - np.broadcast_to(V[:1], q.shape))) < 1e-12
    Ke = np.broadcast_to(K[:1], K.shape)
    assert np.max(np.abs(attention_f64(q, Ke, V) - V.astype(np.float64).mean(0, keepdims=True))) < 1e-12
    perm = np.random.default_rng(3).permutation(K.shape[0])
    assert np.max(np.abs(attention_f64(q, K[perm], V[perm]) - attention_f64(q, K, V))) < 1e-12


def test_attend_includes_current_chunk():
    # a single appended chunk attends only to itself; with one token it returns v
    c = OracleCache(0, 2, 1, 1, 64, 1, "f32")
    k, v = _chunk(0, 1, 1, 64)
    c.append(k, v, 1, 0)
    out = c.attend(np.ones((1, 1, 64), np.float32), 1, 0, f64=True)
    assert np.max(np.abs(out - v)) < 1e-12


def test_workload_generator_is_seeded_and_bf16():
    a = gen(2, 3, 1, 100, 4, 128, "bf16")
    b = gen(2, 3, 1, 100, 4, 128, "bf16")
    assert np.array_equal(a, b)
    assert np.array_equal(round_to_bf16(a), a)
    assert abs(float(a.std()) - 1.0) < 0.05
    q, k, v = chunk_inputs(WORKLOADS["tiny"], 0)
    assert q.shape == (16, 2, 64) and not np.array_equal(q, k)


# ---------------------------------------------------------------- block-causal clip attention
def _clip_cache(S=12, H=2, D=64, grid_w=4, frames=6, cfg=77, dtype="f32"):
    oc = OracleCache(0, frames, S, H, D, grid_w, dtype)
    ks, vs = [], []
    for f in range(frames):
        k = gen(cfg, f, 1, S, H, D, dtype)
        v = gen(cfg, f, 2, S, H, D, dtype)
        oc.append(k, v, 1, f)
        ks.append(k)
        vs.append(v)
    q = gen(cfg, 99, 0, frames * S, H, D, dtype)
    return oc, q, ks, vs


def test_block_causal_brute_force_mask():
    """Explicit token mask M[i, j] = (block(j) <= block(i)) with brute-force fp64 loops on tiny inputs."""
    S, frames, bf = 4, 5, 2
    oc, q, _, _ = _clip_cache(S=S, H=2, D=16, grid_w=2, frames=frames)
    qh = oc.rotate_queries(q, frames, 0).astype(np.float64)
    got = oc.attend_block_causal(q, frames, 0, bf, f64=True)
    blk = lambda i: (i // S) // bf
    for i in range(frames * S):
        vis = [j for j in range(oc.n) if blk(j) <= blk(i)]
        ref = attention_loops_f64(qh[i:i + 1].tolist(), oc.K[vis].tolist(), oc.V[vis].tolist())
        assert np.allclose(got[i], ref[0], rtol=1e-12, atol=1e-12)


def test_block_causal_equals_incremental_cache():
    """Block b's rows equal an ordinary attend after appending only blocks 0..b (the chunk-by-chunk
    inference path): two different computations of the same masked softmax."""
    S, frames, bf = 12, 6, 2
    oc, q, ks, vs = _clip_cache(S=S, frames=frames)
    full = oc.attend_block_causal(q, frames, 0, bf, f64=True)
    inc = OracleCache(0, frames, S, 2, 64, 4, "f32")
    for b in range(frames // bf):
        for f in range(b * bf, (b + 1) * bf):
            inc.append(ks[f], vs[f], 1, f)
        rows = slice(b * bf * S, (b + 1) * bf * S)
        ref = inc.attend(q[rows], bf, b * bf, f64=True)
        assert np.allclose(full[rows], ref, rtol=1e-12, atol=1e-12)


def test_block_causal_one_block_is_full_attention():
    oc, q, _, _ = _clip_cache(frames=4)
    a = oc.attend_block_causal(q, 4, 0, 4, f64=True)
    b = oc.attend(q, 4, 0, f64=True)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- max_attention_size (attention over the newest entries)
def test_max_keys_limits_attention_to_the_newest_entries():
    """A limit at or above n_valid changes nothing; a limit equal to the newest chunk's size equals a cache
    holding only that chunk; a limit inside the sink drops the oldest sink entries; brute-force mask."""
    S, H, D = 8, 2, 16
    oc = OracleCache(2, 5, S, H, D, 4, "f32")
    ks, vs = [], []
    for f in range(9):
        k = gen(31, f, 1, S, H, D, "f32")
        v = gen(31, f, 2, S, H, D, "f32")
        oc.append(k, v, 1, f)
        ks.append(k)
        vs.append(v)
    q = gen(31, 99, 0, S, H, D, "f32")
    full = oc.attend(q, 1, 8, f64=True)
    assert np.array_equal(oc.attend(q, 1, 8, f64=True, max_keys=oc.n), full)
    assert np.array_equal(oc.attend(q, 1, 8, f64=True, max_keys=10 * oc.n), full)
    only = OracleCache(0, 1, S, H, D, 4, "f32")
    only.append(ks[8], vs[8], 1, 8)
    assert np.allclose(oc.attend(q, 1, 8, f64=True, max_keys=S), only.attend(q, 1, 8, f64=True),
                       rtol=0, atol=1e-13)
    qh = oc.rotate_queries(q, 1, 8).astype(np.float64)
    for m in (3, 13, 45, 50):
        got = oc.attend(q, 1, 8, f64=True, max_keys=m)
        vis = list(range(oc.n - m, oc.n))
        ref = attention_loops_f64(qh.tolist(), oc.K[vis].tolist(), oc.V[vis].tolist())
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), m
