"""GPU parity on the five full-size workloads (14B / Wan-1.3B shapes, 1560-token frames).

Cache state (K, V, t, g, counters) is compared bit for bit with the oracle
after every chunk.  Attention is compared on every row at selected chunks and
on 512 sampled rows (all heads) elsewhere; the GPU always computes every row
in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest

from gpu_util import Timer, assert_state_equal, check_attention, dev, log, new_cache
from oracle import make_run
from workloads import WORKLOADS, chunk_inputs

pytestmark = pytest.mark.gpu


def _run_config(name, full_rows_at=(), every=1, compact=False, sample_rows=512):
    from rolling_kv_cache_amd.policies import driver_for
    w = WORKLOADS[name]
    gc = new_cache(w, compact=compact)
    drv = driver_for(name)(gc, w)
    run = make_run(w)
    rng = np.random.default_rng(1234)
    q_prev = q_prev_d = None
    stats = []
    for i in range(w.n_chunks):
        with Timer(f"{name} chunk {i}"):
            q, k, v = chunk_inputs(w, i)
            qd, kd, vd = dev(q, w), dev(k, w), dev(v, w)
            out = drv.step(i, qd, kd, vd, q_prev=q_prev_d).float().cpu().numpy()
            kw = {}
            if getattr(drv, "last", None):
                kw["keep_override"] = drv.last["keep"]
            full = i in full_rows_at or i == w.n_chunks - 1
            rows = None if full else np.sort(rng.choice(q.shape[0], size=min(sample_rows, q.shape[0]),
                                                         replace=False))
            if name == "c5b":
                ref = run.step(i, q, k, v, q_prev=q_prev, rows=rows, **kw)
                if run.last:
                    _check_keep(run.last["scores"], drv.last, run.cache.S_tok, w)
            elif name == "c5c":
                ref = run.step(i, q, k, v, rows=rows, **kw)
                if run.last:
                    _check_relax_keep(run.last["scores"], drv.last, w)
            else:
                ref = run.step(i, q, k, v, rows=rows)
            if i % every == 0 or full or i == w.n_chunks - 1:
                assert_state_equal(gc, run.cache, w, f"{name} chunk {i}")
            got = out if rows is None else out[rows]
            stats.append(check_attention(got, ref, f"{name} chunk {i}"))
            q_prev, q_prev_d = q, qd
    if w.memory is not None:
        from gpu_util import bits, gpu_bits
        k, v, n = gc.export_memory()
        c = run.cache
        assert n == c.mem_frames > 0
        assert np.array_equal(gpu_bits(k), bits(np.concatenate([c._store(c.mem_k[0]), c._store(c.mem_k[1])]),
                                                w.dtype))
        assert np.array_equal(gpu_bits(v), bits(np.concatenate([c._store(c.mem_v[0]), c._store(c.mem_v[1])]),
                                                w.dtype))
    mx = max(s[0] for s in stats)
    rr = max(s[1] for s in stats)
    log(f"{name}: worst max_abs {mx:.3e} worst rel_rms {rr:.3e} over {len(stats)} chunks")


def _check_keep(oracle_scores, last, S_tok, w):
    """Several keep sets are correct at near-ties: accept the GPU's if every kept candidate scores (in the
    oracle) at least as high as every dropped one, up to 1e-5 of the largest score."""
    s = oracle_scores
    keep = last["keep"]
    g = last["scores"]
    assert np.max(np.abs(g - s)) <= 1e-4 * s.max(), "GPU scores differ from the oracle's"
    n = s.shape[0]
    R = 2 * w.frame_seqlen
    cand = np.arange(S_tok, n - R)
    kept = np.intersect1d(cand, keep)
    dropped = np.setdiff1d(cand, keep)
    assert kept.shape[0] == min(4 * w.frame_seqlen, cand.shape[0])
    if dropped.shape[0]:
        assert s[kept].min() >= s[dropped].max() - 1e-5 * s.max()


def _check_relax_keep(oracle_scores, last, w, tol=2e-5):
    """GPU frame scores match the oracle's; the GPU keep set is whole frames, and every kept candidate frame
    scores (in the oracle) at least as high as every dropped one, up to the score tolerance."""
    s = oracle_scores
    g = last["scores"]
    assert g.shape == s.shape and np.max(np.abs(g - s)) <= tol, "GPU relax scores differ from the oracle's"
    S = w.frame_seqlen
    hist = np.asarray(last["keep"][w.sink_frames * S:(w.sink_frames + 4) * S]).reshape(4, S)
    assert np.all(hist[:, 0] % S == 0) and np.all(np.diff(hist, axis=1) == 1)
    kept = hist[:, 0] // S - w.sink_frames
    dropped = np.setdiff1d(np.arange(s.shape[0]), kept)
    if dropped.shape[0]:
        assert s[kept].min() >= s[dropped].max() - 2 * tol


@pytest.mark.timeout(900)
def test_c3_14b_sliding_window_with_sink():
    """40 heads, 6 sink + 12 rolling frames (28080 keys), 91 frames; eviction every chunk from chunk 6."""
    _run_config("c3", full_rows_at=(6,))


@pytest.mark.timeout(900)
def test_c2_wan13b_global_cache():
    _run_config("c2", full_rows_at=(0,))


@pytest.mark.timeout(900)
def test_c4_rolling_sink():
    _run_config("c4", full_rows_at=(6, 7), sample_rows=256)


@pytest.mark.timeout(900)
def test_c5a_infinity_rope():
    _run_config("c5a", full_rows_at=(7,), compact=True, sample_rows=256)


@pytest.mark.timeout(900)
def test_c5b_deep_forcing():
    _run_config("c5b", full_rows_at=(7,), compact=True, sample_rows=256)


@pytest.mark.timeout(900)
def test_c5a_raw_keys_infinity_rope():
    """Infinity-RoPE on a raw-key cache: the per-chunk shifts only move time indices and every attended key is
    the raw key rotated once at its current time."""
    _run_config("c5a_raw", full_rows_at=(7,), compact=True, sample_rows=256)


@pytest.mark.timeout(900)
def test_c6_memrope_memory_tokens():
    """MemRoPE on the 12-head 3 + 18-frame shape: from chunk 7 on every chunk folds 3 evicted frames into the
    long/short memories, which attention sees beside the sink and window; memory state bit-exact at the end."""
    _run_config("c6", full_rows_at=(7,), sample_rows=256)


@pytest.mark.timeout(900)
def test_c5c_relax_forcing():
    _run_config("c5c", full_rows_at=(7,), compact=True, sample_rows=256)


@pytest.mark.timeout(900)
def test_c2_clip_block_causal():
    """The Wan-1.3B 21-frame clip (32760 query rows, 12 heads) attended block-causally in blocks of 3 frames
    over the cache that holds it: 512 sampled rows plus the first and last row of every block."""
    from oracle import OracleCache
    w = WORKLOADS["c2"]
    S = w.frame_seqlen
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, S, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(w.n_chunks):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), w.chunk_start_frame(i))
        oc.append(k, v, w.chunk_frames[i], w.chunk_start_frame(i))
    F = w.total_frames
    (q,) = chunk_inputs(w, 99, tensors=(0,), frames=F)
    with Timer("c2 clip block-causal"):
        out = gc.attend_block_causal(dev(q, w), 0, 3).float().cpu().numpy()
    rng = np.random.default_rng(4321)
    cb = 3 * S
    edges = np.concatenate([np.arange(0, F * S, cb), np.arange(cb - 1, F * S, cb)])
    rows = np.unique(np.concatenate([rng.choice(F * S, size=512, replace=False), edges]))
    mx, rr = check_attention(out[rows], oc.attend_block_causal(q, F, 0, 3, rows=rows), "c2 clip block-causal")
    log(f"c2 clip block-causal: max_abs {mx:.3e} rel_rms {rr:.3e} on {rows.shape[0]} rows")


@pytest.mark.timeout(900)
def test_head_share_split_keys():
    """One GPU's share of the 40-head layer (5 heads, 4680 queries over 28080 keys): 95 query workgroups, so
    the keys are split in 5 parts; 512 sampled rows against the oracle, and the unsplit launch alike."""
    import os
    from oracle import OracleCache
    w = WORKLOADS["c3"]
    H = 5
    S = w.frame_seqlen
    from rolling_kv_cache_amd import KVCache
    import torch
    gc = KVCache(w.sink_frames, w.window_frames, S, H, w.head_dim, w.grid_w, torch.bfloat16, split_attend=True)
    oc = OracleCache(w.sink_frames, w.window_frames, S, H, w.head_dim, w.grid_w, w.dtype)
    q = None
    for i in range(6):
        q, k, v = (x[:, :H].copy() for x in chunk_inputs(w, i))
        gc.append(dev(k, w), dev(v, w), 3 * i)
        oc.append(k, v, 3, 3 * i)
    rows = np.sort(np.random.default_rng(77).choice(q.shape[0], size=512, replace=False))
    ref = oc.attend(q, 3, 15, rows=rows)
    with Timer("head share split"):
        out = gc.attend(dev(q, w), 15).float().cpu().numpy()
    mx, rr = check_attention(out[rows], ref, "head share split")
    gc.set_paths(no_split=True)
    try:
        out1 = gc.attend(dev(q, w), 15).float().cpu().numpy()
    finally:
        gc.set_paths()
    check_attention(out1[rows], ref, "head share unsplit")
    log(f"head share split: max_abs {mx:.3e} rel_rms {rr:.3e}")


@pytest.mark.parametrize("raw_keys", [False, True])
def test_attention_kernel_variants(raw_keys):
    """The running-maximum 8-wave kernel alone (kvc_set_paths KVC_PATH_RUNNING_MAX) beside the default
    fixed-reference kernel: both match the oracle on sampled rows and each other on every row (the same
    tile order; the fixed reference and the running maximum round their fp32 sums differently, so they
    agree to rounding, not bit for bit).  The cache is 8 heads of the 14B-shaped layer after two
    evictions, so the ring holds two key regions with edge tiles."""
    from oracle import OracleCache
    w = WORKLOADS["c3"]
    H = 8
    S = w.frame_seqlen
    from rolling_kv_cache_amd import KVCache
    import torch
    gc = KVCache(w.sink_frames, w.window_frames, S, H, w.head_dim, w.grid_w, torch.bfloat16, raw_keys=raw_keys)
    oc = OracleCache(w.sink_frames, w.window_frames, S, H, w.head_dim, w.grid_w, w.dtype, raw_keys=raw_keys)
    q = None
    for i in range(8):
        q, k, v = (x[:, :H].copy() for x in chunk_inputs(w, i))
        gc.append(dev(k, w), dev(v, w), 3 * i)
        oc.append(k, v, 3, 3 * i)
    rows = np.sort(np.random.default_rng(78).choice(q.shape[0], size=384, replace=False))
    ref = oc.attend(q, 3, 21, rows=rows)
    outs = {}
    for var in ("default", "running_max"):
        log(f"attention variant {var} raw_keys={raw_keys}")
        gc.set_paths(running_max=var == "running_max")
        try:
            outs[var] = gc.attend(dev(q, w), 21).float().cpu().numpy()
        finally:
            gc.set_paths()
        mx, rr = check_attention(outs[var][rows], ref, f"variant {var}")
        log(f"variant {var}: max_abs {mx:.3e} rel_rms {rr:.3e}")
    mx, rr = check_attention(outs["default"], outs["running_max"], "fixed reference vs running maximum, all rows")
    log(f"fixed reference vs running maximum: max_abs {mx:.3e} rel_rms {rr:.3e}")
