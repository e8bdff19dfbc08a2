"""GPU parity of libkvc against the CPU oracle on small shapes that still span several key tiles and
ragged tails, plus error paths.  Every call goes through the C ABI (ctypes binding)."""

import numpy as np
import pytest
import torch

from gpu_util import assert_state_equal, check_attention, dev, log, new_cache, gpu_bits, paths
from oracle import OracleCache, cos_sin_table, make_run, band_split
from workloads import WORKLOADS, Workload, chunk_inputs

pytestmark = pytest.mark.gpu


def _drive(w, n_chunks=None, full_attention=True, compact=False, general=False, split=False, running_max=False):
    from rolling_kv_cache_amd.policies import driver_for
    gc = new_cache(w, compact=compact, split=split)
    drv = driver_for(w.name)(gc, w)
    run = make_run(w)
    q_prev_d = q_prev = None
    for i in range(n_chunks or w.n_chunks):
        log(f"  {w.name} chunk {i}")
        q, k, v = chunk_inputs(w, i)
        qd, kd, vd = dev(q, w), dev(k, w), dev(v, w)
        with paths(gc, general=general, running_max=running_max):
            out = drv.step(i, qd, kd, vd, q_prev=q_prev_d)
        kw = {}
        if getattr(drv, "last", None):
            kw["keep_override"] = drv.last["keep"]
        if w.name.startswith("c5b"):
            ref = run.step(i, q, k, v, q_prev=q_prev, f64=w.dtype == "f32", **kw)
        elif w.name.startswith("c5c"):
            ref = run.step(i, q, k, v, f64=w.dtype == "f32", **kw)
        else:
            ref = run.step(i, q, k, v, f64=w.dtype == "f32")
        assert_state_equal(gc, run.cache, w, f"{w.name} chunk {i}")
        check_attention(out.float().cpu().numpy(), ref, f"{w.name} chunk {i}")
        q_prev, q_prev_d = q, qd
    return gc, run


# ---------------------------------------------------------------- tables
def test_rope_tables_bitwise():
    w = WORKLOADS["c3"]
    gc = new_cache(Workload("tab", 300, 2, 128, "bf16", 30, 52, 1, 2, (1,)))
    (ts, tw), (hs, hw), _ = band_split(128)
    for lo, n in [(-60, 400), (16383 - 50, 51), (-16383, 20)]:
        got = gc.export_tables(0, lo, n)
        c, s = cos_sin_table(range(lo, lo + n), tw)
        assert np.array_equal(got[..., 0].view(np.uint32), c.view(np.uint32))
        assert np.array_equal(got[..., 1].view(np.uint32), s.view(np.uint32))
    for band, npos in ((1, w.grid_h), (2, w.grid_w)):
        got = gc.export_tables(band, 0, npos)
        c, s = cos_sin_table(range(npos), hw)
        assert np.array_equal(got[..., 0].view(np.uint32), c.view(np.uint32))
        assert np.array_equal(got[..., 1].view(np.uint32), s.view(np.uint32))


# ---------------------------------------------------------------- streams at small sizes
def test_tiny_fp32_stream():
    """The Tiny workload in full: 12 one-frame chunks, eviction from chunk 5, fp64 brute-force reference."""
    _drive(WORKLOADS["tiny"])


SMALL_SW = Workload("sw_small", 201, 3, 128, "bf16", 6, 10, 2, 6, (1, 3, 3, 3, 2, 3, 3, 1, 3))


def test_small_bf16_sliding_window_mfma():
    """bf16 head_dim 128 through the matrix-core kernel: 60-token frames, a 1-frame first chunk so later
    chunks straddle the sink/window boundary, ragged 64-slot tiles in both regions, wrap-around."""
    _drive(SMALL_SW)


def test_small_bf16_sliding_window_general_path():
    _drive(SMALL_SW, general=True)


SMALL_SW64 = Workload("sw64_small", 221, 3, 64, "bf16", 6, 10, 2, 6, (1, 3, 3, 3, 2, 3, 3, 1, 3))


@pytest.mark.parametrize("general", [False, True])
def test_small_bf16_head_dim_64(general):
    """bf16 head_dim 64 (key planes of 24 + 40 dims) through its matrix-core kernel and through the general
    path: the same 60-token frames, straddling first chunk, ragged tiles and wrap-around as above."""
    _drive(SMALL_SW64, general=general)


def test_head_dim_64_many_query_blocks():
    """bf16 head_dim 64 with 12 heads and 3-frame chunks of 552 tokens (1656 query rows: six full 256-row
    blocks and a ragged seventh) over a sink and a window whose tiles end inside a tile."""
    _drive(Workload("sw64_big", 222, 12, 64, "bf16", 23, 24, 2, 7, (3, 3, 3, 3)))


def test_small_rolling_sink():
    base = WORKLOADS["c4"]
    _drive(Workload("c4_small", 203, 2, 128, "bf16", 4, 8, base.sink_frames, base.window_frames,
                    (3,) * 20 + (2,), base.bank_frames))


def test_small_infinity_rope():
    base = WORKLOADS["c5a"]
    _drive(Workload("c5a_small", 204, 2, 128, "bf16", 4, 8, base.sink_frames, base.window_frames,
                    (3,) * 14 + (2,), cut_chunks=(7, 11)), compact=True)


def test_small_deep_forcing():
    base = WORKLOADS["c5b"]
    gc, run = _drive(Workload("c5b_small", 205, 2, 128, "bf16", 4, 8, base.sink_frames, base.window_frames,
                              (3,) * 16), compact=True)


@pytest.mark.parametrize("grid", [(4, 8), (5, 7)])
@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("head_dim", [128, 64])
def test_scores_match_oracle(general, head_dim, grid):
    """Attention-mass scores on the matrix-core passes and on the general path: 32- and 35-token frames give
    a ragged sink region and ragged key tiles, and a 2-frame window of 64 or 70 query rows (whole 32-row
    column-pass tiles only, or a ragged last one); head_dim 128 and 64."""
    w = Workload("score_small", 206, 3, head_dim, "bf16", grid[0], grid[1], 1, 5, (2, 2, 2))
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(3):
        q, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    qw, _, _ = chunk_inputs(w, 7, frames=2)
    with paths(gc, general=general):
        s_gpu = gc.score(dev(qw, w), [3, 4]).cpu().numpy().astype(np.float64)
    s_ref = oc.score(qw, 2, [3, 4], f64=True)
    assert abs(s_gpu.sum() - w.heads * 2 * w.frame_seqlen) < 1e-3
    assert np.max(np.abs(s_gpu - s_ref)) < 1e-4 * max(1.0, s_ref.max())


# log2 normalisers: the attention sums its probabilities as rounded to bf16 for the P.V product (relative
# error at most 2^-8 each, so at most 2^-8 in the sum), i.e. log2(1 + 2^-8) = 5.6e-3, plus fp32 slack
ROW_M_TOL = 6e-3


@pytest.mark.parametrize("grid", [(4, 8), (5, 7)])
@pytest.mark.parametrize("variant", ["", "general", "running_max", "split"])
@pytest.mark.parametrize("head_dim", [128, 64])
def test_score_with_attention_row_stats(variant, head_dim, grid):
    """kvc_attend_stats writes each row's log2 softmax normaliser (against the oracle's, on every attention
    path: fixed reference + recompute, general, running maximum, split keys + merge; head_dim 128 and 64),
    and kvc_score_with_stats, which runs only the columns pass on them, gives the scores of kvc_score
    (against the oracle and the two-pass scores).  32- and 35-token frames: ragged key tiles, a sink
    region, and query windows of whole or ragged 32-row column tiles."""
    from rolling_kv_cache_amd import KVCError, KVC_ESTATE
    w = Workload("score_stats", 206, 3, head_dim, "bf16", grid[0], grid[1], 1, 5, (2, 2, 2))
    gc = new_cache(w, split=variant == "split")
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(3):
        q, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    qw, _, _ = chunk_inputs(w, 7, frames=2)
    qd = dev(qw, w)
    N = 2 * w.frame_seqlen
    rs = torch.full((w.heads * N + 5,), float("nan"), dtype=torch.float32, device="cuda")
    with paths(gc, general=variant == "general", running_max=variant == "running_max"):
        out = gc.attend(qd, 3, row_stats=rs).float().cpu().numpy()
        s_two = gc.score(qd, [3, 4]).cpu().numpy().astype(np.float64)
        s_one = gc.score(qd, [3, 4], row_stats=rs).cpu().numpy().astype(np.float64)
    check_attention(out, oc.attend(qw, 2, 3), f"attend with row statistics {variant}")
    m_gpu = rs[:w.heads * N].view(w.heads, N).cpu().numpy().astype(np.float64)
    m_ref = oc.row_normalisers(qw, 2, 3)
    assert np.isnan(rs[w.heads * N:].cpu().numpy()).all(), "row statistics written past heads x rows"
    assert np.max(np.abs(m_gpu - m_ref)) <= ROW_M_TOL, np.max(np.abs(m_gpu - m_ref))
    s_ref = oc.score(qw, 2, [3, 4], f64=True)
    tol = 1e-4 * max(1.0, s_ref.max())
    assert np.max(np.abs(s_two - s_ref)) < tol
    assert abs(s_one.sum() - w.heads * N) < 1e-3 * w.heads * N
    # every term p_ij / l_i carries its row normaliser's relative error (at most 2^-8: the probabilities the
    # attention sums are rounded to bf16), so does each score: against the two-pass scores elementwise, and
    # against the oracle with the two-pass scores' own tolerance on top
    assert np.all(np.abs(s_one - s_two) <= (2.0 ** -8 + 1e-5) * s_two + 1e-7)
    assert np.all(np.abs(s_one - s_ref) <= (2.0 ** -8 + 1e-5) * s_ref + tol)
    # stale statistics are refused: other times, another buffer, and any call that changes the entries
    with pytest.raises(KVCError) as e:
        gc.score(qd, [4, 5], row_stats=rs)
    assert e.value.code == KVC_ESTATE
    with pytest.raises(KVCError) as e:
        gc.score(qd, [3, 4], row_stats=torch.empty_like(rs))
    assert e.value.code == KVC_ESTATE
    gc.retime(1)
    with pytest.raises(KVCError) as e:
        gc.score(qd, [3, 4], row_stats=rs)
    assert e.value.code == KVC_ESTATE
    gc.attend(qd, 3, row_stats=rs)
    gc.score(qd, [3, 4], row_stats=rs)
    _, k, v = chunk_inputs(w, 3, frames=2)
    gc.append(dev(k, w), dev(v, w), 6)
    with pytest.raises(KVCError) as e:
        gc.score(qd, [3, 4], row_stats=rs)
    assert e.value.code == KVC_ESTATE


def test_attend_row_stats_refused_where_attention_reads_other_entries():
    """With an attention limit below the entries, or memory tokens after the first fold, attention reads
    other entries than a score: kvc_attend_stats returns EUNSUPPORTED and leaves no usable statistics."""
    from rolling_kv_cache_amd import KVCError, KVC_EUNSUPPORTED, KVC_ESTATE
    w = Workload("stats_refused", 208, 2, 128, "bf16", 4, 8, 1, 3, (2,) * 3)
    gc = new_cache(w)
    for i in range(3):
        q, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), 2 * i)
    qd = dev(q, w)
    rs = torch.empty(w.heads * 2 * w.frame_seqlen, dtype=torch.float32, device="cuda")
    gc.attend(qd, 4, row_stats=rs)
    gc.set_attention_limit(3 * w.frame_seqlen)
    with pytest.raises(KVCError) as e:
        gc.attend(qd, 4, row_stats=rs)
    assert e.value.code == KVC_EUNSUPPORTED
    with pytest.raises(KVCError) as e:
        gc.score(qd, [4, 5], row_stats=rs)
    assert e.value.code == KVC_ESTATE
    gc.set_attention_limit(0)
    wm = MEM_SMALL
    gm = new_cache(wm)
    for i in range(wm.n_chunks):
        q, k, v = chunk_inputs(wm, i)
        gm.append(dev(k, wm), dev(v, wm), wm.chunk_start_frame(i))
    rm = torch.empty(wm.heads * wm.chunk_frames[-1] * wm.frame_seqlen, dtype=torch.float32, device="cuda")
    with pytest.raises(KVCError) as e:
        gm.attend(dev(q, wm), wm.chunk_start_frame(wm.n_chunks - 1), row_stats=rm)
    assert e.value.code == KVC_EUNSUPPORTED


def test_replace_newest_denoise_steps():
    """Four denoising re-writes of the newest chunk, then the clean commit, before each new chunk."""
    w = Workload("replace", 207, 2, 128, "bf16", 4, 8, 1, 4, (2,) * 6)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(6):
        for step in range(5):
            q, k, v = chunk_inputs(w, 10 * i + step, frames=2)
            rep = step > 0
            gc.append(dev(k, w), dev(v, w), 2 * i, replace_newest=rep)
            oc.append(k, v, 2, 2 * i, replace_newest=rep)
            out = gc.attend(dev(q, w))
            check_attention(out.float().cpu().numpy(), oc.attend(q, 2), f"replace {i}.{step}")
        assert_state_equal(gc, oc, w, f"replace chunk {i}")


def test_uniform_retime_keeps_attention():
    """Relative-position invariance on the GPU: shift every entry and the queries by the same delta."""
    w = SMALL_SW
    gc = new_cache(w)
    for i in range(5):
        q, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), w.chunk_start_frame(i))
    a = gc.attend(dev(q, w), 30).float().cpu().numpy()
    gc.retime(57)
    b = gc.attend(dev(q, w), 87).float().cpu().numpy()
    check_attention(b, a, "uniform retime")


@pytest.mark.parametrize("dtype,D,H", [("bf16", 128, 3), ("bf16", 128, 24), ("bf16", 128, 29), ("bf16", 128, 64),
                                       ("f32", 128, 5), ("bf16", 64, 26), ("f32", 64, 7)])
def test_retime_workgroup_shapes(dtype, D, H):
    """Retime on caches whose head count and time-band width pick each workgroup shape (8 slots and up to
    five head lanes with 24 or more heads, 32 or 16 slots below; a round of eight heads and a rest of more
    or fewer than four) and whose 55-token frames end inside workgroups: the cache state stays bit-exact
    with the oracle after plain, clamped and partial-range shifts."""
    w = Workload(f"rt_{dtype}_{D}_{H}", 230, H, D, dtype, 5, 11, 1, 4, (2,) * 4)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(4):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    n = gc.info()["n_valid"]
    for d, cl, lo, hi in [(3, False, 0, None), (-5, True, 0, None), (2, False, 7, n - 13), (-1, True, 50, n)]:
        log(f"  {w.name} retime {d} {cl} [{lo}, {hi})")
        gc.retime(d, cl, lo, hi)
        oc.retime(d, cl, lo, hi)
        assert_state_equal(gc, oc, w, f"{w.name} after retime {d} {cl} [{lo}, {hi})")


@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("variant", ["", "running_max"])
def test_attend_score_jump(variant, head_dim):
    """Keys of the oldest frames are tiny and a later chunk's keys and queries are 4x N(0,1): the later
    scores exceed every score of the first key tile by about 42 to 110 in exp2 units (at both head dims), so
    the head_dim-128 fixed-reference kernel must flag its blocks, and the running-maximum kernels (the
    recompute pass, or the only kernel at head_dim 64) raise their maximum mid-row and rescale O (without
    it P overflows to inf)."""
    w = Workload("jump", 207, 2, head_dim, "bf16", 9, 23, 1, 6, (2,) * 4)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(3):
        q, k, v = chunk_inputs(w, i, frames=2)
        f = 4.0 if i == 2 else 1.0 / 64
        k = (k * f).astype(np.float32)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    q = (q * 4.0).astype(np.float32)
    rs = torch.empty(w.heads * 2 * w.frame_seqlen, dtype=torch.float32, device="cuda")
    with paths(gc, running_max=variant == "running_max"):
        out = gc.attend(dev(q, w), 4).float().cpu().numpy()
        out_rs = gc.attend(dev(q, w), 4, row_stats=rs).float().cpu().numpy()
    check_attention(out, oc.attend(q, 2, 4), f"score jump {variant or 'default'}")
    assert np.array_equal(out, out_rs)
    # the rows the recompute pass redid carry its (running-maximum) normalisers
    m_gpu = rs.view(w.heads, -1).cpu().numpy().astype(np.float64)
    assert np.max(np.abs(m_gpu - oc.row_normalisers(q, 2, 4))) <= ROW_M_TOL


def test_scores_score_jump():
    """Attention-mass scores where the later keys' scores exceed every score of the first key tile by about
    48 to 90 in exp2 units: the fixed-reference rows pass must flag those query blocks and the
    running-maximum pass redo them (without it the row sums overflow).  Against the fp64 oracle, with the
    sum over entries equal to heads x query rows."""
    w = Workload("sjump", 243, 2, 128, "bf16", 9, 23, 1, 6, (2,) * 4)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(3):
        _, k, v = chunk_inputs(w, i, frames=2)
        k = (k * (4.0 if i == 2 else 1.0 / 64)).astype(np.float32)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    (q,) = chunk_inputs(w, 97, tensors=(0,), frames=2)
    q = (q * 4.0).astype(np.float32)
    got = gc.score(dev(q, w), [4, 5]).cpu().numpy().astype(np.float64)
    ref = oc.score(q, 2, [4, 5], f64=True)
    assert np.isfinite(got).all()
    assert abs(got.sum() - w.heads * 2 * w.frame_seqlen) < 1e-3 * w.heads * 2 * w.frame_seqlen
    assert np.max(np.abs(got - ref)) <= 1e-4 * max(1.0, ref.max())


# ---------------------------------------------------------------- edge and error paths
def test_error_paths_leave_state_unchanged():
    from rolling_kv_cache_amd import KVCError
    w = Workload("err", 208, 2, 128, "bf16", 4, 8, 1, 3, (1,) * 4, bank_frames=2)
    gc = new_cache(w)
    q, k, v = chunk_inputs(w, 0)
    with pytest.raises(KVCError) as e:
        gc.attend(dev(q, w), 0)                                   # empty cache
    assert e.value.code == 3
    with pytest.raises(KVCError):
        gc.sink_push(0, 1, 0)                                     # bank incomplete
    gc.append(dev(k, w), dev(v, w), 0)
    gc.append(dev(k, w), dev(v, w), 1)
    before = {n: gpu_bits(x) if x.dtype != torch.int32 and x.dtype != torch.int64 else x.cpu().numpy()
              for n, x in gc.export().items()}
    info = gc.info()
    big = torch.zeros((4 * 32, 2, 128), dtype=torch.bfloat16, device="cuda")
    bad_calls = [
        lambda: gc.append(big, big, 5),                           # chunk larger than the window
        lambda: gc.append(torch.cat([dev(k, w)] * 2), torch.cat([dev(v, w)] * 2), 1, replace_newest=True),
        lambda: gc.retime(1, False, 0, info["n_valid"] + 1),        # range past n_valid
        lambda: gc.retime(20000),                                   # |delta| > KVC_MAX_POS
        lambda: gc.compact([0, 1]),                                 # no KVC_CREATE_COMPACT
        lambda: gc.append(dev(k, w), dev(v, w), 16384),            # time past the table
        lambda: gc.sink_push(1, 2, 5),                              # bank frames past the bank
    ]
    for j, call in enumerate(bad_calls):
        with pytest.raises(KVCError):
            call()
        after = gc.export()
        for n, x in after.items():
            y = gpu_bits(x) if x.dtype not in (torch.int32, torch.int64) else x.cpu().numpy()
            assert np.array_equal(y, before[n]), (j, n)
        assert gc.info() == info, j


def test_set_stream_and_paths():
    """kvc_set_stream makes the new stream wait for the work queued on the old one: appends queued on the
    default stream, then attention on a second stream without any synchronization, matches the oracle.
    kvc_set_paths refuses unknown bits."""
    from rolling_kv_cache_amd import lib
    w = SMALL_SW
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(6):
        q, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), w.chunk_start_frame(i))
        oc.append(k, v, w.chunk_frames[i], w.chunk_start_frame(i))
    qd = dev(q, w)
    s2 = torch.cuda.Stream()
    gc.set_stream(s2)
    with torch.cuda.stream(s2):
        out = gc.attend(qd, w.chunk_start_frame(5))
    s2.synchronize()
    check_attention(out.float().cpu().numpy(), oc.attend(q, w.chunk_frames[5], w.chunk_start_frame(5)), "stream")
    assert lib.kvc_set_paths(gc._h, 8) == 1 and lib.kvc_set_paths(gc._h, 0xFFFF) == 1
    gc.set_paths(running_max=True, no_split=True)
    gc.set_paths()


def test_compact_validation():
    from rolling_kv_cache_amd import KVCError
    w = Workload("cval", 209, 2, 128, "bf16", 4, 8, 1, 3, (1,) * 4)
    gc = new_cache(w, compact=True)
    for i in range(4):
        q, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), i)
    n = gc.info()["n_valid"]
    for keep in ([0, 2, 1], [1, 2, 3], list(range(32)) + [n], list(range(32)) + [40, 40]):
        with pytest.raises(KVCError):
            gc.compact(keep)
    gc.compact(list(range(32)) + [40, 70, 71, 127])
    assert gc.info()["n_valid"] == 36


def test_non_finite_key_storage():
    """Storage rounding of non-finite and overflowing keys: a NaN is stored as the quiet bf16 NaN (0x7FC0
    with a sign), infinities as infinities, and rotated values past the bf16 range round to infinity -- the
    oracle's rounding, bit for bit except the NaN sign (IEEE arithmetic leaves a NaN result's sign open).
    Values are written only, never attended."""
    w = Workload("nan", 242, 2, 128, "bf16", 4, 8, 1, 3, (1,) * 2)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    rng = np.random.default_rng(5)
    for i in range(2):
        _, k, v = chunk_inputs(w, i)
        flat = k.reshape(-1)
        pos = rng.choice(flat.shape[0], size=96, replace=False)
        big = np.array([0x7F7F0000], np.uint32).view(np.float32)[0]       # the largest finite bf16
        specials = np.array([np.nan, -np.nan, np.inf, -np.inf, big, -big], np.float32)
        flat[pos] = np.resize(specials, pos.shape[0])
        gc.append(dev(k, w), dev(v, w), 5 * i)
        oc.append(k, v, 1, 5 * i)
    st = gc.export()
    kb = gpu_bits(st["K"]).astype(np.uint32)
    ko = (np.ascontiguousarray(oc.K, np.float32).view(np.uint32) >> 16).astype(np.uint32)
    nan_o = (ko & 0x7FFF) > 0x7F80
    nan_g = (kb & 0x7FFF) > 0x7F80
    assert nan_o.any() and np.array_equal(nan_o, nan_g)
    assert np.all(kb[nan_g] & 0x7FFF == 0x7FC0)
    assert np.array_equal(kb[~nan_g], ko[~nan_g])
    assert np.isinf(oc.K).any()


# ---------------------------------------------------------------- block-causal attention of a whole clip
def _clip(w, frames, chunk=2):
    """Cache (GPU and oracle) holding `frames` frames appended chunk by chunk from time 0, plus the clip's
    queries."""
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    f = 0
    i = 0
    while f < frames:
        n = min(chunk, frames - f)
        _, k, v = chunk_inputs(w, i, frames=n)
        gc.append(dev(k, w), dev(v, w), f)
        oc.append(k, v, n, f)
        f += n
        i += 1
    (q,) = chunk_inputs(w, 99, tensors=(0,), frames=frames)
    return gc, oc, q


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("sink,block", [(0, 2), (1, 3), (1, 8), (0, 1)])
def test_block_causal_small(general, sink, block):
    """207-token frames (a block boundary every 207*block rows, never on a 64-key or 256-row tile edge), a
    sink region or none, a last block cut short (8 frames in blocks of 3), one block (full attention) and
    frame-wise causality (block 1)."""
    w = Workload("bc", 210, 2, 128, "bf16", 9, 23, sink, 8 - sink, (2,) * 4)
    gc, oc, q = _clip(w, 8)
    with paths(gc, general=general):
        out = gc.attend_block_causal(dev(q, w), 0, block).float().cpu().numpy()
    check_attention(out, oc.attend_block_causal(q, 8, 0, block), f"block-causal sink {sink} block {block}")
    if block >= 8:
        check_attention(out, gc.attend(dev(q, w), 0).float().cpu().numpy(), "one block == attend")


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("sink,block", [(0, 2), (1, 3), (0, 1)])
def test_block_causal_head_dim_64(general, sink, block):
    """The block-causal clip of the test above at head_dim 64 (bf16): its own matrix-core kernel and the
    general path against the oracle."""
    w = Workload("bc64", 223, 2, 64, "bf16", 9, 23, sink, 8 - sink, (2,) * 4)
    gc, oc, q = _clip(w, 8)
    with paths(gc, general=general):
        out = gc.attend_block_causal(dev(q, w), 0, block).float().cpu().numpy()
    check_attention(out, oc.attend_block_causal(q, 8, 0, block), f"head_dim 64 block-causal sink {sink} block {block}")


@pytest.mark.parametrize("head_dim", [128, 64])
def test_maximum_query_frames_and_top_time_positions(head_dim):
    """The largest legal calls: 32 query frames (KVC_MAX_Q_FRAMES) attending to, and scoring, a 34-frame
    cache whose times reach the top of the time range (16383 = KVC_MAX_POS), and a 32-frame
    block-causal clip, all against the oracle (head_dim 128 and 64, bf16)."""
    from rolling_kv_cache_amd import KVC_MAX_POS, KVC_MAX_Q_FRAMES
    F = KVC_MAX_Q_FRAMES
    w = Workload("maxq", 224, 2, head_dim, "bf16", 6, 10, 2, F, (4,) * 9)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    t0 = KVC_MAX_POS - 35
    for i in range(9):                      # 36 frames, the newest at KVC_MAX_POS: the first two evicted
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), t0 + 4 * i)
        oc.append(k, v, 4, t0 + 4 * i)
    assert_state_equal(gc, oc, w, "maxq cache")
    (q,) = chunk_inputs(w, 97, tensors=(0,), frames=F)
    tq = KVC_MAX_POS - F + 1
    out = gc.attend(dev(q, w), tq).float().cpu().numpy()
    check_attention(out, oc.attend(q, F, tq), f"{F}-frame attend at the top time positions")
    tf = list(range(tq, tq + F))
    s_gpu = gc.score(dev(q, w), tf).cpu().numpy().astype(np.float64)
    s_ref = oc.score(q, F, tf, f64=True)
    assert abs(s_gpu.sum() - w.heads * F * w.frame_seqlen) < 1e-2
    assert np.max(np.abs(s_gpu - s_ref)) < 1e-4 * max(1.0, s_ref.max())
    wc = Workload("maxq_bc", 225, 2, head_dim, "bf16", 6, 10, 0, F, (4,) * 8)
    gcc, occ, qc = _clip(wc, F, chunk=4)
    out = gcc.attend_block_causal(dev(qc, wc), 0, 3).float().cpu().numpy()
    check_attention(out, occ.attend_block_causal(qc, F, 0, 3), f"{F}-frame block-causal clip")


def test_block_causal_partial_cache_and_time_offset():
    """The clip's queries see only what the cache holds (6 of 8 frames cached), rotated from t0 = 5."""
    w = Workload("bcp", 211, 2, 128, "bf16", 9, 23, 0, 8, (2,) * 3)
    gc, oc, _ = _clip(w, 6)
    (q,) = chunk_inputs(w, 98, tensors=(0,), frames=8)
    out = gc.attend_block_causal(dev(q, w), 5, 3).float().cpu().numpy()
    check_attention(out, oc.attend_block_causal(q, 8, 5, 3), "block-causal partial cache")


def test_block_causal_errors():
    from rolling_kv_cache_amd import KVCError
    w = Workload("bce", 212, 2, 128, "bf16", 4, 8, 1, 3, (1,) * 6)
    gc, _, q = _clip(w, 4, chunk=1)
    qd = dev(q, w)
    for bad in (0, 33):
        with pytest.raises(KVCError) as e:
            gc.attend_block_causal(qd, 0, bad)
        assert e.value.code == 1
    gc.attend_block_causal(qd, 0, 2)                              # sink full, window full, heads at 0
    _, k, v = chunk_inputs(w, 50, frames=1)
    gc.append(dev(k, w), dev(v, w), 4)                            # evicts: the window head moves
    with pytest.raises(KVCError) as e:
        gc.attend_block_causal(qd, 0, 2)
    assert e.value.code == 5


# ---------------------------------------------------------------- Relax Forcing frame scores
RELAX_TOL = 2e-5        # fp32 sums and cosines against the fp64 oracle (scores lie in [-1, 2])


@pytest.mark.parametrize("dtype,grid,D", [("bf16", (9, 60), 128), ("f32", (4, 4), 64), ("bf16", (5, 7), 64)])
def test_relax_scores_match_oracle(dtype, grid, D):
    """Frames of 540 tokens (three 256-token slices, the last ragged) or 16 / 35 tokens, a two-frame sink,
    a window that has wrapped (its ring head is not at slot 0), several weights and tail lengths."""
    w = Workload("rx", 213, 3, D, dtype, grid[0], grid[1], 2, 7, (1,) * 12)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(12):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), i)
        oc.append(k, v, 1, i)
    assert gc.info()["n_valid"] == oc.n
    for tail, wt in ((2, 0.5), (1, 0.3), (5, 1.0), (3, 0.0)):
        got = gc.relax_scores(tail, wt).cpu().numpy()
        ref = oc.relax_scores(tail, wt)
        assert got.shape == ref.shape
        err = float(np.max(np.abs(got - ref)))
        log(f"  relax {dtype} D={D} tail {tail} w {wt}: max err {err:.2e}")
        assert err <= RELAX_TOL, (tail, wt, err)


def test_relax_scores_40_heads_and_frame_limit():
    """40 heads x 128 dims: the Gram pass takes the 5120-long frame sums in two LDS chunks.  Then a cache
    of 70 one-frame appends: more than 64 frames in one call is refused."""
    from rolling_kv_cache_amd import KVCError
    w = Workload("rx40", 216, 40, 128, "bf16", 4, 8, 1, 8, (1,) * 9)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(9):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), i)
        oc.append(k, v, 1, i)
    got = gc.relax_scores(2, 0.5).cpu().numpy()
    assert np.max(np.abs(got - oc.relax_scores(2, 0.5))) <= RELAX_TOL
    w = Workload("rxmax", 217, 1, 64, "bf16", 2, 2, 0, 70, (1,) * 70)
    gc = new_cache(w)
    for i in range(70):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), i)
    with pytest.raises(KVCError) as e:
        gc.relax_scores(7)                                          # 63 candidates + 7 = 70 frames
    assert e.value.code == 5


def test_relax_scores_errors():
    from rolling_kv_cache_amd import KVCError
    w = Workload("rxe", 215, 2, 128, "bf16", 4, 8, 1, 5, (1,) * 6)
    gc = new_cache(w, compact=True)
    for i in range(6):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), i)
    gc.relax_scores(2)
    for tail, wt in ((0, 0.5), (5, 0.5), (6, 0.5), (2, 1.5), (2, -0.1), (2, float("nan"))):
        with pytest.raises(KVCError) as e:
            gc.relax_scores(tail, wt)
        assert e.value.code == 1, (tail, wt)
    gc.compact(list(range(32)) + list(range(40, 100)))                # leaves a partial frame
    with pytest.raises(KVCError) as e:
        gc.relax_scores(1)
    assert e.value.code == 1


# ---------------------------------------------------------------- raw-key caches (time band placed at attention)
from dataclasses import replace as _replace


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("base", [SMALL_SW, SMALL_SW64], ids=["d128", "d64"])
def test_raw_keys_sliding_window(general, base):
    """Stored keys (time band raw, height/width rotated) bit-exact, attention against the oracle's fresh
    rotation, on the ragged sink/window workload (head_dim 128 and 64: the time band placed, then the
    matrix-core kernel of that width, or the general path)."""
    _drive(_replace(base, name="sw_raw", raw_keys=True), general=general)


def test_raw_keys_tiny_fp32():
    _drive(_replace(WORKLOADS["tiny"], name="tiny_raw", raw_keys=True))


@pytest.mark.parametrize("variant", ["", "running_max"])
def test_raw_keys_infinity_rope(variant):
    """Shift with clamp every chunk, flush and cut: index-only retimes, keys rotated at attention."""
    base = WORKLOADS["c5a"]
    w = Workload("c5a_small", 206, 2, 128, "bf16", 4, 8, base.sink_frames, base.window_frames,
                 (3,) * 14 + (2,), cut_chunks=(7, 11), raw_keys=True)
    _drive(w, compact=True, running_max=variant == "running_max")


def test_raw_keys_negative_times_and_block_causal():
    """A shift below time 0 without clamp, then a whole-clip block-causal attend on a raw cache; score and
    relax scores are refused on such a cache."""
    from rolling_kv_cache_amd import KVCError
    w = Workload("rawneg", 218, 2, 128, "bf16", 9, 23, 1, 7, (2,) * 4, raw_keys=True)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                     raw_keys=True)
    for i in range(4):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    (q,) = chunk_inputs(w, 97, tensors=(0,), frames=8)
    check_attention(gc.attend_block_causal(dev(q, w), 0, 2).float().cpu().numpy(),
                    oc.attend_block_causal(q, 8, 0, 2), "raw block-causal")
    gc.retime(-30)
    oc.retime(-30, False)
    assert_state_equal(gc, oc, w, "raw after negative shift")
    (q2,) = chunk_inputs(w, 96, tensors=(0,), frames=2)
    check_attention(gc.attend(dev(q2, w), -24).float().cpu().numpy(), oc.attend(q2, 2, -24), "raw negative t")
    # scores and Relax scores see the keys placed at their (negative) times
    got = gc.score(dev(q2, w), [-24, -23]).cpu().numpy()
    ref = oc.score(q2, 2, [-24, -23])
    assert np.max(np.abs(got - ref)) <= 1e-4 * ref.max()
    assert np.max(np.abs(gc.relax_scores(2).cpu().numpy() - oc.relax_scores(2))) <= RELAX_TOL


# ---------------------------------------------------------------- MemRoPE memory tokens
def _check_memory(gc, oc, w, tag):
    from gpu_util import bits
    k, v, n = gc.export_memory()
    assert n == oc.mem_frames, (tag, n, oc.mem_frames)
    if n == 0:
        return
    ko = np.concatenate([oc._store(oc.mem_k[0]), oc._store(oc.mem_k[1])])
    vo = np.concatenate([oc._store(oc.mem_v[0]), oc._store(oc.mem_v[1])])
    assert np.array_equal(gpu_bits(k), bits(ko, w.dtype)), f"{tag}: memory keys differ"
    assert np.array_equal(gpu_bits(v), bits(vo, w.dtype)), f"{tag}: memory values differ"


def _drive_memory(w, general=False):
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                     raw_keys=True, memory=w.memory)
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        t0 = w.chunk_start_frame(i)
        gc.append(dev(k, w), dev(v, w), t0)
        oc.append(k, v, w.chunk_frames[i], t0)
        with paths(gc, general=general):
            out = gc.attend(dev(q, w), t0).float().cpu().numpy()
        assert_state_equal(gc, oc, w, f"{w.name} chunk {i}")
        _check_memory(gc, oc, w, f"{w.name} chunk {i}")
        check_attention(out, oc.attend(q, w.chunk_frames[i], t0, f64=w.dtype == "f32"), f"{w.name} chunk {i}")
    assert oc.mem_frames > 0
    return gc, oc


MEM_SMALL = _replace(SMALL_SW, name="mem_small", raw_keys=True, memory=(0.9, 0.5))


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("head_dim", [128, 64])
def test_memory_tokens_small(general, head_dim):
    """Memory state bit-exact and attention (sink + memories + window) after every chunk, with 60-token
    frames whose memory slots straddle 64-slot tiles; head_dim 128 and 64."""
    _drive_memory(MEM_SMALL if head_dim == 128 else _replace(MEM_SMALL, name="mem64", head_dim=64), general=general)


def test_memory_tokens_tiny_fp32_and_extreme_rates():
    _drive_memory(_replace(WORKLOADS["tiny"], name="tiny_mem", raw_keys=True, memory=(0.7, 0.2)))
    _drive_memory(_replace(MEM_SMALL, name="mem_extreme", memory=(1.0, 0.0)))


def test_memory_tokens_errors():
    from rolling_kv_cache_amd import KVCError, KVCache
    w = MEM_SMALL
    with pytest.raises(KVCError) as e:
        KVCache(2, 6, w.frame_seqlen, 3, 128, w.grid_w, memory=(0.9, 0.5))     # memory without raw keys
    assert e.value.code == 1
    gc, _ = _drive_memory(_replace(MEM_SMALL, chunk_frames=(3, 3, 3)))
    for rates in ((1.5, 0.5), (0.5, -0.1), (float("nan"), 0.5)):
        with pytest.raises(KVCError) as e:
            gc.set_memory_rates(*rates)
        assert e.value.code == 1
    q, _, _ = chunk_inputs(w, 0, frames=2)
    with pytest.raises(KVCError) as e:
        gc.attend_block_causal(dev(q, w), 0, 1)
    assert e.value.code == 5
    cc = new_cache(_replace(MEM_SMALL, name="mem_c"), compact=True)
    for i in range(3):
        _, k, v = chunk_inputs(w, i, frames=3)
        cc.append(dev(k, w), dev(v, w), 3 * i)
    with pytest.raises(KVCError) as e:
        cc.compact(list(range(cc.info()["n_valid"])))
    assert e.value.code == 5
    plain = new_cache(_replace(SMALL_SW, name="plain"))
    for call in (plain.export_memory, lambda: plain.set_memory_rates(0.5, 0.5)):
        with pytest.raises(KVCError) as e:
            call()
        assert e.value.code == 5


# ---------------------------------------------------------------- attention limited to the newest entries
@pytest.mark.parametrize("general,raw", [(False, False), (True, False), (False, True)])
def test_attention_limit(general, raw):
    """After every chunk of the ragged sink/window workload, attention over the newest m entries for m = all,
    one chunk, a window suffix that wraps the ring, and the sink's last 37 entries plus the whole window
    (ranges that start inside a 64-slot tile)."""
    w = _replace(SMALL_SW, name="lim", raw_keys=raw)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                     raw_keys=raw)
    S = w.frame_seqlen
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        t0 = w.chunk_start_frame(i)
        F = w.chunk_frames[i]
        gc.append(dev(k, w), dev(v, w), t0)
        oc.append(k, v, F, t0)
        n = oc.n
        nw = n - oc.n_sink
        for m in sorted({n, F * S, max(1, nw - 37), min(n, nw + 37), 1}):
            gc.set_attention_limit(m)
            with paths(gc, general=general):
                out = gc.attend(dev(q, w), t0).float().cpu().numpy()
            check_attention(out, oc.attend(q, F, t0, max_keys=m), f"chunk {i} limit {m}")
        gc.set_attention_limit(0)


def test_attention_limit_refusals():
    from rolling_kv_cache_amd import KVCError
    w = SMALL_SW
    gc = new_cache(w)
    with pytest.raises(KVCError) as e:
        gc.set_attention_limit(-1)
    assert e.value.code == 1
    for i in range(4):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), w.chunk_start_frame(i))
    gc.set_attention_limit(100)
    (q,) = chunk_inputs(w, 95, tensors=(0,), frames=2)
    with pytest.raises(KVCError) as e:
        gc.attend_block_causal(dev(q, w), 0, 1)
    assert e.value.code == 5
    # a Rolling-Sink sink that has rolled: the visible tail of the sink is two slot ranges plus the window
    base = WORKLOADS["c4"]
    rw = Workload("c4_lim", 220, 2, 128, "bf16", 4, 8, 3, 2, (1,) * 8, bank_frames=4)
    rc = new_cache(rw)
    for i in range(6):
        _, k, v = chunk_inputs(rw, i)
        rc.append(dev(k, rw), dev(v, rw), i)
    rc.sink_push(0, 1, 6)
    n = rc.info()["n_valid"]
    rc.set_attention_limit(n - 5)
    (q,) = chunk_inputs(rw, 94, tensors=(0,), frames=1)
    with pytest.raises(KVCError) as e:
        rc.attend(dev(q, rw), 7)
    assert e.value.code == 5
    m = new_cache(_replace(MEM_SMALL, name="mem_lim"))
    for i in range(4):
        _, k, v = chunk_inputs(w, i, frames=3)
        m.append(dev(k, w), dev(v, w), 3 * i)
    m.set_attention_limit(50)
    (q,) = chunk_inputs(w, 93, tensors=(0,), frames=1)
    with pytest.raises(KVCError) as e:
        m.attend(dev(q, w), 12)
    assert e.value.code == 5


# ---------------------------------------------------------------- layer groups and the denoise loop
def _group(w, n, compact=False):
    from rolling_kv_cache_amd import create_group
    return create_group(n, w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w,
                        dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32, bank_frames=w.bank_frames,
                        compact=compact, raw_keys=w.raw_keys)


def test_denoise_loop_over_a_layer_group():
    """Three layers over one workspace: per chunk four sampling passes and the commit (pass 0 writes, the
    rest re-write in place), each layer attending with its own q/k/v; after every second chunk one batched
    retime of all layers (alternately a shift of +2 and a clamped shift of -3).  Every pass's attention and
    every layer's cache state against the oracle."""
    from oracle import DenoiseLoopRun
    from rolling_kv_cache_amd import retime_layers
    from rolling_kv_cache_amd.policies import DenoiseLoop
    from workloads import denoise_inputs
    w = SMALL_SW
    L = 3
    caches = _group(w, L)
    loop = DenoiseLoop(caches, w)
    run = DenoiseLoopRun(w, L)
    for i in range(w.n_chunks):
        for s in range(5):
            for layer in range(L):
                q, k, v = denoise_inputs(w, i, s, layer)
                out = loop.pass_layer(i, layer, s, dev(q, w), dev(k, w), dev(v, w)).float().cpu().numpy()
                check_attention(out, run.step(i, layer, s, q, k, v), f"chunk {i} pass {s} layer {layer}")
        if i % 2 == 1:
            delta, clamp = (2, False) if i % 4 == 1 else (-3, True)
            retime_layers(caches, delta, clamp)
            for c in run.caches:
                c.retime(delta, clamp)
        for layer in range(L):
            assert_state_equal(caches[layer], run.caches[layer], w, f"chunk {i} layer {layer}")


def test_layer_batched_sink_push_and_compact():
    """Rolling-Sink pushes and a Deep-Forcing-style compaction as single launches over two layers, each
    layer's state against the oracle."""
    from rolling_kv_cache_amd import compact_layers, sink_push_layers
    base = WORKLOADS["c4"]
    w = Workload("grp", 221, 2, 128, "bf16", 4, 8, 3, 4, (1,) * 12, bank_frames=6)
    caches = _group(w, 2, compact=True)
    oc = [OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                      w.bank_frames) for _ in range(2)]
    for i in range(8):
        for layer in range(2):
            _, k, v = chunk_inputs(w, 10 * layer + i, frames=1)
            caches[layer].append(dev(k, w), dev(v, w), i)
            oc[layer].append(k, v, 1, i)
    sink_push_layers(caches, 2, 1, 8)
    sink_push_layers(caches, 4, 2, 9)
    for c in oc:
        c.sink_push(2, 1, 8)
        c.sink_push(4, 2, 9)
    n = oc[0].n
    keep = np.concatenate([np.arange(oc[0].n_sink), oc[0].n_sink + np.arange(0, n - oc[0].n_sink, 3)])
    compact_layers(caches, keep)
    for c in oc:
        c.compact(keep)
    for layer in range(2):
        assert_state_equal(caches[layer], oc[layer], w, f"layer {layer}")


def test_layer_batch_refusals():
    from rolling_kv_cache_amd import KVCError, retime_layers
    w = SMALL_SW
    caches = _group(w, 3)
    other = _group(w, 2)
    _, k, v = chunk_inputs(w, 0)
    for c in caches + other:
        c.append(dev(k, w), dev(v, w), 0)
    for bad, code in (([caches[0], caches[2]], 1), ([caches[1], caches[0]], 1), ([caches[0], other[1]], 1),
                      ([new_cache(w), caches[1]], 1)):
        with pytest.raises(KVCError) as e:
            retime_layers(bad, 1)
        assert e.value.code == code
    caches[1].append(dev(k, w), dev(v, w), 1)                     # layer 1 moves on alone
    with pytest.raises(KVCError) as e:
        retime_layers(caches, 1)
    assert e.value.code == 3
    retime_layers(caches[:1], 1)                                   # one layer: the plain call


def test_compact_across_the_ring_wrap():
    """Regression: a compaction whose kept window entries cross the ring's wrap (the window has evicted, so
    its logical start is mid-buffer) -- the source slots of the kept entries fall again after the wrap and
    every source tile they touch must be gathered."""
    w = Workload("wrapc", 222, 2, 128, "bf16", 4, 8, 3, 4, (1,) * 8)
    gc = new_cache(w, compact=True)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(9):
        _, k, v = chunk_inputs(w, i, frames=1)
        gc.append(dev(k, w), dev(v, w), i)
        oc.append(k, v, 1, i)
    assert gc.info()["window_head"] != 0
    keep = np.concatenate([np.arange(oc.n_sink), oc.n_sink + np.arange(0, oc.n - oc.n_sink, 3)])
    gc.compact(keep)
    oc.compact(keep)
    assert_state_equal(gc, oc, w, "compaction across the wrap")


@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("variant", ["", "running_max"])
def test_block_causal_score_jump(variant, head_dim):
    """Block-causal attention where the later blocks' scores exceed the first key tile's by tens of exp2
    units: at head_dim 128 the fixed-reference kernel must flag those blocks and the running-maximum pass
    redo them; at head_dim 64 the running-maximum kernel alone must rescale mid-row."""
    w = Workload("bcjump", 223, 2, head_dim, "bf16", 9, 23, 0, 6, (2,) * 3)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(3):
        _, k, v = chunk_inputs(w, i, frames=2)
        k = (k * (4.0 if i >= 1 else 1.0 / 64)).astype(np.float32)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    (q,) = chunk_inputs(w, 98, tensors=(0,), frames=6)
    q = (q * 4.0).astype(np.float32)
    with paths(gc, running_max=variant == "running_max"):
        out = gc.attend_block_causal(dev(q, w), 0, 2).float().cpu().numpy()
    check_attention(out, oc.attend_block_causal(q, 6, 0, 2), f"block-causal score jump {variant or 'default'}")


# ---------------------------------------------------------------- split-key attention
@pytest.mark.parametrize("raw", [False, True])
def test_split_key_attention(raw):
    """Three heads and chunks of up to 180 queries give a handful of workgroups, so the keys are split in
    parts (2 to 8 as the cache grows) and merged; ragged tiles, sink/window regions and wrap as before."""
    _drive(_replace(SMALL_SW, name="split", raw_keys=raw), split=True)


def test_split_key_attention_flush_and_retime():
    base = WORKLOADS["c5a"]
    _drive(Workload("c5a_split", 224, 2, 128, "bf16", 4, 8, base.sink_frames, base.window_frames,
                    (3,) * 14 + (2,), cut_chunks=(7, 11)), compact=True, split=True)


@pytest.mark.parametrize("name", ["c5b", "c5c"])
def test_raw_keys_deep_and_relax_forcing(name):
    """Deep Forcing (attention-mass scores, compaction, gap-closing retimes) and Relax Forcing on raw-key
    caches: the scores read the keys placed at their current times; state bit-exact, attention against the
    oracle."""
    base = WORKLOADS[name]
    _drive(Workload(name + "_small", 225, 2, 128, "bf16", 4, 8, base.sink_frames, base.window_frames, (3,) * 16,
                    raw_keys=True), compact=True)


def test_split_keys_with_limit_and_memory():
    """Split-key launches over ranges that start inside a tile (attention limit) and over the memory slots
    of a MemRoPE cache."""
    w = _replace(SMALL_SW, name="split_lim")
    gc = new_cache(w, split=True)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype)
    for i in range(w.n_chunks):
        q, k, v = chunk_inputs(w, i)
        t0 = w.chunk_start_frame(i)
        gc.append(dev(k, w), dev(v, w), t0)
        oc.append(k, v, w.chunk_frames[i], t0)
        n = oc.n
        m = max(1, n - 150)
        gc.set_attention_limit(m)
        out = gc.attend(dev(q, w), t0).float().cpu().numpy()
        check_attention(out, oc.attend(q, w.chunk_frames[i], t0, max_keys=m), f"split limit chunk {i}")
        gc.set_attention_limit(0)
    wm = _replace(MEM_SMALL, name="split_mem")
    gm = new_cache(wm, split=True)
    om = OracleCache(wm.sink_frames, wm.window_frames, wm.frame_seqlen, wm.heads, wm.head_dim, wm.grid_w, wm.dtype,
                     raw_keys=True, memory=wm.memory)
    for i in range(wm.n_chunks):
        q, k, v = chunk_inputs(wm, i)
        t0 = wm.chunk_start_frame(i)
        gm.append(dev(k, wm), dev(v, wm), t0)
        om.append(k, v, wm.chunk_frames[i], t0)
        out = gm.attend(dev(q, wm), t0).float().cpu().numpy()
        check_attention(out, om.attend(q, wm.chunk_frames[i], t0), f"split memory chunk {i}")
    assert om.mem_frames > 0


# ---------------------------------------------------------------- seeded random operation sequences
RANDOM_CASES = [  # seed, raw keys, memory tokens, split-key attention, dtype, head_dim
    (1, False, False, False, "bf16", 128), (2, False, False, False, "bf16", 128),
    (3, True, False, False, "bf16", 128), (4, True, False, False, "bf16", 128),
    (5, True, True, False, "bf16", 128), (6, True, True, True, "bf16", 128),
    (7, False, False, True, "bf16", 128), (8, True, False, True, "bf16", 128),
    (9, False, False, False, "f32", 128), (10, True, True, False, "f32", 64),
    (13, False, False, False, "bf16", 64), (14, True, False, False, "bf16", 64),
]


@pytest.mark.parametrize("seed,raw,memory,split,dtype,head_dim", RANDOM_CASES)
def test_random_operation_sequences(seed, raw, memory, split, dtype, head_dim):
    """At least 80 seeded random operations (more until ten attends were checked) on a small cache (sink 2 + window 5 frames of 24 tokens, 4-frame bank,
    compaction buffer; bf16 or fp32, head_dim 128 or 64): appends and newest-chunk re-writes, retimes of
    random ranges with and without clamp, random compactions, sink pushes, memory-rate changes, attends at
    random times with random limits, block-causal attends, attention-mass scores and Relax Forcing frame
    scores.  Every operation goes to the oracle first;
    where it refuses, the library must refuse too and keep its state; after every operation the cache states
    (and memory tokens) are equal bit for bit, and every attend agrees.  The library also refuses, as
    documented, a limited attend whose visible entries span a rolled sink and a block-causal attend once a
    ring has rolled."""
    from oracle import OracleError
    from rolling_kv_cache_amd import KVCError
    w = Workload(f"rand{seed}", 230 + seed, 2, head_dim, dtype, 4, 6, 2, 5, (1,), bank_frames=4, raw_keys=raw,
                 memory=(0.9, 0.5) if memory else None)
    gc = new_cache(w, compact=True, split=split)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                     w.bank_frames, raw_keys=raw, memory=w.memory)
    rng = np.random.default_rng(seed)
    ops = ["append", "append", "replace", "retime", "compact", "push", "attend", "attend", "bcausal", "score",
           "relax"] + (["rates"] if memory else [])
    t_next, last_F, uid, pushed, attended, refused, scored = 0, None, 0, False, 0, 0, 0
    for step in range(240):
        if step >= 80 and attended >= 10:
            break           # at least 80 operations, longer until ten attends have been checked
        op = str(rng.choice(ops))
        uid += 1
        tag = f"seed {seed} step {step} {op}"
        if op in ("append", "replace"):
            F = int(rng.integers(1, 3)) if op == "append" else (last_F or 1)
            _, k, v = chunk_inputs(w, 100 + uid, frames=F)
            t0 = t_next if op == "append" else max(0, t_next - F)
            kd, vd, rep = dev(k, w), dev(v, w), op == "replace"
            call_o = lambda: oc.append(k, v, F, t0, replace_newest=rep)
            call_g = lambda: gc.append(kd, vd, t0, replace_newest=rep)
        elif op == "retime":
            n = oc.n
            lo = int(rng.integers(0, n + 1)) if n else 0
            hi = int(rng.integers(lo, n + 1)) if n else 0
            d, cl = int(rng.integers(-5, 6)), bool(rng.integers(0, 2))
            call_o = lambda: oc.retime(d, cl, lo, hi)
            call_g = lambda: gc.retime(d, cl, lo, hi)
        elif op == "compact":
            n, ns = oc.n, oc.n_sink
            extra = np.zeros(0, np.int64)
            if n > ns:
                extra = np.sort(rng.choice(np.arange(ns, n), size=int(rng.integers(0, n - ns + 1)), replace=False))
            keep = np.concatenate([np.arange(ns), extra]).astype(np.int64)
            if keep.shape[0] == 0:
                continue
            call_o = lambda: oc.compact(keep)
            call_g = lambda: gc.compact(keep)
        elif op == "push":
            b, F = int(rng.integers(0, 4)), int(rng.integers(1, 3))
            t0 = int(rng.integers(0, 20))
            call_o = lambda: oc.sink_push(b, F, t0)
            call_g = lambda: gc.sink_push(b, F, t0)
        elif op == "rates":
            al, ash = (float(x) for x in rng.choice([0.0, 0.25, 0.5, 0.9, 1.0], size=2))

            def call_o():
                oc.memory = (al, ash)
            call_g = lambda: gc.set_memory_rates(al, ash)
        elif op == "score":
            if oc.n == 0:
                continue
            F = int(rng.integers(1, 3))
            qt = [int(x) for x in rng.integers(-8, 30, size=F)]
            (q,) = chunk_inputs(w, 700 + uid, tensors=(0,), frames=F)
            got = gc.score(dev(q, w), qt).cpu().numpy().astype(np.float64)
            ref = oc.score(q, F, qt, f64=True)
            assert np.max(np.abs(got - ref)) <= 1e-4 * max(1.0, ref.max()), tag
            scored += 1
            continue
        elif op == "relax":
            tail, wt = int(rng.integers(1, 4)), float(rng.choice([0.0, 0.3, 0.5, 1.0]))
            try:
                ref = oc.relax_scores(tail, wt)
            except OracleError:
                ref = None
            if ref is None:
                with pytest.raises(KVCError):
                    gc.relax_scores(tail, wt)
            else:
                assert np.max(np.abs(gc.relax_scores(tail, wt).cpu().numpy() - ref)) <= RELAX_TOL, tag
                scored += 1
            continue
        elif op == "bcausal":
            if oc.n == 0:
                continue
            F, bf, t0 = int(rng.integers(1, 4)), int(rng.integers(1, 3)), int(rng.integers(0, 10))
            (q,) = chunk_inputs(w, 500 + uid, tensors=(0,), frames=F)
            try:
                ref = oc.attend_block_causal(q, F, t0, bf)
            except OracleError:
                ref = None
            inf = gc.info()
            rolled = inf["sink_head"] != 0 or inf["window_head"] != 0
            try:
                out = gc.attend_block_causal(dev(q, w), t0, bf).float().cpu().numpy()
            except KVCError as e:
                # the oracle's refusal, or the documented one: logical order no longer equals slot order
                assert ref is None or (rolled and e.code == 5), (tag, str(e))
                refused += 1
                continue
            assert ref is not None and not rolled, f"{tag}: attended where a refusal is due"
            check_attention(out, ref, tag)
            attended += 1
            continue
        else:
            if oc.n == 0:
                continue
            F = int(rng.integers(1, 3))
            (q,) = chunk_inputs(w, 500 + uid, tensors=(0,), frames=F)
            t0 = int(rng.integers(-8, 30))
            m = int(rng.integers(1, oc.n + 1)) if rng.integers(0, 3) == 0 else 0
            try:
                ref = oc.attend(q, F, t0, max_keys=m or None)
            except OracleError:
                ref = None
            gc.set_attention_limit(m)
            try:
                out = gc.attend(dev(q, w), t0).float().cpu().numpy()
            except KVCError as e:
                # the oracle's refusal, or the documented one: a limit whose visible entries span a rolled sink
                assert ref is None or (m and e.code == 5 and pushed), (tag, str(e))
                refused += 1
                continue
            finally:
                gc.set_attention_limit(0)
            assert ref is not None, f"{tag}: the oracle refuses, the library attends"
            check_attention(out, ref, tag)
            attended += 1
            continue
        try:
            call_o()
            ok = True
        except OracleError:
            ok = False
        if ok:
            call_g()
            if op == "append":
                t_next, last_F = t0 + F, F
            elif op == "compact" and oc.newest is None:
                last_F = None
            elif op == "push":
                pushed = True
        else:
            before = gc.info()
            with pytest.raises(KVCError):
                call_g()
            assert gc.info() == before, tag
        if oc.n:
            assert_state_equal(gc, oc, w, tag)
        if memory:
            _check_memory(gc, oc, w, tag)
    log(f"  seed {seed}: {step} operations, {attended} attends, {refused} refused, {scored} scores")
    assert attended >= 10


@pytest.mark.parametrize("seed,raw", [(11, False), (12, True)])
def test_random_layer_group_sequences(seed, raw):
    """60 seeded random operations on a three-layer group (same small geometry as above): per-layer appends,
    re-writes and attends with each layer's own data; retimes, compactions and sink pushes as batched calls
    over a random run of consecutive layers, followed by the same call over the other layers.  While the
    layers differ, a batched call over the whole group must be refused with its state kept (ESTATE).  Every
    layer's state against its own oracle after every step."""
    from oracle import OracleError
    from rolling_kv_cache_amd import KVCError, compact_layers, retime_layers, sink_push_layers
    L = 3
    w = Workload(f"grp{seed}", 250 + seed, 2, 128, "bf16", 4, 6, 2, 5, (1,), bank_frames=4, raw_keys=raw)
    caches = _group(w, L, compact=True)
    ocs = [OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                       w.bank_frames, raw_keys=raw) for _ in range(L)]
    rng = np.random.default_rng(seed)
    t_next, last_F, uid, attended, batched = 0, None, 0, 0, 0
    for step in range(60):
        op = str(rng.choice(["append", "append", "replace", "retime", "retime", "compact", "push", "attend"]))
        uid += 1
        tag = f"seed {seed} step {step} {op}"
        oc0 = ocs[0]
        if op in ("append", "replace"):
            F = int(rng.integers(1, 3)) if op == "append" else (last_F or 1)
            t0 = t_next if op == "append" else max(0, t_next - F)
            rep = op == "replace"
            try:
                for li in range(L):
                    _, k, v = chunk_inputs(w, 1000 * li + uid, frames=F)
                    ocs[li].append(k, v, F, t0, replace_newest=rep)
                    caches[li].append(dev(k, w), dev(v, w), t0, replace_newest=rep)
            except OracleError:
                assert li == 0, tag
                with pytest.raises(KVCError):
                    caches[0].append(dev(k, w), dev(v, w), t0, replace_newest=rep)
            else:
                if op == "append":
                    t_next, last_F = t0 + F, F
        elif op == "attend":
            if oc0.n == 0:
                continue
            li, F, t0 = int(rng.integers(0, L)), int(rng.integers(1, 3)), int(rng.integers(-8, 30))
            (q,) = chunk_inputs(w, 5000 + uid, tensors=(0,), frames=F)
            out = caches[li].attend(dev(q, w), t0).float().cpu().numpy()
            check_attention(out, ocs[li].attend(q, F, t0), f"{tag} layer {li}")
            attended += 1
            continue
        else:
            if op == "retime":
                n = oc0.n
                lo = int(rng.integers(0, n + 1)) if n else 0
                hi = int(rng.integers(lo, n + 1)) if n else 0
                d, cl = int(rng.integers(-5, 6)), bool(rng.integers(0, 2))
                do_o = lambda c: c.retime(d, cl, lo, hi)
                do_g = lambda cs: retime_layers(cs, d, cl, lo, hi)
            elif op == "compact":
                n, ns = oc0.n, oc0.n_sink
                extra = np.zeros(0, np.int64)
                if n > ns:
                    extra = np.sort(rng.choice(np.arange(ns, n), size=int(rng.integers(0, n - ns + 1)),
                                               replace=False))
                keep = np.concatenate([np.arange(ns), extra]).astype(np.int64)
                if keep.shape[0] == 0:
                    continue
                do_o = lambda c: c.compact(keep)
                do_g = lambda cs: compact_layers(cs, keep)
            else:
                b, F, t0 = int(rng.integers(0, 4)), int(rng.integers(1, 3)), int(rng.integers(0, 20))
                do_o = lambda c: c.sink_push(b, F, t0)
                do_g = lambda cs: sink_push_layers(cs, b, F, t0)
            try:
                do_o(ocs[0])
            except OracleError:
                before = caches[0].info()
                with pytest.raises(KVCError):
                    do_g(caches)
                assert caches[0].info() == before, tag
            else:
                for c in ocs[1:]:
                    do_o(c)
                a = int(rng.integers(0, L))
                e = int(rng.integers(a + 1, L + 1))
                do_g(caches[a:e])
                batched += 1
                if (a, e) != (0, L):
                    t_a, g_a = caches[a].slot_times()
                    t_o, g_o = caches[0 if a > 0 else L - 1].slot_times()
                    if caches[a].info() != caches[0 if a > 0 else L - 1].info() or not (
                            np.array_equal(t_a, t_o) and np.array_equal(g_a, g_o)):
                        before = [c.info() for c in caches]
                        with pytest.raises(KVCError) as ex:
                            do_g(caches)
                        assert ex.value.code == 3, tag
                        assert [c.info() for c in caches] == before, tag
                    if a > 0:
                        do_g(caches[:a])
                    if e < L:
                        do_g(caches[e:])
                if op == "compact" and oc0.newest is None:
                    last_F = None
        for li in range(L):
            if ocs[li].n:
                assert_state_equal(caches[li], ocs[li], w, f"{tag} layer {li}")
    log(f"  seed {seed}: {attended} attends, {batched} batched calls")
    assert attended >= 5 and batched >= 10


# ---------------------------------------------------------------- raw keys: placed planes vs per-key rotation
def test_raw_keys_placed_attention_equals_general_path():
    """On bf16 head_dim-128 raw-key caches kvc_attend first places every slot's time band (and the memory
    tokens) into the workspace's placed plane and runs the plain matrix-core kernels; the general path
    rotates each key's time band at its slot's time inside its dot product.  Over a plain window, an
    attention limit, memory tokens, split keys and block-causal attention both match the oracle and each
    other within the attention tolerance."""
    def both(call):
        a = call().float().cpu().numpy()
        with paths(gc, general=True):
            b = call().float().cpu().numpy()
        check_attention(a, b, "placed vs general")
        return a

    for memory, split in ((None, False), ((0.9, 0.5), False), (None, True), ((0.9, 0.5), True)):
        w = _replace(SMALL_SW, name="raw_placed", raw_keys=True, memory=memory)
        gc = new_cache(w, split=split)
        oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                         raw_keys=True, memory=memory)
        for i in range(w.n_chunks):
            q, k, v = chunk_inputs(w, i)
            t0 = w.chunk_start_frame(i)
            gc.append(dev(k, w), dev(v, w), t0)
            oc.append(k, v, w.chunk_frames[i], t0)
            if i % 3 == 2:
                gc.retime(-2, True)
                oc.retime(-2, True)
            tag = f"memory {memory} split {split} chunk {i}"
            out = both(lambda: gc.attend(dev(q, w), t0 + 1))
            check_attention(out, oc.attend(q, w.chunk_frames[i], t0 + 1), tag)
            if memory is None and oc.n > 100:
                m = oc.n - 70
                gc.set_attention_limit(m)
                try:
                    out = both(lambda: gc.attend(dev(q, w), t0))
                finally:
                    gc.set_attention_limit(0)
                check_attention(out, oc.attend(q, w.chunk_frames[i], t0, max_keys=m), tag + " limited")
        assert memory is None or oc.mem_frames > 0
    # block-causal over a raw clip cache
    w = Workload("raw_placed_bc", 241, 2, 128, "bf16", 6, 10, 0, 8, (2, 2, 2, 2), raw_keys=True)
    gc = new_cache(w)
    oc = OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, w.dtype,
                     raw_keys=True)
    for i in range(4):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), 2 * i)
        oc.append(k, v, 2, 2 * i)
    gc.retime(3)
    oc.retime(3, False)
    (q,) = chunk_inputs(w, 90, tensors=(0,), frames=8)
    out = both(lambda: gc.attend_block_causal(dev(q, w), 3, 2))
    check_attention(out, oc.attend_block_causal(q, 8, 3, 2), "raw placed block-causal")
