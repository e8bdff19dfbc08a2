"""kvc_relax_scores_noalloc (scratch held by the library, nothing allocated per call) against
kvc_relax_scores (caller-provided scratch) through the C ABI: the same kernels on the same cache, so the
scores must be identical bit for bit, on consecutive calls over caches of decreasing size (the second call
finds the first call's values in the shared scratch), on a raw-key cache (whose placed key planes also live
in the scratch), and a cache too large for the held scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

from gpu_util import dev, log
from workloads import Workload, chunk_inputs

pytestmark = pytest.mark.gpu


def _filled(w, n_chunks):
    from rolling_kv_cache_amd import KVCache
    gc = KVCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w, torch.bfloat16,
                 raw_keys=w.raw_keys)
    for i in range(n_chunks):
        _, k, v = chunk_inputs(w, i)
        gc.append(dev(k, w), dev(v, w), w.chunk_start_frame(i))
    return gc


def _same(gc, tail, weight, tag):
    ref = gc.relax_scores(tail, weight).cpu().numpy()
    got = gc.relax_scores_noalloc(tail, weight).cpu().numpy()
    assert ref.shape == got.shape and np.isfinite(ref).all(), tag
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), f"{tag}: {np.abs(ref - got).max()}"
    log(f"  {tag}: {ref.shape[0]} candidates equal")


def test_relax_noalloc_matches_caller_scratch():
    from rolling_kv_cache_amd import KVCError, lib
    # the Relax Forcing shape: 12 heads x 128, 1560-token frames, 3 sink + 18 window frames, full
    big = Workload("rnoalloc", 250, 12, 128, "bf16", 30, 52, 3, 18, (3,) * 7)
    gc = _filled(big, 7)
    _same(gc, 2, 0.5, "full 3+18-frame cache")
    # then a smaller input on the same GPU: fewer heads, frames and candidates
    small = Workload("rnoalloc_s", 251, 4, 128, "bf16", 9, 60, 1, 8, (2,) * 4)
    gs = _filled(small, 4)
    _same(gs, 3, 0.3, "smaller cache after the full one")
    _same(gc, 1, 0.8, "full cache again")
    # raw keys: the placed key planes share the held scratch
    raw = Workload("rnoalloc_r", 252, 6, 128, "bf16", 9, 60, 2, 10, (2,) * 6, raw_keys=True)
    gr = _filled(raw, 6)
    gr.retime(-3, clamp0=True)
    _same(gr, 2, 0.5, "raw-key cache")
    # a cache whose scratch exceeds the held array: refused with ENOMEM, nothing enqueued
    huge = Workload("rnoalloc_h", 253, 400, 128, "bf16", 4, 4, 3, 18, (3,) * 7)
    gh = _filled(huge, 7)
    need = int(lib.kvc_relax_scratch_bytes(gh._h))
    assert need > 8 << 20
    with pytest.raises(KVCError) as e:
        gh.relax_scores_noalloc(2, 0.5)
    assert e.value.code == 2
    _same(gs, 2, 0.5, "smaller cache after the refusal")
