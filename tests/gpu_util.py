"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import contextlib
import sys
import time

import numpy as np
import torch

ATT_MAX_ABS = 2e-2      # attention tolerance: max-abs ...
ATT_REL_RMS = 5e-3      # ... and relative RMS against the fp32 oracle


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def dev(x: np.ndarray, w) -> torch.Tensor:
    """Upload a bf16-valued float32 array exactly (no rounding happens for bf16-representable values)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=torch_dtype(w))


def new_cache(w, compact=False, split=False):
    from rolling_kv_cache_amd import KVCache
    return KVCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w,
                   dtype=torch_dtype(w), bank_frames=w.bank_frames, compact=compact, raw_keys=w.raw_keys,
                   memory=w.memory, split_attend=split)


def bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bits of bf16-valued float32 (upper half) or of float32."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16) if dtype == "bf16" else u


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def assert_state_equal(gc, oc, w, tag=""):
    """GPU cache (logical-order export) == oracle state, bit for bit."""
    info = gc.info()
    assert info["n_valid"] == oc.n, (tag, info["n_valid"], oc.n)
    assert info["global_end"] == oc.global_end, tag
    assert info["sink_filled"] == oc.n_sink, tag
    st = gc.export()
    t = st["t"].cpu().numpy()
    g = st["g"].cpu().numpy()
    assert np.array_equal(g, oc.g), f"{tag}: g differs"
    assert np.array_equal(t, oc.t), f"{tag}: t differs"
    kb = gpu_bits(st["K"])
    ko = bits(oc.K, w.dtype)
    if not np.array_equal(kb, ko):
        bad = np.argwhere(kb != ko)
        raise AssertionError(f"{tag}: K differs at {bad.shape[0]} elements, first {bad[:5].tolist()}")
    vb = gpu_bits(st["V"])
    vo = bits(oc.V, w.dtype)
    if not np.array_equal(vb, vo):
        bad = np.argwhere(vb != vo)
        raise AssertionError(f"{tag}: V differs at {bad.shape[0]} elements, first {bad[:5].tolist()}")
    ht, hg = gc.slot_times()
    assert np.array_equal(ht, oc.t) and np.array_equal(hg, oc.g), f"{tag}: host mirror differs"


def check_attention(out: np.ndarray, ref: np.ndarray, tag="", max_abs=ATT_MAX_ABS, rel_rms=ATT_REL_RMS):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(out - ref)
    mx = float(err.max())
    rr = float(np.sqrt(np.sum((out - ref) ** 2) / np.sum(ref ** 2)))
    assert np.isfinite(out).all(), f"{tag}: non-finite output"
    assert mx <= max_abs and rr <= rel_rms, f"{tag}: max_abs {mx:.3e} rel_rms {rr:.3e}"
    return mx, rr


class Timer:
    def __init__(self, tag):
        self.tag = tag

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log(f"  [{self.tag}] {time.time() - self.t:.1f}s")


@contextlib.contextmanager
def paths(gc, **kw):
    """Run the body with kernel paths selected on cache gc (kvc_set_paths), then restore the defaults."""
    gc.set_paths(**kw)
    try:
        yield
    finally:
        gc.set_paths()
