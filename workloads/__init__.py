"""Seeded synthetic workloads shared by the GPU path's tests/bench and the oracle.

This module holds workload *shapes* and a seeded random generator only; it
contains none of the cache method's arithmetic (no RoPE, no eviction, no
attention, no schedules derived from the method).

Shapes stand in for the pages' workloads:
  * Wan 480x832 video -> 60x104/4 = 1560 latent tokens per frame on a 30x52
    grid (LingBot-World 2.0 sliding-window article, "how the window rolls when
    full", worked example).
  * Wan-1.3B self-attention: 12 heads x 128 (Causal-Forcing KV-cache article,
    section 3 "KV Cache", cache tensor shape); 14B-class: 40 heads x 128.
  * 3-latent-frame chunks (LingBot article, "chunked inference";
    rCM length-extrapolation article, --chunk_t 3).
Every q/k/v element is i.i.d. N(0,1): float32 standard_normal from
numpy.random.default_rng([cfg_id, chunk, tensor_id]) (tensor_id 0=q, 1=k,
2=v), then rounded to bfloat16 by torch's CPU cast for bf16 workloads. The
arrays returned are float32 holding bf16-representable values, laid out
[tokens, heads, head_dim] (the pages' [B, L, H, D] with B=1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    heads: int
    head_dim: int
    dtype: str              # "bf16" or "f32"
    grid_h: int
    grid_w: int
    sink_frames: int        # kvc_create sink_frames
    window_frames: int      # kvc_create window_frames (rolling part, incl. current chunk)
    chunk_frames: tuple     # frames per chunk, in stream order
    bank_frames: int = 0    # raw-block bank captured during the first appends (Rolling Sink)
    # synthetic shot boundaries: chunk indices before which a hard cut happens
    cut_chunks: tuple = field(default_factory=tuple)
    # raw-key cache (keys kept un-rotated in time, placed at attention time)
    raw_keys: bool = False
    # MemRoPE memory tokens (alpha_long, alpha_short) on a raw-key cache, or None
    memory: tuple | None = None

    @property
    def frame_seqlen(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def capacity(self) -> int:
        return (self.sink_frames + self.window_frames) * self.frame_seqlen

    @property
    def n_chunks(self) -> int:
        return len(self.chunk_frames)

    @property
    def total_frames(self) -> int:
        return int(sum(self.chunk_frames))

    def chunk_start_frame(self, i: int) -> int:
        return int(sum(self.chunk_frames[:i]))


WORKLOADS = {
    # 2 heads x 64, fp32, 4x4 latent grid, 1-frame chunks, sink 1 + window 4, 12 chunks
    "tiny": Workload("tiny", 0, 2, 64, "f32", 4, 4, 1, 4, (1,) * 12),
    # Wan-1.3B single layer, global cache of 21 frames, 7 chunks of 3, no eviction
    "c2": Workload("c2", 1, 12, 128, "bf16", 30, 52, 0, 21, (3,) * 7),
    # 14B-class: 40 heads, 6 sink frames + 12-frame rolling part = 18-frame window
    # (28080 tokens), 91 latent frames (361 pixel frames) = 30 chunks of 3 + 1
    "c3": Workload("c3", 2, 40, 128, "bf16", 30, 52, 6, 12, (3,) * 30 + (1,)),
    # Rolling Sink: 15 sink frames (5 blocks) + 6 rolling (recent + current block),
    # bank = first 6 blocks, 257 latent frames (1025 pixel frames) = 85 x 3 + 2
    "c4": Workload("c4", 3, 12, 128, "bf16", 30, 52, 15, 6, (3,) * 85 + (2,), bank_frames=18),
    # Infinity-RoPE: 1 sink block + 18 frames, 140 latent frames = 46 x 3 + 2;
    # shots 5 s | 10 s# | 10 s# | 10 s# at 16 fps (4 latent frames per second):
    # cuts at latent 20/60/100, rounded up to chunk starts 21/60/102 -> chunks 7, 20, 34
    "c5a": Workload("c5a", 4, 12, 128, "bf16", 30, 52, 3, 18, (3,) * 46 + (2,),
                    cut_chunks=(7, 20, 34)),
    # Deep-Forcing token compaction on the same shape, absolute times
    "c5b": Workload("c5b", 5, 12, 128, "bf16", 30, 52, 3, 18, (3,) * 46 + (2,)),
    # Relax Forcing frame selection on the same shape (sink 3 + History 4 + Tail 2 frames kept)
    "c5c": Workload("c5c", 6, 12, 128, "bf16", 30, 52, 3, 18, (3,) * 46 + (2,)),
    # MemRoPE: sliding window + sink on a raw-key cache whose evicted frames fold into long/short
    # EMA memory tokens (rates 0.9 / 0.5)
    "c6": Workload("c6", 7, 12, 128, "bf16", 30, 52, 3, 18, (3,) * 46 + (2,), raw_keys=True, memory=(0.9, 0.5)),
    # Infinity-RoPE on a raw-key cache: every per-chunk shift is an index update
    "c5a_raw": Workload("c5a_raw", 4, 12, 128, "bf16", 30, 52, 3, 18, (3,) * 46 + (2,),
                        cut_chunks=(7, 20, 34), raw_keys=True),
}


def _to_bf16_values(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)
    return t.numpy()


def gen(cfg_id: int, chunk: int, tensor_id: int, n_tokens: int, heads: int,
        head_dim: int, dtype: str) -> np.ndarray:
    """i.i.d. N(0,1) [n_tokens, heads, head_dim] float32 (bf16-exact when dtype=='bf16')."""
    rng = np.random.default_rng([cfg_id, chunk, tensor_id])
    x = rng.standard_normal((n_tokens, heads, head_dim), dtype=np.float32)
    if dtype == "bf16":
        x = _to_bf16_values(x)
    return np.ascontiguousarray(x)


def chunk_inputs(w: Workload, chunk: int, tensors=(TENSOR_Q, TENSOR_K, TENSOR_V), frames=None):
    """The seeded q/k/v of one chunk of workload w (tokens = frames * frame_seqlen); `frames` overrides the
    schedule's frame count (and allows chunk ids past the schedule)."""
    n = (w.chunk_frames[chunk] if frames is None else frames) * w.frame_seqlen
    return tuple(gen(w.cfg_id, chunk, tid, n, w.heads, w.head_dim, w.dtype) for tid in tensors)


def small_variant(w: Workload, heads: int | None = None, grid=None, n_chunks: int | None = None) -> Workload:
    """Same schedule family at a reduced size (fewer heads / smaller grid / fewer chunks)."""
    gh, gw = grid if grid is not None else (w.grid_h, w.grid_w)
    cf = w.chunk_frames if n_chunks is None else w.chunk_frames[:n_chunks]
    return Workload(w.name + "_small", w.cfg_id + 100, heads or w.heads, w.head_dim, w.dtype,
                    gh, gw, w.sink_frames, w.window_frames, tuple(cf), w.bank_frames,
                    tuple(c for c in w.cut_chunks if c < len(cf)), w.raw_keys, w.memory)


DENOISE_STEPS = 4        # the 4-step distilled models' timesteps, then one commit pass at t = 0


def denoise_inputs(w: Workload, chunk: int, step: int, layer: int = 0, frames=None):
    """q/k/v of one denoising step (0..DENOISE_STEPS-1, then DENOISE_STEPS = the clean commit pass) of one
    layer for chunk `chunk`: a seeded stream of its own per (layer, chunk, step)."""
    n = (w.chunk_frames[chunk] if frames is None else frames) * w.frame_seqlen
    sub = 1_000_000 + (layer * 10_000 + chunk) * 8 + step
    return tuple(gen(w.cfg_id, sub, tid, n, w.heads, w.head_dim, w.dtype) for tid in (TENSOR_Q, TENSOR_K, TENSOR_V))
