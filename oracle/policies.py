"""Cache policies of the pages, driven step by step over a chunk stream (oracle side).

Each ``Run`` owns an OracleCache and exposes ``step(i, q, k, v, ...)`` which
performs chunk i's cache operations and returns its attention output.

* SlidingWindowRun -- FIFO window + pinned sink, or a global cache when the
  capacity covers the whole stream (LingBot-World 2.0 article; rCM article,
  strategy 1).  Chunk i is written at its absolute start frame.
* RollingSinkRun -- Rolling Sink (Rolling Sink summary, "method step details";
  rCM article, strategy 2): context Cat(x[0,S), x[i-(K-S), i)) with the sink's
  time indices sliding to [i-K, i-K+S) and its content taken from
  Roll(x[0,K)), forward on even cycles and reversed on odd cycles.
* InfinityRopeRun -- Infinity-RoPE (rCM article, strategy 3): the newest block
  always sits at the end of the trained horizon f_limit, older blocks shift
  back together, times below 0 clamp to 0, KV flush keeps the sink + last
  block, a RoPE cut adds an artificial jump of rope_cut_delta frames.
* DeepForcingRun -- Deep Forcing (rCM article, strategy 4): keep Deep Sink +
  Top-C tokens by attention score + Recent Tail, compact, then close the time
  holes of the sink and compressed regions in place.
* RelaxForcingRun -- Relax Forcing (rCM article, strategy 5): the same Sink +
  kept history + Tail shape, with whole History frames chosen by cosine
  alignment with the Tail plus a complement bonus (see relax.py).

Readings (the pages leave these open): a block is one chunk of 3 frames; for
Rolling Sink the segment of Roll read at step i starts at i-K, so at i = K the
context is the plain cache of blocks 0..K-1 and the method is continuous when
the bank fills; the Roll endpoint is repeated (0..5, 5..0, 0..5, ...); for
Infinity-RoPE the newest block occupies [f_limit-F, f_limit), the clamp is per
entry and the sink is shifted and clamped with the rest; for Deep Forcing the
query window is the previous chunk's queries at their own times, ties go to
the lower logical index, and one time delta closes each region's gap.
"""
from __future__ import annotations

import numpy as np

from .cache import OracleCache
from .relax import top_frames


def roll_index(n: int, K: int) -> int:
    """Block of x[0,K) found at position n of Roll(x[0,K)): forward on even cycles, reverse on odd."""
    c, r = divmod(n, K)
    return r if c % 2 == 0 else K - 1 - r


def _cache_for(w):
    return OracleCache(w.sink_frames, w.window_frames, w.frame_seqlen, w.heads, w.head_dim, w.grid_w,
                       w.dtype, w.bank_frames, raw_keys=getattr(w, "raw_keys", False),
                       memory=getattr(w, "memory", None))


class SlidingWindowRun:
    def __init__(self, w):
        self.w = w
        self.cache = _cache_for(w)

    def step(self, i, q, k, v, rows=None, f64=False):
        F = self.w.chunk_frames[i]
        t0 = self.w.chunk_start_frame(i)
        self.cache.append(k, v, F, t0)
        return self.cache.attend(q, F, t0, rows=rows, f64=f64)


class RollingSinkRun:
    """K cached blocks (excluding the current one), S of them sink; blocks of `block` frames."""

    def __init__(self, w, block=3):
        self.w = w
        self.block = block
        self.S_blocks = w.sink_frames // block
        self.K = w.bank_frames // block
        self.cache = _cache_for(w)

    def pushed_block(self, i):
        """(bank block, time block) pushed into the sink at step i, or None."""
        if i < self.K + 1:
            return None
        n = i - (self.K - self.S_blocks) - 1
        return roll_index(n, self.K), n

    def step(self, i, q, k, v, rows=None, f64=False):
        F = self.w.chunk_frames[i]
        t0 = self.w.chunk_start_frame(i)
        p = self.pushed_block(i)
        if p is not None:
            b, n = p
            self.cache.sink_push(b * self.block, self.block, n * self.block)
        self.cache.append(k, v, F, t0)
        return self.cache.attend(q, F, t0, rows=rows, f64=f64)


class InfinityRopeRun:
    def __init__(self, w, f_limit=21, rope_cut_delta=21):
        self.w = w
        self.f_limit = f_limit
        self.cut = rope_cut_delta
        self.cache = _cache_for(w)

    def step(self, i, q, k, v, rows=None, f64=False):
        c = self.cache
        F = self.w.chunk_frames[i]
        if i >= 1:
            if i in self.w.cut_chunks:
                n_new = c.newest[1]
                keep = np.concatenate([np.arange(c.n_sink), np.arange(c.n - n_new, c.n)])
                c.compact(keep)
                c.retime(-(F + self.cut), True, 0, c.n)
            else:
                c.retime(-F, True, 0, c.n)
        t0 = self.f_limit - F
        c.append(k, v, F, t0)
        return c.attend(q, F, t0, rows=rows, f64=f64)


class DeepForcingRun:
    def __init__(self, w, top_frames=4, recent_frames=2):
        self.w = w
        self.C = top_frames * w.frame_seqlen
        self.R = recent_frames * w.frame_seqlen
        self.cache = _cache_for(w)
        self.last = {}

    def needs_compaction(self, i):
        return self.cache.n + self.w.chunk_frames[i] * self.w.frame_seqlen > self.cache.C_tok

    def select(self, scores):
        """Keep set from per-entry scores: whole sink, Top-C candidates, recent tail."""
        c = self.cache
        n = c.n
        cand = np.arange(c.S_tok, n - self.R, dtype=np.int64)
        order = np.argsort(-np.asarray(scores)[cand], kind="stable")   # ties: lower index first
        top = np.sort(cand[order[:self.C]])
        return np.concatenate([np.arange(c.S_tok, dtype=np.int64), top, np.arange(n - self.R, n, dtype=np.int64)])

    def step(self, i, q, k, v, q_prev=None, keep_override=None, rows=None, f64=False):
        c = self.cache
        w = self.w
        F = w.chunk_frames[i]
        t0 = w.chunk_start_frame(i)
        self.last = {}
        if self.needs_compaction(i):
            Fp = w.chunk_frames[i - 1]
            tp = w.chunk_start_frame(i - 1)
            scores = c.score(q_prev, Fp, [tp + f for f in range(Fp)], f64=f64)
            keep = self.select(scores)
            self.last = {"scores": scores, "keep": keep}
            if keep_override is not None:
                keep = np.asarray(keep_override, dtype=np.int64)
            c.compact(keep)
            d_c, d_s = _close_gaps(c, keep.shape[0] - c.S_tok - self.R)
            self.last.update({"d_c": d_c, "d_s": d_s})
        c.append(k, v, F, t0)
        return c.attend(q, F, t0, rows=rows, f64=f64)


def _close_gaps(c, n_comp):
    """After compaction to sink + n_comp compressed entries + tail: shift the compressed region so it ends
    one frame before the tail starts, then the sink so it ends one frame before the compressed region
    starts (one time delta per region, no clamp)."""
    comp = (c.S_tok, c.S_tok + n_comp)
    d_c = (int(c.t[comp[1]:c.n].min()) - 1) - int(c.t[comp[0]:comp[1]].max())
    c.retime(d_c, False, comp[0], comp[1])
    d_s = (int(c.t[comp[0]:comp[1]].min()) - 1) - int(c.t[0:c.S_tok].max())
    c.retime(d_s, False, 0, c.S_tok)
    return d_c, d_s


class RelaxForcingRun:
    """Relax Forcing (rCM article, strategy 5): Sink + History + Tail.  On the same trigger as Deep
    Forcing (the next chunk does not fit), the History candidates -- whole frames between the sink and
    the Tail (the last recent_frames frames) -- are scored by cosine alignment with the Tail plus the
    complement bonus (relax_frame_scores), the Top-K frames are kept whole, the cache is compacted and
    the time gaps are closed as for Deep Forcing."""

    def __init__(self, w, top_frames=4, recent_frames=2, weight=0.5):
        self.w = w
        self.K = top_frames
        self.Rf = recent_frames
        self.R = recent_frames * w.frame_seqlen
        self.weight = weight
        self.cache = _cache_for(w)
        self.last = {}

    def needs_compaction(self, i):
        return self.cache.n + self.w.chunk_frames[i] * self.w.frame_seqlen > self.cache.C_tok

    def select(self, scores):
        c = self.cache
        S = self.w.frame_seqlen
        frames = c.n_sink // S + top_frames(scores, self.K)
        hist = (frames[:, None] * S + np.arange(S)[None, :]).reshape(-1)
        return np.concatenate([np.arange(c.n_sink), hist, np.arange(c.n - self.R, c.n)]).astype(np.int64)

    def step(self, i, q, k, v, keep_override=None, rows=None, f64=False, **_):
        c = self.cache
        w = self.w
        F = w.chunk_frames[i]
        t0 = w.chunk_start_frame(i)
        self.last = {}
        if self.needs_compaction(i):
            scores = c.relax_scores(self.Rf, self.weight)
            keep = self.select(scores)
            self.last = {"scores": scores, "keep": keep}
            if keep_override is not None:
                keep = np.asarray(keep_override, dtype=np.int64)
            c.compact(keep)
            d_c, d_s = _close_gaps(c, keep.shape[0] - c.S_tok - self.R)
            self.last.update({"d_c": d_c, "d_s": d_s})
        c.append(k, v, F, t0)
        return c.attend(q, F, t0, rows=rows, f64=f64)


class DenoiseLoopRun:
    """Chunk-wise denoising over a cache per layer (Causal-Forcing article, section 4, block-wise denoising;
    LingBot-World 2.0 article: after each block's sampling steps a clean pass at t = 0 writes the block's
    KV).  Per chunk and layer: step 0 writes the chunk's frames (rolling the window), steps 1..steps-1 and
    the commit pass re-write the same frames in place (no new content, no roll), and every pass attends.
    The plain sliding-window schedule; the chunk is written at its absolute start frame."""

    def __init__(self, w, layers, steps=4):
        self.w, self.L, self.steps = w, layers, steps
        self.caches = [_cache_for(w) for _ in range(layers)]

    def step(self, i, layer, s, q, k, v, rows=None, f64=False):
        c = self.caches[layer]
        F = self.w.chunk_frames[i]
        t0 = self.w.chunk_start_frame(i)
        c.append(k, v, F, t0, replace_newest=s > 0)
        return c.attend(q, F, t0, rows=rows, f64=f64)


def make_run(w):
    """Run of a workload by name prefix; anything else is a plain sliding window / global cache."""
    return {"c4": RollingSinkRun, "c5a": InfinityRopeRun, "c5b": DeepForcingRun, "c5c": RelaxForcingRun}.get(
        w.name.split("_")[0], SlidingWindowRun)(w)
