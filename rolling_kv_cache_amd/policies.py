"""Cache policies of the pages as host-side schedules over a GPU ``KVCache``.

Only integer bookkeeping happens here (which frames go where, at which time
index, which entries to keep); every tensor operation is a libkvc call.

A schedule object needs ``chunk_frames`` (frames per chunk, in stream order),
``frame_seqlen`` and, for Infinity-RoPE, ``cut_chunks``.

* SlidingWindow -- FIFO window with a pinned sink, or a global cache when the
  capacity covers the stream (LingBot-World 2.0 article, "how the window rolls
  when full", "sink_size attention sink"; rCM article, strategy 1): chunk i is
  appended at its absolute start frame and its queries attend.
* RollingSink -- Rolling Sink (Rolling Sink summary, "method step details";
  rCM article, strategy 2): once the bank of the first K blocks is complete,
  each step pushes block Roll(n) of the bank into the sink at time n (block
  units), n = i - (K - S) - 1, so the sink covers time blocks [i-K, i-K+S);
  Roll runs forward on even cycles and backward on odd ones.
* InfinityRope -- Infinity-RoPE (rCM article, strategy 3): every older entry
  shifts back by the new chunk's length with a clamp at 0, the newest chunk
  is written at [f_limit - F, f_limit); at a shot boundary the cache is
  flushed to the sink plus the last chunk and then cut by rope_cut_delta.
* DeepForcing -- Deep Forcing (rCM article, strategy 4): when the next chunk
  does not fit, score entries by the attention mass the previous chunk's
  queries give them, keep the sink, the Top-C candidates and the recent tail,
  compact, and close the time gaps of the compressed region and the sink.
* RelaxForcing -- Relax Forcing (rCM article, strategy 5): the same shape of
  kept cache, with whole History frames chosen by cosine alignment of their
  keys with the Tail plus a complement bonus.
"""
from __future__ import annotations

import numpy as np
import torch


def roll_block(n: int, K: int) -> int:
    """Bank block at position n of the rolled bank order (forward cycle, then backward cycle, ...)."""
    cycle, pos = divmod(n, K)
    return pos if cycle % 2 == 0 else K - 1 - pos


def _start_frame(sched, i):
    return int(sum(sched.chunk_frames[:i]))


class SlidingWindow:
    def __init__(self, cache, sched):
        self.cache, self.sched = cache, sched

    def step(self, i, q, k, v, **_):
        t0 = _start_frame(self.sched, i)
        self.cache.append(k, v, t0)
        return self.cache.attend(q, t0)


class RollingSink:
    def __init__(self, cache, sched, block_frames=3, cache_blocks=6, sink_blocks=5):
        self.cache, self.sched = cache, sched
        self.B, self.K, self.Sb = block_frames, cache_blocks, sink_blocks

    def push_for(self, i):
        """(bank block, time block) pushed at step i, None before the bank fills."""
        if i <= self.K:
            return None
        n = i - (self.K - self.Sb) - 1
        return roll_block(n, self.K), n

    def step(self, i, q, k, v, **_):
        p = self.push_for(i)
        if p is not None:
            blk, n = p
            self.cache.sink_push(blk * self.B, self.B, n * self.B)
        t0 = _start_frame(self.sched, i)
        self.cache.append(k, v, t0)
        return self.cache.attend(q, t0)


class InfinityRope:
    def __init__(self, cache, sched, f_limit=21, rope_cut_delta=21):
        self.cache, self.sched = cache, sched
        self.f_limit, self.cut = f_limit, rope_cut_delta

    def step(self, i, q, k, v, **_):
        c = self.cache
        F = self.sched.chunk_frames[i]
        if i > 0:
            info = c.info()
            if i in self.sched.cut_chunks:
                n, ns = info["n_valid"], info["sink_filled"]
                last = info["newest_frames"] * self.sched.frame_seqlen
                c.compact(np.concatenate([np.arange(ns), np.arange(n - last, n)]))   # KV flush
                c.retime(-(F + self.cut), clamp0=True)                               # RoPE cut
            else:
                c.retime(-F, clamp0=True)                                            # block-relative shift
        t0 = self.f_limit - F
        c.append(k, v, t0)
        return c.attend(q, t0)


class DeepForcing:
    """Every attend keeps its rows' softmax normalisers (kvc_attend_stats); the scoring of the previous
    chunk's queries, which sees the cache that attention saw, then runs only its columns pass
    (kvc_score_with_stats).  use_row_stats=False scores with both passes (kvc_score)."""

    def __init__(self, cache, sched, top_frames=4, recent_frames=2, use_row_stats=True):
        self.cache, self.sched = cache, sched
        self.C = top_frames * sched.frame_seqlen
        self.R = recent_frames * sched.frame_seqlen
        self.last = {}
        self.row_stats = None
        if use_row_stats:
            rows = max(sched.chunk_frames) * sched.frame_seqlen
            self.row_stats = torch.empty(cache.H * rows, dtype=torch.float32, device=cache.device)

    def keep_set(self, scores: np.ndarray, n: int, sink: int) -> np.ndarray:
        cand = np.arange(sink, n - self.R)
        # stable sort on descending score: equal scores keep the lower logical index first
        order = np.argsort(-scores[cand], kind="stable")
        top = np.sort(cand[order[:self.C]])
        return np.concatenate([np.arange(sink), top, np.arange(n - self.R, n)]).astype(np.int32)

    def step(self, i, q, k, v, q_prev=None, **_):
        c = self.cache
        S = self.sched.frame_seqlen
        F = self.sched.chunk_frames[i]
        info = c.info()
        self.last = {}
        if info["n_valid"] + F * S > info["capacity"]:
            Fp = self.sched.chunk_frames[i - 1]
            tp = _start_frame(self.sched, i - 1)
            scores = c.score(q_prev, [tp + f for f in range(Fp)], row_stats=self.row_stats)
            scores = scores.cpu().numpy().astype(np.float64)
            sink = info["sink_tokens"]
            keep = self.keep_set(scores, info["n_valid"], sink)
            self.last = {"scores": scores, "keep": keep}
            c.compact(keep)
            d_c, d_s = _close_gaps(c, sink, keep.shape[0] - sink - self.R)
            self.last.update({"d_c": d_c, "d_s": d_s})
        t0 = _start_frame(self.sched, i)
        c.append(k, v, t0)
        return c.attend(q, t0, row_stats=self.row_stats)


class RelaxForcing:
    """Relax Forcing (rCM article, strategy 5): on the same trigger as Deep Forcing, score the whole
    frames between the sink and the Tail (the last recent_frames frames) by cosine alignment with the
    Tail plus a complement bonus (kvc_relax_scores), keep the Top-K frames whole with the sink and the
    Tail, compact, and close the time gaps as Deep Forcing does."""

    def __init__(self, cache, sched, top_frames=4, recent_frames=2, weight=0.5):
        self.cache, self.sched = cache, sched
        self.K, self.Rf, self.weight = top_frames, recent_frames, weight
        self.last = {}

    def keep_set(self, scores: np.ndarray, n: int, sink: int) -> np.ndarray:
        S = self.sched.frame_seqlen
        order = np.argsort(-scores, kind="stable")            # equal scores keep the lower frame first
        frames = sink // S + np.sort(order[:self.K])
        hist = (frames[:, None] * S + np.arange(S)[None, :]).reshape(-1)
        return np.concatenate([np.arange(sink), hist, np.arange(n - self.Rf * S, n)]).astype(np.int32)

    def step(self, i, q, k, v, **_):
        c = self.cache
        S = self.sched.frame_seqlen
        F = self.sched.chunk_frames[i]
        info = c.info()
        self.last = {}
        if info["n_valid"] + F * S > info["capacity"]:
            scores = c.relax_scores(self.Rf, self.weight).cpu().numpy().astype(np.float64)
            sink = info["sink_filled"]
            keep = self.keep_set(scores, info["n_valid"], sink)
            self.last = {"scores": scores, "keep": keep}
            c.compact(keep)
            d_c, d_s = _close_gaps(c, sink, keep.shape[0] - sink - self.Rf * S)
            self.last.update({"d_c": d_c, "d_s": d_s})
        t0 = _start_frame(self.sched, i)
        c.append(k, v, t0)
        return c.attend(q, t0)


class DenoiseLoop:
    """Chunk-wise denoising over one cache per layer (Causal-Forcing article, section 4; LingBot-World 2.0
    article): for each chunk, pass 0 writes the chunk's frames (rolling the window), passes 1..steps-1 and
    the clean commit pass at t = 0 re-write them in place (KVC_APPEND_REPLACE_NEWEST), and each pass
    attends.  Inside a pass the layers run in order, each with its own q/k/v."""

    def __init__(self, caches, sched, steps=4):
        self.caches, self.sched, self.steps = caches, sched, steps

    def pass_layer(self, i, layer, s, q, k, v):
        c = self.caches[layer]
        t0 = _start_frame(self.sched, i)
        c.append(k, v, t0, replace_newest=s > 0)
        return c.attend(q, t0)


def _close_gaps(c, sink, n_comp):
    """Shift the compressed region to end one frame before the tail, then the sink to end one frame before
    the compressed region (one time delta each, no clamp)."""
    t, _ = c.slot_times()
    lo, hi = sink, sink + n_comp
    d_c = (int(t[hi:].min()) - 1) - int(t[lo:hi].max())
    c.retime(d_c, False, lo, hi)
    t, _ = c.slot_times()
    d_s = (int(t[lo:hi].min()) - 1) - int(t[:sink].max())
    c.retime(d_s, False, 0, sink)
    return d_c, d_s


def driver_for(name: str):
    """Policy of a workload by name prefix; anything else is a plain sliding window / global cache."""
    return {"c4": RollingSink, "c5a": InfinityRope, "c5b": DeepForcing, "c5c": RelaxForcing}.get(name.split("_")[0], SlidingWindow)
