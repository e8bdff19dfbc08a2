"""Oracle cache state machine: explicit concatenation, physical left-shift eviction.

Logical order is: sink entries (oldest first), then the rolling window (oldest
first, newest chunk last).  Every entry keeps its stored key (what the cache
holds: the rotated key, bf16-rounded for bf16 caches), its value, its time
index t, its global token index g, its raw key (for the fp64 semantic
reference) and its token-in-frame index (for h/w positions).

Sources:
  * capacity fixed at creation: kv_size = frame_seqlen * local_attn_size
    (LingBot-World 2.0 article, "chunked inference"); memory precomputed by
    cache_max_len() (rCM length-extrapolation article, intro).
  * roll rule (LingBot article, "how the window rolls when full"): when
    new + local_end > kv_size, num_evicted = new + local_end - kv_size; the
    contents after the sink are shifted left by num_evicted, the sink never
    moves, the roped K/V of the new block are written at the tail.  The '+'
    and '>' lost in the page's extraction are restored; the page's own worked
    numbers (a 4680-token block evicts an equal 4680 from a full 28080 cache)
    fix that reading.
  * the sink is the first sink_size frames of the stream (LingBot article,
    "sink_size attention sink").
  * the newest block may be written again in place by later denoising steps
    before the clean commit; rolling only happens for genuinely new content
    (LingBot article, roll condition; Causal-Forcing article, section 4).
  * in-place time re-rotation of cached keys (rCM article, Deep Forcing:
    rope_time_delta_), clamping negative time indices to 0 (rCM article,
    Infinity-RoPE item 2), KV flush keeping sink + last block (item 3).
  * Rolling Sink bank of the first K blocks and the sink refilled from it
    (rCM article, strategy 2; Rolling Sink summary, "method step details").
"""
from __future__ import annotations

import numpy as np

from .bf16 import round_to_bf16
from .rope import band_split, rotate_f32, token_positions
from .attention import attention_f32, attention_f64
from .score import attention_mass_scores, row_normalisers
from .relax import relax_frame_scores


class OracleError(ValueError):
    pass


class OracleCache:
    def __init__(self, sink_frames, window_frames, frame_seqlen, heads, head_dim, grid_w,
                 dtype="bf16", bank_frames=0, raw_keys=False, memory=None):
        self.S = frame_seqlen
        self.H = heads
        self.D = head_dim
        self.grid_w = grid_w
        self.dtype = dtype
        self.S_tok = sink_frames * frame_seqlen
        self.W_tok = window_frames * frame_seqlen
        self.C_tok = self.S_tok + self.W_tok
        self.bank_tok = bank_frames * frame_seqlen
        # raw-key mode (MemRoPE, rCM article): keys are kept un-rotated in time and placed at their
        # current time when attended; a retime then only changes t
        self.raw_keys = raw_keys
        # MemRoPE memory tokens (rCM article): (alpha_long, alpha_short) or None
        if memory is not None and not raw_keys:
            raise OracleError("memory tokens need a raw-key cache")
        self.memory = memory
        self.mem_k = np.zeros((2, frame_seqlen, heads, head_dim), np.float32)   # EMA state, fp32
        self.mem_v = np.zeros((2, frame_seqlen, heads, head_dim), np.float32)
        self.mem_frames = 0                                                     # frames folded so far
        e = np.zeros((0, heads, head_dim), np.float32)
        self.K, self.V, self.Kraw = e.copy(), e.copy(), e.copy()
        self.t = np.zeros(0, np.int64)
        self.g = np.zeros(0, np.int64)
        self.tok = np.zeros(0, np.int64)          # token index inside its frame
        self.n_sink = 0
        self.global_end = 0
        self.newest = None                        # (g0, n_tokens, frames)
        self.bank_K = np.zeros((self.bank_tok, heads, head_dim), np.float32)
        self.bank_V = np.zeros((self.bank_tok, heads, head_dim), np.float32)

    # ------------------------------------------------------------------ helpers
    @property
    def n(self) -> int:
        return int(self.t.shape[0])

    def _store(self, x):
        return round_to_bf16(x) if self.dtype == "bf16" else np.asarray(x, np.float32)

    def _rotate(self, x, t, tok, bands=(True, True, True)):
        h = tok // self.grid_w
        w = tok % self.grid_w
        return self._store(rotate_f32(x, t, h, w, bands))

    def _stored_key(self, k, t, tok):
        """The key as the cache stores it: fully rotated, or (raw-key mode) with only the height and
        width bands rotated -- those positions never change -- and the time band left raw."""
        if self.raw_keys:
            return self._rotate(k, t, tok, bands=(False, True, True))
        return self._rotate(k, t, tok)

    def attention_keys(self):
        """Keys as attention sees them: the stored keys, or (raw-key mode) the raw keys freshly rotated at
        every entry's current time (the plain definition, from Kraw)."""
        if self.raw_keys:
            return self._rotate(self.Kraw, self.t, self.tok)
        return self.K

    def _take(self, idx):
        idx = np.asarray(idx, dtype=np.int64)
        for name in ("K", "V", "Kraw", "t", "g", "tok"):
            setattr(self, name, getattr(self, name)[idx])

    def _cat(self, parts):
        for name in ("K", "V", "Kraw", "t", "g", "tok"):
            setattr(self, name, np.concatenate([p[name] for p in parts], axis=0))

    def _entries(self, lo, hi):
        return {n: getattr(self, n)[lo:hi] for n in ("K", "V", "Kraw", "t", "g", "tok")}

    # ------------------------------------------------------------------ append
    def append(self, k, v, frames, t0, replace_newest=False):
        """Write `frames` new frames at times t0 .. t0+frames-1 (rotating k), FIFO-evicting if full."""
        N = frames * self.S
        k = np.asarray(k, np.float32)
        v = np.asarray(v, np.float32)
        if k.shape != (N, self.H, self.D) or v.shape != k.shape:
            raise OracleError("k/v shape")
        if N > self.W_tok:
            raise OracleError("chunk larger than the rolling window")
        t, _, _ = token_positions(N, self.S, self.grid_w, t0)
        tok = np.arange(N, dtype=np.int64) % self.S
        Kst = self._stored_key(k, t, tok)
        if replace_newest:
            if self.newest is None or self.newest[2] != frames:
                raise OracleError("no newest chunk of that size to replace")
            g0 = self.newest[0]
            idx = np.nonzero((self.g >= g0) & (self.g < g0 + N))[0]
            if idx.shape[0] != N:
                raise OracleError("newest chunk no longer whole")
            order = np.argsort(self.g[idx], kind="stable")
            idx = idx[order]
            self.K[idx], self.V[idx], self.Kraw[idx], self.t[idx] = Kst, v, k, t
            self._capture_bank(g0, k, v)
            return
        g0 = self.global_end
        new = {"K": Kst, "V": v.copy(), "Kraw": k.copy(), "t": t, "g": g0 + np.arange(N, dtype=np.int64),
               "tok": tok}
        self._cat([self._entries(0, self.n), new])
        self.n_sink = min(self.S_tok, self.n_sink + N)
        if self.n > self.C_tok:
            n_evict = self.n - self.C_tok
            if self.memory is not None:
                self._fold(self.S_tok, n_evict)
            # physical left shift of everything after the sink: window = window[n_evict:]
            sink = self._entries(0, self.S_tok)
            window = self._entries(self.S_tok + n_evict, self.n)
            self._cat([sink, window])
        self.newest = (g0, N, frames)
        self.global_end += N
        self._capture_bank(g0, k, v)

    def _fold(self, lo, n):
        """MemRoPE: fold the evicted entries [lo, lo + n) -- whole frames, oldest first -- into the long and
        short memories, M = alpha * M + (1 - alpha) * E per grid position, in fp32 with every product and the
        sum rounded separately; the first evicted frame initialises both."""
        if n % self.S or np.any(self.tok[lo:lo + n] != np.arange(n) % self.S):
            raise OracleError("memory folds whole frames")
        for f in range(n // self.S):
            ek = self.K[lo + f * self.S: lo + (f + 1) * self.S]
            ev = self.V[lo + f * self.S: lo + (f + 1) * self.S]
            for m, alpha in enumerate(self.memory):
                if self.mem_frames == 0:
                    self.mem_k[m] = ek
                    self.mem_v[m] = ev
                else:
                    a = np.float32(alpha)
                    b = np.float32(1.0) - a
                    self.mem_k[m] = (a * self.mem_k[m]) + (b * ek)
                    self.mem_v[m] = (a * self.mem_v[m]) + (b * ev)
            self.mem_frames += 1

    def memory_entries(self):
        """The memory tokens as attention sees them (none before the first fold): keys = the state rounded to
        the cache dtype, i.e. a stored key with its time band raw, placed (time band rotated) just before the
        oldest window entry -- the long memory at t_w - 2, the short at t_w - 1; values = the state rounded."""
        if self.memory is None or self.mem_frames == 0:
            return None
        t_w = int(self.t[self.n_sink])
        keys, vals, times = [], [], []
        zero = np.zeros(self.S, np.int64)
        for m, dt in ((0, 2), (1, 1)):
            stored = self._store(self.mem_k[m])
            tm = np.full(self.S, t_w - dt, np.int64)
            keys.append(self._store(rotate_f32(stored, tm, zero, zero, bands=(True, False, False))))
            vals.append(self._store(self.mem_v[m]))
            times.append(tm)
        return np.concatenate(keys), np.concatenate(vals), np.concatenate(times)

    def _capture_bank(self, g0, k, v):
        if self.bank_tok == 0 or g0 >= self.bank_tok:
            return
        m = min(self.bank_tok - g0, k.shape[0])
        self.bank_K[g0:g0 + m] = k[:m]
        self.bank_V[g0:g0 + m] = v[:m]

    # ------------------------------------------------------------------ retime
    def retime(self, delta, clamp0, lo=0, hi=None):
        """Shift times of logical entries [lo, hi) by delta (clamped at 0 if clamp0), re-rotating in place.

        Storage model: the time band of the *stored* key is rotated by the
        actual change t' - t and rounded again; the other bands are untouched.
        """
        hi = self.n if hi is None else hi
        if not (0 <= lo <= hi <= self.n):
            raise OracleError("retime range")
        if hi == lo:
            return
        t_old = self.t[lo:hi]
        t_new = np.maximum(0, t_old + delta) if clamp0 else t_old + delta
        if self.raw_keys:                       # index only: keys are placed at attention time
            self.t[lo:hi] = t_new
            return
        dlt = t_new - t_old
        blk = self.K[lo:hi]
        rot = rotate_f32(blk, dlt, np.zeros_like(dlt), np.zeros_like(dlt), bands=(True, False, False))
        (ts, tw) = band_split(self.D)[0]
        out = blk.copy()
        out[:, :, ts:ts + tw] = self._store(rot[:, :, ts:ts + tw])
        self.K[lo:hi] = out
        self.t[lo:hi] = t_new

    # ------------------------------------------------------------------ compact
    def compact(self, keep_idx):
        """Keep exactly the logical entries keep_idx (sorted, unique, containing the whole sink)."""
        if self.memory is not None:
            raise OracleError("compaction is not defined with memory tokens")
        keep = np.asarray(keep_idx, dtype=np.int64)
        if keep.ndim != 1 or keep.shape[0] == 0:
            raise OracleError("keep_idx empty")
        if np.any(np.diff(keep) <= 0):
            raise OracleError("keep_idx not sorted unique")
        if keep[0] < 0 or keep[-1] >= self.n:
            raise OracleError("keep_idx out of range")
        if keep.shape[0] < self.n_sink or np.any(keep[:self.n_sink] != np.arange(self.n_sink)):
            raise OracleError("keep_idx drops a sink entry")
        if self.newest is not None:
            g0, N, _ = self.newest
            kept_g = self.g[keep]
            if np.count_nonzero((kept_g >= g0) & (kept_g < g0 + N)) != N:
                self.newest = None
        self._take(keep)

    # ------------------------------------------------------------------ sink push
    def sink_push(self, bank_frame, frames, t0):
        """Rolling-Sink sink FIFO step: drop the oldest `frames` sink frames, append bank frames
        [bank_frame, bank_frame+frames) freshly rotated at times t0 .. t0+frames-1."""
        N = frames * self.S
        if self.memory is not None:
            raise OracleError("sink push is not defined with memory tokens")
        if self.bank_tok == 0 or self.global_end < self.bank_tok:
            raise OracleError("bank incomplete")
        if self.n_sink != self.S_tok or N > self.S_tok:
            raise OracleError("sink not full / block too large")
        b0 = bank_frame * self.S
        if b0 < 0 or b0 + N > self.bank_tok:
            raise OracleError("bank range")
        raw = self.bank_K[b0:b0 + N]
        t, _, _ = token_positions(N, self.S, self.grid_w, t0)
        tok = (b0 + np.arange(N, dtype=np.int64)) % self.S
        new = {"K": self._stored_key(raw, t, tok), "V": self.bank_V[b0:b0 + N].copy(), "Kraw": raw.copy(),
               "t": t, "g": b0 + np.arange(N, dtype=np.int64), "tok": tok}
        self._cat([self._entries(N, self.S_tok), new, self._entries(self.S_tok, self.n)])

    # ------------------------------------------------------------------ queries
    def rotate_queries(self, q, frames, t0):
        N = frames * self.S
        q = np.asarray(q, np.float32)
        if q.shape != (N, self.H, self.D):
            raise OracleError("q shape")
        t, _, _ = token_positions(N, self.S, self.grid_w, t0)
        tok = np.arange(N, dtype=np.int64) % self.S
        return self._rotate(q, t, tok)

    def newest_time(self):
        g0 = self.newest[0]
        return int(self.t[np.nonzero(self.g == g0)[0][0]])

    def attend(self, q, frames, t0=None, rows=None, f64=False, max_keys=None):
        """softmax(q_hat K^T / sqrt(D)) V over every valid entry, no mask; q rotated at t0.

        max_keys (LingBot-World 2.0 article, max_attention_size: queries read only the last
        max_attention_size positions of the cache buffer, whose order is sink first, then the window
        oldest to newest): attend to the last max_keys entries in logical order only."""
        t0 = self.newest_time() if t0 is None else t0
        qh = self.rotate_queries(q, frames, t0)
        if rows is not None:
            qh = qh[np.asarray(rows)]
        K, V = self.attention_keys(), self.V
        if max_keys is not None and max_keys < self.n:
            if max_keys < 1 or self.memory is not None:
                raise OracleError("max_keys")
            K, V = K[self.n - max_keys:], V[self.n - max_keys:]
        mem = self.memory_entries()
        if mem is not None:
            K = np.concatenate([K, mem[0]])
            V = np.concatenate([V, mem[1]])
        if f64:
            return attention_f64(qh, K, V)
        return attention_f32(qh, K, V)

    def attend_block_causal(self, q, frames, t0, block_frames, rows=None, f64=False):
        """Block-causal attention of a whole clip, for a cache that holds the clip from its first frame.

        The rCM length-extrapolation article points to a block-level attention mask for the clip-level
        (teacher-forced) training path, and the Causal-Forcing article (section 4, block-wise denoising)
        splits a 21-frame clip into blocks of num_frame_per_block frames.  Reading taken: query frame f
        (rotated at t0 + f) belongs to block f // block_frames and attends to the cached entries of
        blocks 0..that block, i.e. to the first min(n, (block + 1) * block_frames * S) entries in logical
        order; there is no mask inside a block.
        """
        if self.memory is not None:
            raise OracleError("block-causal attention is not defined with memory tokens")
        qh = self.rotate_queries(q, frames, t0)
        N = frames * self.S
        rows = np.arange(N) if rows is None else np.asarray(rows)
        blk = rows // (block_frames * self.S)
        fn = attention_f64 if f64 else attention_f32
        K = self.attention_keys()
        out = np.empty((len(rows), self.H, self.D), np.float64 if f64 else np.float32)
        for b in np.unique(blk):
            sel = np.nonzero(blk == b)[0]
            n_vis = min(self.n, int(b + 1) * block_frames * self.S)
            out[sel] = fn(qh[rows[sel]], K[:n_vis], self.V[:n_vis])
        return out

    def relax_scores(self, tail_frames, weight=0.5):
        """Relax Forcing scores of the History candidates: the whole frames between the sink and the
        last tail_frames frames (which form the Tail).  The cache must hold whole frames."""
        S = self.S
        if self.n % S or self.n_sink % S:
            raise OracleError("relax scores need whole frames")
        first = self.n_sink // S
        n_cand = self.n // S - tail_frames - first
        if tail_frames < 1 or n_cand < 1:
            raise OracleError("relax scores need a tail and at least one candidate")
        return relax_frame_scores(self.attention_keys(), S, first, n_cand, tail_frames, weight)

    def score(self, q_win, frames, t_frames, f64=False):
        """Per-entry attention mass of the query window, summed over heads and query rows."""
        N = frames * self.S
        t = np.repeat(np.asarray(t_frames, np.int64), self.S)
        tok = np.arange(N, dtype=np.int64) % self.S
        qh = self._rotate(np.asarray(q_win, np.float32), t, tok)
        return attention_mass_scores(qh, self.attention_keys(), np.float64 if f64 else np.float32)

    def row_normalisers(self, q, frames, t0):
        """Each row's log2 softmax normaliser [H, N] for queries of frames t0 .. t0+frames-1 over the entries
        attention reads (score.row_normalisers on the rotated, storage-rounded queries)."""
        return row_normalisers(self.rotate_queries(q, frames, t0), self.attention_keys())

    def state(self):
        return {"K": self.K, "V": self.V, "t": self.t, "g": self.g, "n_sink": self.n_sink,
                "global_end": self.global_end}
