"""CPU oracle for the bounded, ring-indexed video KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything here.
The product path (``rolling_kv_cache_amd``) never touches this package, and
this package imports nothing from it; the two share only the seeded input
generator in ``workloads``.

The oracle is deliberately plain and slow: numpy only (plus Python's ``math``
for the RoPE tables), explicit concatenation, a physical left-shift eviction,
fresh re-rotation, fp32 BLAS attention over the same bf16 inputs and fp64
references.  Sources it follows (cited by page and section throughout):

* LingBot-World 2.0 sliding-window article (icman.com.cn/news/50396):
  fixed ``kv_size``, the roll rule ``num_evicted = new + local_end - kv_size``
  with a left shift that starts after the sink, absolute-frame RoPE.
* Causal-Forcing article (lqnn.cn/news/227985), section 3 "KV Cache": only the
  current block's queries attend to cached history plus the new block.
* rCM length-extrapolation article (dpshk.com/news/6097349): Rolling Sink bank,
  Infinity-RoPE shift/clamp/flush/cut, Deep-Forcing scoring and compaction,
  in-place time re-rotation, Relax Forcing frame selection.
* Rolling Sink paper summary (paper.rainbus.top/paper/2602.07775), "method step
  details": Cat(x[0,S), x[i-(K-S), i)), sliding indices, Roll with
  forward/reverse alternation.
* Attention itself: softmax(QK^T / sqrt(d_k)) V (stated on the infinite-canvas
  article, lshu.cn/news/4311, and implied by all pages).

Parity status: every function here is pinned by tests under ``tests/`` (see
the ``test_oracle_*`` modules) except the exact RoPE *convention* (band order,
interleaved pairing, base), which the pages leave open: that convention is
"parity unpinned" -- any convention satisfies the invariants that are tested.
"""
from .bf16 import round_to_bf16, bf16_ulp
from .rope import band_split, inv_freq, cos_sin_table, token_positions, rotate_f32, rotate_f64
from .cache import OracleCache, OracleError
from .attention import attention_f32, attention_f64, attention_loops_f64
from .score import attention_mass_scores, row_normalisers
from .policies import (SlidingWindowRun, RollingSinkRun, InfinityRopeRun, DeepForcingRun,
                       RelaxForcingRun, DenoiseLoopRun, roll_index, make_run)
from .relax import relax_frame_scores, top_frames

__all__ = [
    "round_to_bf16", "bf16_ulp", "band_split", "inv_freq", "cos_sin_table", "token_positions",
    "rotate_f32", "rotate_f64", "OracleCache", "OracleError", "attention_f32", "attention_f64",
    "attention_loops_f64", "attention_mass_scores", "row_normalisers", "SlidingWindowRun", "RollingSinkRun",
    "InfinityRopeRun", "DeepForcingRun", "RelaxForcingRun", "DenoiseLoopRun", "roll_index", "make_run",
    "relax_frame_scores", "top_frames",
]
