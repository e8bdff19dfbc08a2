"""rolling_kv_cache_amd -- bounded, ring-indexed KV cache for chunk-wise video attention on MI355X.

Thin ctypes binding over ``libkvc.so`` (C ABI in ``include/kvc.h``).  PyTorch
only provides device memory and the stream; every step of the cache runs in
the library's HIP kernels.  Importing this package fails loudly when the
library has not been built (``python rolling_kv_cache_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK, KVC_EINVAL, KVC_ENOMEM, KVC_ESTATE, KVC_EDEVICE, KVC_EUNSUPPORTED = range(6)
KVC_BF16, KVC_F32 = 0, 1
KVC_T_NEWEST = -(2 ** 31)
KVC_APPEND_REPLACE_NEWEST = 1
KVC_CREATE_COMPACT = 1
KVC_CREATE_RAW_KEYS = 2
KVC_CREATE_MEMORY = 4
KVC_CREATE_SPLIT_ATTEND = 8
KVC_PATH_RUNNING_MAX = 1
KVC_PATH_GENERAL = 2
KVC_PATH_NO_SPLIT = 4
KVC_MAX_POS = 16383
KVC_MAX_Q_FRAMES = 32

# Every symbol include/kvc.h declares.
EXPORTED = ("kvc_workspace_bytes", "kvc_create", "kvc_destroy", "kvc_set_stream", "kvc_set_paths", "kvc_append",
            "kvc_attend", "kvc_attend_stats",
            "kvc_attend_blockcausal", "kvc_retime", "kvc_score_scratch_bytes", "kvc_score", "kvc_score_with_stats",
            "kvc_relax_scratch_bytes",
            "kvc_relax_scores", "kvc_relax_scores_noalloc", "kvc_set_attention_limit", "kvc_set_memory_rates", "kvc_export_memory",
            "kvc_compact", "kvc_sink_push", "kvc_group_workspace_bytes", "kvc_create_group", "kvc_retime_layers",
            "kvc_compact_layers", "kvc_sink_push_layers",
            "kvc_info",
            "kvc_slot_times", "kvc_export", "kvc_export_tables", "kvc_last_error")


class KVCError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"kvc error {code}: {msg}")
        self.code = code


class _Info(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int32), ("n_valid", ctypes.c_int32), ("sink_tokens", ctypes.c_int32),
                ("window_tokens", ctypes.c_int32), ("sink_filled", ctypes.c_int32),
                ("window_filled", ctypes.c_int32), ("sink_head", ctypes.c_int32), ("window_head", ctypes.c_int32),
                ("global_end", ctypes.c_int64), ("newest_valid", ctypes.c_int32),
                ("newest_frames", ctypes.c_int32), ("newest_t", ctypes.c_int32), ("bank_tokens", ctypes.c_int32),
                ("newest_g", ctypes.c_int64), ("bank_complete", ctypes.c_int32), ("window_buffer", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python rolling_kv_cache_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, u32, sz, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_void_p
    p32, p64, pf = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_float)
    sig = {
        "kvc_workspace_bytes": (sz, [i32, i32, i32, i32, i32, ctypes.c_int, i32, u32]),
        "kvc_create": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, ctypes.c_int, i32, u32, vp, sz, vp,
                                      ctypes.POINTER(vp)]),
        "kvc_destroy": (ctypes.c_int, [vp]),
        "kvc_group_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, ctypes.c_int, i32, u32]),
        "kvc_create_group": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, i32, ctypes.c_int, i32, u32, vp, sz, vp,
                                            ctypes.POINTER(vp)]),
        "kvc_retime_layers": (ctypes.c_int, [ctypes.POINTER(vp), i32, i32, i32, i32, i32]),
        "kvc_compact_layers": (ctypes.c_int, [ctypes.POINTER(vp), i32, p32, i32]),
        "kvc_sink_push_layers": (ctypes.c_int, [ctypes.POINTER(vp), i32, i32, i32, i32]),
        "kvc_set_stream": (ctypes.c_int, [vp, vp]),
        "kvc_set_paths": (ctypes.c_int, [vp, u32]),
        "kvc_append": (ctypes.c_int, [vp, vp, vp, i32, i32, u32]),
        "kvc_attend": (ctypes.c_int, [vp, vp, i32, i32, vp]),
        "kvc_attend_stats": (ctypes.c_int, [vp, vp, i32, i32, vp, vp]),
        "kvc_attend_blockcausal": (ctypes.c_int, [vp, vp, i32, i32, i32, vp]),
        "kvc_retime": (ctypes.c_int, [vp, i32, i32, i32, i32]),
        "kvc_score_scratch_bytes": (sz, [vp, i32]),
        "kvc_score": (ctypes.c_int, [vp, vp, i32, p32, vp, vp, sz]),
        "kvc_score_with_stats": (ctypes.c_int, [vp, vp, i32, p32, vp, vp, vp, sz]),
        "kvc_relax_scratch_bytes": (sz, [vp]),
        "kvc_relax_scores": (ctypes.c_int, [vp, i32, ctypes.c_float, vp, vp, sz]),
        "kvc_relax_scores_noalloc": (ctypes.c_int, [vp, i32, ctypes.c_float, vp]),
        "kvc_set_attention_limit": (ctypes.c_int, [vp, i32]),
        "kvc_set_memory_rates": (ctypes.c_int, [vp, ctypes.c_float, ctypes.c_float]),
        "kvc_export_memory": (ctypes.c_int, [vp, vp, vp, ctypes.POINTER(ctypes.c_int32)]),
        "kvc_compact": (ctypes.c_int, [vp, p32, i32]),
        "kvc_sink_push": (ctypes.c_int, [vp, i32, i32, i32]),
        "kvc_info": (ctypes.c_int, [vp, ctypes.POINTER(_Info)]),
        "kvc_slot_times": (ctypes.c_int, [vp, p32, p64]),
        "kvc_export": (ctypes.c_int, [vp, vp, vp, vp, vp]),
        "kvc_export_tables": (ctypes.c_int, [vp, i32, i32, i32, pf]),
        "kvc_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def _check(code: int):
    if code != KVC_OK:
        raise KVCError(code, lib.kvc_last_error().decode())


def _dt(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return KVC_BF16
    if dtype == torch.float32:
        return KVC_F32
    raise ValueError(f"unsupported cache dtype {dtype}")


def _create_flags(compact=False, raw_keys=False, memory=False, split_attend=False) -> int:
    return ((KVC_CREATE_COMPACT if compact else 0) | (KVC_CREATE_RAW_KEYS if raw_keys else 0)
            | (KVC_CREATE_MEMORY if memory else 0) | (KVC_CREATE_SPLIT_ATTEND if split_attend else 0))


def workspace_bytes(sink_frames, window_frames, frame_seqlen, heads, head_dim, dtype=torch.bfloat16,
                    bank_frames=0, compact=False, raw_keys=False, memory=False, split_attend=False) -> int:
    return int(lib.kvc_workspace_bytes(sink_frames, window_frames, frame_seqlen, heads, head_dim, _dt(dtype),
                                       bank_frames, _create_flags(compact, raw_keys, memory, split_attend)))


class KVCache:
    """One layer's cache.  Methods mirror the C calls: append, attend, retime, score, compact, sink_push."""

    def __init__(self, sink_frames, window_frames, frame_seqlen, heads, head_dim, grid_w,
                 dtype=torch.bfloat16, bank_frames=0, compact=False, device="cuda", stream=None, raw_keys=False,
                 memory=None, split_attend=False, _handle=None, _workspace=None):
        """memory: (alpha_long, alpha_short) for MemRoPE memory tokens on a raw-key cache, or None."""
        self.S, self.H, self.D = frame_seqlen, heads, head_dim
        self.dtype = dtype
        self.device = torch.device(device)
        if _handle is not None:                 # a member of a layer group (create_group)
            self._ws_raw = _workspace
            self._stream = stream
            self._h = _handle
            if memory is not None:
                _check(lib.kvc_set_memory_rates(self._h, float(memory[0]), float(memory[1])))
            self._score_scratch = None
            self._relax_scratch = None
            return
        nbytes = workspace_bytes(sink_frames, window_frames, frame_seqlen, heads, head_dim, dtype, bank_frames,
                                 compact, raw_keys, memory is not None, split_attend)
        if nbytes == 0:
            raise KVCError(KVC_EINVAL, "unsupported geometry")
        self._ws_raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self._ws_raw.data_ptr()) % 256
        self.workspace = self._ws_raw[off:off + nbytes]
        self._stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        _check(lib.kvc_create(sink_frames, window_frames, frame_seqlen, heads, head_dim, grid_w, _dt(dtype),
                              bank_frames, _create_flags(compact, raw_keys, memory is not None, split_attend),
                              ctypes.c_void_p(self.workspace.data_ptr()), nbytes,
                              ctypes.c_void_p(self._stream.cuda_stream), ctypes.byref(h)))
        self._h = h
        if memory is not None:
            _check(lib.kvc_set_memory_rates(h, float(memory[0]), float(memory[1])))
        self._score_scratch = None
        self._relax_scratch = None

    def close(self):
        if getattr(self, "_h", None):
            lib.kvc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -------------------------------------------------------------- marshalling
    def _tensor(self, x: torch.Tensor, frames: int, name: str):
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor")
        if x.dtype != self.dtype:
            raise ValueError(f"{name} dtype {x.dtype} != cache dtype {self.dtype}")
        if tuple(x.shape) != (frames * self.S, self.H, self.D) or not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous [{frames * self.S}, {self.H}, {self.D}]")
        return ctypes.c_void_p(x.data_ptr())

    def _frames_of(self, x: torch.Tensor) -> int:
        if x.dim() != 3 or x.shape[0] % self.S != 0:
            raise ValueError("token count must be a multiple of frame_seqlen")
        return x.shape[0] // self.S

    def set_stream(self, stream):
        _check(lib.kvc_set_stream(self._h, ctypes.c_void_p(stream.cuda_stream)))
        self._stream = stream

    def set_paths(self, running_max: bool = False, general: bool = False, no_split: bool = False):
        """Kernel paths of later calls (all False: the default kernels); for comparisons and tests."""
        _check(lib.kvc_set_paths(self._h, (KVC_PATH_RUNNING_MAX if running_max else 0)
                                 | (KVC_PATH_GENERAL if general else 0) | (KVC_PATH_NO_SPLIT if no_split else 0)))

    # -------------------------------------------------------------- verbs
    def append(self, k, v, t_index: int, replace_newest: bool = False):
        F = self._frames_of(k)
        _check(lib.kvc_append(self._h, self._tensor(k, F, "k"), self._tensor(v, F, "v"), F, int(t_index),
                              KVC_APPEND_REPLACE_NEWEST if replace_newest else 0))

    def attend(self, q, t_index=None, out=None, row_stats=None):
        """row_stats: a contiguous float32 CUDA tensor of at least heads x query rows elements; the call then
        also writes each row's log2 softmax normaliser there (kvc_attend_stats), for score(..., row_stats)."""
        F = self._frames_of(q)
        if out is None:
            out = torch.empty_like(q)
        t = KVC_T_NEWEST if t_index is None else int(t_index)
        if row_stats is None:
            _check(lib.kvc_attend(self._h, self._tensor(q, F, "q"), F, t, self._tensor(out, F, "out")))
        else:
            self._check_f32(row_stats, self.H * F * self.S, "row_stats")
            _check(lib.kvc_attend_stats(self._h, self._tensor(q, F, "q"), F, t, self._tensor(out, F, "out"),
                                        ctypes.c_void_p(row_stats.data_ptr())))
        return out

    @staticmethod
    def _check_f32(x, n, name):
        if (not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.float32
                or not x.is_contiguous() or x.numel() < n):
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor of at least {n} elements")

    def attend_block_causal(self, q, t_index, block_frames: int, out=None):
        """Block-causal attention of a whole clip held by this cache from its first frame."""
        F = self._frames_of(q)
        if out is None:
            out = torch.empty_like(q)
        _check(lib.kvc_attend_blockcausal(self._h, self._tensor(q, F, "q"), F, int(t_index), int(block_frames),
                                          self._tensor(out, F, "out")))
        return out

    def retime(self, delta: int, clamp0: bool = False, lo: int = 0, hi=None):
        hi = self.info()["n_valid"] if hi is None else hi
        _check(lib.kvc_retime(self._h, int(delta), 1 if clamp0 else 0, int(lo), int(hi)))

    def score(self, q_win, q_t, out=None, row_stats=None):
        """row_stats: the tensor of the latest attend(..., row_stats=...) of these queries at these times over
        the unchanged cache; only the columns pass then runs (kvc_score_with_stats)."""
        F = self._frames_of(q_win)
        q_t = np.ascontiguousarray(np.asarray(q_t, dtype=np.int32))
        if q_t.shape != (F,):
            raise ValueError("q_t must hold one time index per query frame")
        need = int(lib.kvc_score_scratch_bytes(self._h, F))
        if need == 0:
            raise KVCError(KVC_EINVAL, "score: q_frames out of range")
        if self._score_scratch is None or self._score_scratch.numel() < need + 256:
            self._score_scratch = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
        off = (-self._score_scratch.data_ptr()) % 256
        n = self.info()["n_valid"]
        if out is None:
            out = torch.empty(n, dtype=torch.float32, device=self.device)
        elif (out.device.type != "cuda" or out.dtype != torch.float32 or not out.is_contiguous()
              or out.numel() < n):
            raise ValueError("out must be a contiguous float32 CUDA tensor of at least n_valid elements")
        qt = q_t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        scratch = ctypes.c_void_p(self._score_scratch.data_ptr() + off)
        if row_stats is None:
            _check(lib.kvc_score(self._h, self._tensor(q_win, F, "q_win"), F, qt, ctypes.c_void_p(out.data_ptr()),
                                 scratch, need))
        else:
            self._check_f32(row_stats, self.H * F * self.S, "row_stats")
            _check(lib.kvc_score_with_stats(self._h, self._tensor(q_win, F, "q_win"), F, qt,
                                            ctypes.c_void_p(row_stats.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                            scratch, need))
        return out

    def relax_scores(self, tail_frames: int, weight: float = 0.5, out=None):
        """Relax Forcing scores of the whole frames between the sink and the last tail_frames frames."""
        info = self.info()
        n_cand = max(1, info["n_valid"] // self.S - info["sink_filled"] // self.S - int(tail_frames))
        need = int(lib.kvc_relax_scratch_bytes(self._h))
        if self._relax_scratch is None or self._relax_scratch.numel() < need + 256:
            self._relax_scratch = torch.empty(need + 256, dtype=torch.uint8, device=self.device)
        off = (-self._relax_scratch.data_ptr()) % 256
        if out is None:
            out = torch.empty(n_cand, dtype=torch.float32, device=self.device)
        elif (out.device.type != "cuda" or out.dtype != torch.float32 or not out.is_contiguous()
              or out.numel() < n_cand):
            raise ValueError("out must be a contiguous float32 CUDA tensor of at least n_cand elements")
        _check(lib.kvc_relax_scores(self._h, int(tail_frames), float(weight), ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(self._relax_scratch.data_ptr() + off), need))
        return out

    def relax_scores_noalloc(self, tail_frames: int, weight: float = 0.5, out=None):
        """relax_scores on the scratch the library holds per GPU (kvc_relax_scores_noalloc): the call itself
        allocates nothing; `out` (float32, at least n_cand elements) is allocated here only when not given."""
        info = self.info()
        n_cand = max(1, info["n_valid"] // self.S - info["sink_filled"] // self.S - int(tail_frames))
        if out is None:
            out = torch.empty(n_cand, dtype=torch.float32, device=self.device)
        elif (out.device.type != "cuda" or out.dtype != torch.float32 or not out.is_contiguous()
              or out.numel() < n_cand):
            raise ValueError("out must be a contiguous float32 CUDA tensor of at least n_cand elements")
        _check(lib.kvc_relax_scores_noalloc(self._h, int(tail_frames), float(weight), ctypes.c_void_p(out.data_ptr())))
        return out

    def set_attention_limit(self, max_keys: int):
        """Attend only to the newest max_keys entries (0: no limit)."""
        _check(lib.kvc_set_attention_limit(self._h, int(max_keys)))

    def set_memory_rates(self, alpha_long: float, alpha_short: float):
        _check(lib.kvc_set_memory_rates(self._h, float(alpha_long), float(alpha_short)))

    def export_memory(self):
        """(k, v, n_folded): the long then the short memory tokens [2S, H, D] (keys in stored form)."""
        k = torch.empty((2 * self.S, self.H, self.D), dtype=self.dtype, device=self.device)
        v = torch.empty_like(k)
        n = ctypes.c_int32()
        _check(lib.kvc_export_memory(self._h, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                     ctypes.byref(n)))
        return k, v, int(n.value)

    def compact(self, keep_idx):
        keep = np.ascontiguousarray(np.asarray(keep_idx, dtype=np.int32))
        _check(lib.kvc_compact(self._h, keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(keep.shape[0])))

    def sink_push(self, bank_frame: int, n_frames: int, t_index: int):
        _check(lib.kvc_sink_push(self._h, int(bank_frame), int(n_frames), int(t_index)))

    # -------------------------------------------------------------- inspection
    def info(self) -> dict:
        inf = _Info()
        _check(lib.kvc_info(self._h, ctypes.byref(inf)))
        return {f: getattr(inf, f) for f, _ in _Info._fields_}

    def slot_times(self):
        n = self.info()["n_valid"]
        t = np.empty(n, np.int32)
        g = np.empty(n, np.int64)
        _check(lib.kvc_slot_times(self._h, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  g.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return t, g

    def export(self):
        n = self.info()["n_valid"]
        k = torch.empty((max(n, 1), self.H, self.D), dtype=self.dtype, device=self.device)
        v = torch.empty_like(k)
        t = torch.empty(max(n, 1), dtype=torch.int32, device=self.device)
        g = torch.empty(max(n, 1), dtype=torch.int64, device=self.device)
        _check(lib.kvc_export(self._h, ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                              ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(g.data_ptr())))
        return {"K": k[:n], "V": v[:n], "t": t[:n], "g": g[:n]}

    def export_tables(self, band: int, pos_lo: int, n_pos: int):
        width = {0: self.D - 4 * (self.D // 6), 1: 2 * (self.D // 6), 2: 2 * (self.D // 6)}[band]
        out = np.empty((n_pos, width // 2, 2), np.float32)
        _check(lib.kvc_export_tables(self._h, band, pos_lo, n_pos, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
        return out


def create_group(n_layers, sink_frames, window_frames, frame_seqlen, heads, head_dim, grid_w,
                 dtype=torch.bfloat16, bank_frames=0, compact=False, device="cuda", stream=None, raw_keys=False,
                 memory=None):
    """n_layers caches over one workspace (kvc_create_group): per-layer append/attend as usual, and the
    layer-uniform operations batched with retime_layers / compact_layers / sink_push_layers."""
    device = torch.device(device)
    flags = _create_flags(compact, raw_keys, memory is not None)
    nbytes = int(lib.kvc_group_workspace_bytes(n_layers, sink_frames, window_frames, frame_seqlen, heads, head_dim,
                                               _dt(dtype), bank_frames, flags))
    if nbytes == 0:
        raise KVCError(KVC_EINVAL, "unsupported geometry")
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    stream = stream if stream is not None else torch.cuda.current_stream(device)
    hs = (ctypes.c_void_p * n_layers)()
    _check(lib.kvc_create_group(n_layers, sink_frames, window_frames, frame_seqlen, heads, head_dim, grid_w,
                                _dt(dtype), bank_frames, flags, ctypes.c_void_p(raw.data_ptr() + off), nbytes,
                                ctypes.c_void_p(stream.cuda_stream), hs))
    return [KVCache(sink_frames, window_frames, frame_seqlen, heads, head_dim, grid_w, dtype, bank_frames, compact,
                    device, stream, raw_keys, memory, _handle=ctypes.c_void_p(hs[i]), _workspace=raw)
            for i in range(n_layers)]


def _handles(caches):
    arr = (ctypes.c_void_p * len(caches))()
    for i, c in enumerate(caches):
        arr[i] = c._h.value if isinstance(c._h, ctypes.c_void_p) else c._h
    return arr


def retime_layers(caches, delta: int, clamp0: bool = False, lo: int = 0, hi=None):
    hi = caches[0].info()["n_valid"] if hi is None else hi
    _check(lib.kvc_retime_layers(_handles(caches), len(caches), int(delta), 1 if clamp0 else 0, int(lo), int(hi)))


def compact_layers(caches, keep_idx):
    keep = np.ascontiguousarray(np.asarray(keep_idx, dtype=np.int32))
    _check(lib.kvc_compact_layers(_handles(caches), len(caches), keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  int(keep.shape[0])))


def sink_push_layers(caches, bank_frame: int, n_frames: int, t_index: int):
    _check(lib.kvc_sink_push_layers(_handles(caches), len(caches), int(bank_frame), int(n_frames), int(t_index)))


__all__ = ["KVCache", "KVCError", "lib", "workspace_bytes", "EXPORTED", "LIB_PATH", "create_group", "retime_layers",
           "compact_layers", "sink_push_layers"]
