"""bfloat16 round-to-nearest-even, written from the IEEE-754 definition.

bfloat16 keeps the upper 16 bits of a binary32 value.  Rounding to nearest,
ties to even, adds 0x7FFF plus the lowest kept bit to the binary32 pattern and
truncates.  This is the storage rounding the cache applies after rotating a
key (the pages fix no precision; bf16 storage is the reading recorded for the
14B/1.3B-shaped workloads).  Pinned against torch's CPU cast and hand values in
tests/test_oracle_bf16.py.
"""
import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array whose values are the RNE bfloat16 roundings."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    r = np.where(is_nan, (u.astype(np.uint32) & 0x80000000) | 0x7FC00000, r).astype(np.uint32)
    return r.view(np.float32).reshape(x.shape)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits): 2**(floor(log2|x|) - 7)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    e = np.maximum(e, -126.0)
    return 2.0 ** (e - 7)
