"""3D rotary position embedding (time / height / width) for video latent tokens.

What the pages fix: keys (and queries) are rotated at the *absolute* frame
number of their chunk (LingBot-World 2.0 sliding-window article, "two easily
missed details": RoPE takes the absolute frame from current_start_frame;
Causal-Forcing article, section 3: causal_rope_apply at start_frame), RoPE
rotates each dimension pair by a position-proportional angle with a
per-dimension frequency (Rolling Sink summary, "RoPE position encoding").

Readings taken where the pages are silent (parity unpinned as a convention):
  * head_dim D is split into a time band of D - 2*(2*floor(D/6)) dims and
    height/width bands of 2*floor(D/6) dims each: 44/42/42 for D=128,
    24/20/20 for D=64; bands are laid out t, h, w along the head dimension;
  * inside a band, dims (2p, 2p+1) form pair p with frequency
    theta_p = 10000 ** (-(2p) / band_width), computed in fp64;
  * token j of a chunk starting at frame t0 has t = t0 + j // S,
    h = (j % S) // grid_w, w = (j % S) % grid_w (row-major latent grid);
  * tables: c = float32(cos(float64(pos) * theta)), s = float32(sin(...)),
    with Python's math.cos / math.sin (the C library's);
  * rotation arithmetic, each product and sum rounded to fp32, no fused
    multiply-add:  x' = (x*c) - (y*s),  y' = (x*s) + (y*c).
"""
from __future__ import annotations

import math

import numpy as np


def band_split(D: int):
    """[(start, width)] for the time, height and width bands of a D-wide head."""
    b = 2 * (D // 6)
    dt = D - 2 * b
    return [(0, dt), (dt, b), (dt + b, b)]


def inv_freq(width: int):
    """fp64 frequencies theta_p = 10000^(-(2p)/width), p = 0 .. width/2 - 1."""
    return [10000.0 ** (-(2.0 * p) / width) for p in range(width // 2)]


def cos_sin_table(positions, width: int):
    """float32 cos/sin of float64(pos) * theta_p: arrays [len(positions), width/2]."""
    th = inv_freq(width)
    pos = list(int(p) for p in positions)
    c = np.empty((len(pos), len(th)), np.float32)
    s = np.empty((len(pos), len(th)), np.float32)
    for a, p in enumerate(pos):
        for j, tj in enumerate(th):
            ang = float(p) * tj
            c[a, j] = np.float32(math.cos(ang))
            s[a, j] = np.float32(math.sin(ang))
    return c, s


def token_positions(n_tokens: int, frame_seqlen: int, grid_w: int, t0: int, tok0: int = 0):
    """(t, h, w) integer positions of tokens tok0 .. tok0+n_tokens-1 of a chunk starting at frame t0."""
    j = np.arange(tok0, tok0 + n_tokens, dtype=np.int64)
    f = j // frame_seqlen
    i = j % frame_seqlen
    return t0 + f, i // grid_w, i % grid_w


def _rotate_band_f32(x: np.ndarray, start: int, width: int, pos: np.ndarray) -> None:
    """In place: rotate dims [start, start+width) of x[N, H, D] (float32) by pos[N]."""
    uniq, inv = np.unique(np.asarray(pos, dtype=np.int64), return_inverse=True)
    c_tab, s_tab = cos_sin_table(uniq, width)
    c = c_tab[inv][:, None, :]          # [N, 1, P]
    s = s_tab[inv][:, None, :]
    xe = x[:, :, start:start + width:2].copy()
    xo = x[:, :, start + 1:start + width:2].copy()
    # float32 numpy ufuncs round every product and every sum separately
    x[:, :, start:start + width:2] = (xe * c) - (xo * s)
    x[:, :, start + 1:start + width:2] = (xe * s) + (xo * c)


def rotate_f32(x: np.ndarray, t, h, w, bands=(True, True, True)) -> np.ndarray:
    """fp32 rotation of x[N, H, D] at per-token positions (t, h, w); returns a new array.

    ``bands`` selects which of the (time, height, width) bands are rotated.
    """
    x = np.array(x, dtype=np.float32, copy=True)
    D = x.shape[2]
    for (start, width), pos, on in zip(band_split(D), (t, h, w), bands):
        if on and width > 0:
            _rotate_band_f32(x, start, width, np.asarray(pos))
    return x


def rotate_f64(x: np.ndarray, t, h, w) -> np.ndarray:
    """fp64 reference: complex multiplication of each pair (x_2p + i x_2p+1) by e^{i pos theta_p}."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[2]
    out = np.empty_like(x)
    for (start, width), pos in zip(band_split(D), (t, h, w)):
        th = np.array(inv_freq(width), dtype=np.float64)
        ang = np.asarray(pos, dtype=np.float64)[:, None] * th[None, :]
        z = x[:, :, start:start + width:2] + 1j * x[:, :, start + 1:start + width:2]
        z = z * np.exp(1j * ang)[:, None, :]
        out[:, :, start:start + width:2] = z.real
        out[:, :, start + 1:start + width:2] = z.imag
    return out
