"""Pins for the oracle's bf16 rounding and 3D RoPE (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import (band_split, bf16_ulp, cos_sin_table, inv_freq, rotate_f32, rotate_f64, round_to_bf16,
                    token_positions)


# ---------------------------------------------------------------- bf16 RNE
def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 1.0, 7.0, 1e5)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_to_bf16(x).view(np.uint32), ref.view(np.uint32))


def test_bf16_ties_to_even_hand_values():
    one = np.float32(1.0)
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20, 3.0], np.float32)
    exp = np.array([1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7, 3.0], np.float32)
    assert np.array_equal(round_to_bf16(vals), exp)
    assert round_to_bf16(np.array([one]))[0] == one


def test_bf16_ulp():
    assert bf16_ulp(np.array([1.0]))[0] == 2 ** -7
    assert bf16_ulp(np.array([3.0]))[0] == 2 ** -6
    assert bf16_ulp(np.array([-5.0]))[0] == 2 ** -5


# ---------------------------------------------------------------- RoPE bands / frequencies
def test_band_split_44_42_42():
    assert band_split(128) == [(0, 44), (44, 42), (86, 42)]
    assert band_split(64) == [(0, 24), (24, 20), (44, 20)]
    for D in (64, 128):
        (a, wa), (b, wb), (c, wc) = band_split(D)
        assert wa + wb + wc == D and wa % 2 == wb % 2 == wc % 2 == 0


def test_inv_freq_endpoints_and_monotone():
    th = inv_freq(44)
    assert th[0] == 1.0
    assert abs(th[-1] - 10000.0 ** (-42 / 44)) < 1e-18
    assert all(a > b for a, b in zip(th, th[1:]))
    assert len(inv_freq(42)) == 21


def test_table_angle_addition():
    # cos/sin tables satisfy the angle-addition identities to fp32 accuracy
    p, q = 37, 154
    c1, s1 = cos_sin_table([p], 44)
    c2, s2 = cos_sin_table([q], 44)
    c3, s3 = cos_sin_table([p + q], 44)
    c_add = c1.astype(np.float64) * c2 - s1.astype(np.float64) * s2
    s_add = s1.astype(np.float64) * c2 + c1.astype(np.float64) * s2
    assert np.max(np.abs(c_add - c3)) < 4e-7 and np.max(np.abs(s_add - s3)) < 4e-7
    c0, s0 = cos_sin_table([0], 42)
    assert np.all(c0 == 1.0) and np.all(s0 == 0.0)
    cn, sn = cos_sin_table([-5, 5], 42)
    assert np.array_equal(cn[0], cn[1]) and np.array_equal(sn[0], -sn[1])


def test_token_positions_row_major_grid():
    t, h, w = token_positions(4680, 1560, 52, 9)
    assert (t[0], h[0], w[0]) == (9, 0, 0)
    assert (t[1559], h[1559], w[1559]) == (9, 29, 51)
    assert (t[1560], h[1560], w[1560]) == (10, 0, 0)
    assert (t[4679], h[4679], w[4679]) == (11, 29, 51)
    assert h.max() == 29 and w.max() == 51


# ---------------------------------------------------------------- rotation
def _rand(n, H, D, seed=0):
    return np.random.default_rng(seed).standard_normal((n, H, D)).astype(np.float32)


def test_rotation_identity_at_origin():
    x = _rand(16, 2, 128)
    z = np.zeros(16, np.int64)
    assert np.array_equal(rotate_f32(x, z, z, z).view(np.uint32), x.view(np.uint32))


@pytest.mark.parametrize("D", [64, 128])
def test_rotation_matches_complex_multiplication(D):
    # the real-arithmetic rotation equals multiplying each (even, odd) pair as a complex number
    # by e^{i pos theta}: a swapped sign, a wrong pair or band would fail this
    x = _rand(40, 3, D, 1)
    rng = np.random.default_rng(2)
    t, h, w = rng.integers(-50, 300, 40), rng.integers(0, 30, 40), rng.integers(0, 52, 40)
    r32 = rotate_f32(x, t, h, w).astype(np.float64)
    r64 = rotate_f64(x, t, h, w)
    assert np.max(np.abs(r32 - r64)) < 2e-6 * max(1.0, np.abs(r64).max())


def test_rotation_bands_act_on_their_own_dims():
    x = _rand(8, 1, 128, 3)
    t = np.full(8, 11)
    z = np.zeros(8, np.int64)
    rt = rotate_f32(x, t, z, z)
    assert np.array_equal(rt[:, :, 44:], x[:, :, 44:])
    assert not np.array_equal(rt[:, :, :44], x[:, :, :44])
    rh = rotate_f32(x, z, np.full(8, 7), z)
    assert np.array_equal(rh[:, :, :44], x[:, :, :44]) and np.array_equal(rh[:, :, 86:], x[:, :, 86:])


def test_rotation_preserves_pair_norms():
    x = _rand(30, 2, 128, 4).astype(np.float64)
    rng = np.random.default_rng(5)
    t, h, w = rng.integers(0, 1000, 30), rng.integers(0, 30, 30), rng.integers(0, 52, 30)
    r = rotate_f64(x, t, h, w)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12


def test_relative_position_invariance_fp64():
    # R(tq + d) q . R(tk + d) k == R(tq) q . R(tk) k
    q = _rand(1, 4, 128, 6)
    k = _rand(1, 4, 128, 7)
    h, w = np.array([3]), np.array([17])
    for tq, tk, d in [(20, 5, 7), (3, 3, 100), (0, 18, -40)]:
        a = (rotate_f64(q, [tq + d], h, w) * rotate_f64(k, [tk + d], h, w)).sum(-1)
        b = (rotate_f64(q, [tq], h, w) * rotate_f64(k, [tk], h, w)).sum(-1)
        assert np.max(np.abs(a - b)) < 1e-12


def test_composed_rotation_equals_single():
    # rotating by t1 then by t2 (fp64) equals rotating by t1 + t2: the time delta re-rotation is sound
    x = _rand(5, 2, 128, 8)
    z = np.zeros(5, np.int64)
    a = rotate_f64(rotate_f64(x, np.full(5, 9), z, z), np.full(5, -4), z, z)
    b = rotate_f64(x, np.full(5, 5), z, z)
    assert np.max(np.abs(a - b)) < 1e-12
