"""Pins of the oracle's RoPE (oracle/rope.py) against closed forms and an independent route."""
import math

import numpy as np
import pytest

import brute
from oracle import rope
from synth.configs import TINY_FP32, WAN13B_1LAYER, default_rope_split


def cfg_axes(dt, dh, dw, theta=10000.0):
    return TINY_FP32.with_(head_dim=dt + dh + dw, rope_dim_t=dt, rope_dim_h=dh, rope_dim_w=dw,
                           rope_theta=theta)


def rot(cfg, x, t, h, w):
    return rope.rotate_pairs(np.asarray(x, np.float64), rope.angles(cfg, t, h, w))


def test_pair0_unit_frequency_hand_values():
    # omega_0 = theta^0 = 1 on every axis: p = 1 turns pair 0 by exactly one radian,
    # counter-clockwise: (1, 0) -> (cos 1, sin 1) and (0, 1) -> (-sin 1, cos 1).
    cfg = cfg_axes(24, 20, 20)
    x = np.zeros(64)
    x[0] = 1.0
    y = rot(cfg, x, 1.0, 0.0, 0.0)
    assert y[0] == pytest.approx(math.cos(1.0), abs=1e-15)
    assert y[1] == pytest.approx(math.sin(1.0), abs=1e-15)
    assert np.all(y[2:] == 0.0)
    x = np.zeros(64)
    x[1] = 1.0
    y = rot(cfg, x, 1.0, 0.0, 0.0)
    assert (y[0], y[1]) == pytest.approx((-math.sin(1.0), math.cos(1.0)), abs=1e-15)


def test_frequency_exponent_and_axis_order():
    # d_t = d_h = d_w = 4, theta = 1e4: the second pair of each axis has omega = 1e4^(-2/4)
    # = 0.01, so position 100 turns it by exactly one radian, and the first pair by 100 rad.
    cfg = cfg_axes(4, 4, 4)
    x = np.tile([1.0, 0.0], 6)
    for axis, pos in enumerate([(100.0, 0.0, 0.0), (0.0, 100.0, 0.0), (0.0, 0.0, 100.0)]):
        y = rot(cfg, x, *pos)
        for pair in range(6):
            expect = 0.0
            if pair == 2 * axis:
                expect = 100.0
            elif pair == 2 * axis + 1:
                expect = 1.0
            assert y[2 * pair] == pytest.approx(math.cos(expect), abs=1e-12), (axis, pair)
            assert y[2 * pair + 1] == pytest.approx(math.sin(expect), abs=1e-12), (axis, pair)


def test_matches_complex_multiplication_route():
    cfg = WAN13B_1LAYER
    g = np.random.default_rng(0)
    x = g.standard_normal((7, cfg.head_dim))
    t = g.integers(-50, 50, 7).astype(float)
    h = g.integers(0, cfg.grid_h, 7).astype(float)
    w = g.integers(0, cfg.grid_w, 7).astype(float)
    np.testing.assert_allclose(rot(cfg, x, t, h, w), brute.complex_rope(cfg, x, t, h, w), atol=1e-12)


def test_norm_identity_composition():
    cfg = WAN13B_1LAYER
    g = np.random.default_rng(1)
    x = g.standard_normal((5, cfg.head_dim))
    y = rot(cfg, x, 17.0, 3.0, 29.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    np.testing.assert_array_equal(rot(cfg, x, 0.0, 0.0, 0.0), x)
    a = rope.angles(cfg, 5.0, 2.0, 1.0)
    b = rope.angles(cfg, -3.0, 7.0, 4.0)
    np.testing.assert_allclose(rope.rotate_pairs(rope.rotate_pairs(x, a), b),
                               rope.rotate_pairs(x, a + b), atol=1e-12)


def test_relative_position_invariance():
    # <R(p + c) q, R(p' + c) k> = <R(p) q, R(p') k>: shifting every temporal position by one
    # constant leaves every score unchanged (what makes a RoPE rebase legal).
    cfg = WAN13B_1LAYER
    g = np.random.default_rng(2)
    q, k = g.standard_normal((2, 64, cfg.head_dim))
    h, w = 5.0, 9.0
    for c in (1.0, -32.0, 1000.0):
        s0 = np.einsum("nd,md->nm", rot(cfg, q, 40.0, h, w), rot(cfg, k, 33.0, h, w))
        s1 = np.einsum("nd,md->nm", rot(cfg, q, 40.0 + c, h, w), rot(cfg, k, 33.0 + c, h, w))
        np.testing.assert_allclose(s0, s1, atol=1e-10)
    # ... while a shift of only one side does change the scores
    s2 = np.einsum("nd,md->nm", rot(cfg, q, 41.0, h, w), rot(cfg, k, 33.0, h, w))
    assert np.max(np.abs(s2 - s0)) > 1e-3


def test_token_grid_row_major():
    hh, ww = rope.token_grid(30, 52)
    assert (hh[0], ww[0]) == (0, 0)
    assert (hh[51], ww[51]) == (0, 51)
    assert (hh[52], ww[52]) == (1, 0)
    assert (hh[1559], ww[1559]) == (29, 51)


def test_rope_frame_uses_grid_positions():
    cfg = TINY_FP32
    g = np.random.default_rng(3)
    x = g.standard_normal((cfg.tokens, cfg.num_heads, cfg.head_dim))
    np.testing.assert_allclose(rope.rope_frame(cfg, x, 6), brute.frame_rope(cfg, x, 6), atol=1e-12)


def test_default_split():
    assert default_rope_split(128) == (44, 42, 42)
    assert default_rope_split(64) == (24, 20, 20)
