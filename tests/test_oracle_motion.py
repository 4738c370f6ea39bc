"""Pins of the oracle's motion estimate and noise-rate EMA (oracle/motion.py)."""
import math

import numpy as np
import pytest

from oracle import motion


def test_identical_frames_give_zero_motion_and_max_noise():
    x = np.random.default_rng(0).standard_normal((1, 4, 6, 8))
    frames = np.repeat(x, 5, axis=0)
    d = motion.frame_distances(frames)
    assert np.all(d == 0.0)
    s = motion.noise_schedule(d, sigma=1.0, k=4, lam=0.9, s_min=0.25, s_max=1.0)
    assert np.all(s == 1.0)


def test_constant_rms_drift_gives_delta():
    g = np.random.default_rng(1)
    x = [g.standard_normal(999)]
    for _ in range(6):
        u = g.standard_normal(999)
        u /= math.sqrt(np.mean(u * u))
        x.append(x[-1] + 0.05 * u)
    np.testing.assert_allclose(motion.frame_distances(np.array(x)), 0.05, rtol=1e-12)


def test_jump_gives_sqrt2_and_clips():
    g = np.random.default_rng(2)
    frames = g.standard_normal((2, 16, 60, 104))
    d = motion.frame_distances(frames)
    assert d[0] == pytest.approx(math.sqrt(2.0), abs=0.01)
    assert motion.normalised(d, sigma=1.0, k=4)[0] == 1.0
    s = motion.noise_schedule(d, sigma=1.0, k=4, lam=1.0, s_min=0.25, s_max=1.0)
    assert s[0] == 0.25                                     # full motion -> lower bound


def test_window_max_hand_values():
    d = np.array([0.1, 0.5, 0.1, 0.1, 0.1, 0.1])
    # windows (k = 4): [0.1], [0.1,.5], [.1,.5,.1], [.1,.5,.1,.1], [.5,.1,.1,.1], [.1,.1,.1,.1]
    np.testing.assert_allclose(motion.normalised(d, sigma=1.0, k=4), [0.1, 0.5, 0.5, 0.5, 0.5, 0.1])
    np.testing.assert_allclose(motion.normalised(d, sigma=0.25, k=1), [0.4, 1.0, 0.4, 0.4, 0.4, 0.4])


def test_ema_closed_form_for_constant_target():
    # constant dhat -> constant target; s_t = target + (1 - lam)^t (s_0 - target)
    lam, s_min, s_max, dh = 0.3, 0.25, 1.0, 0.4
    d = np.full(12, dh)
    s = motion.noise_schedule(d, sigma=1.0, k=3, lam=lam, s_min=s_min, s_max=s_max, s0=1.0)
    target = s_max - (s_max - s_min) * dh
    t = np.arange(1, 13)
    np.testing.assert_allclose(s, target + (1 - lam) ** t * (1.0 - target), rtol=1e-14)


def test_more_motion_means_less_noise():
    lo = motion.noise_schedule(np.full(5, 0.1), 1.0, 4, 0.9, 0.25, 1.0)
    hi = motion.noise_schedule(np.full(5, 0.6), 1.0, 4, 0.9, 0.25, 1.0)
    assert np.all(hi < lo) and np.all(lo <= 1.0) and np.all(hi >= 0.25)
