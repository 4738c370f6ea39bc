"""Pins of the SLO-aware (B, T') choice: closed-form fits and hand-derived selections."""
import pytest

from oracle import slo


def test_fit_recovers_an_exact_line():
    frames = [1, 2, 4, 8]
    c0, c1 = slo.fit_latency(frames, [0.003 + 0.0015 * x for x in frames])
    assert c0 == pytest.approx(0.003, abs=1e-15) and c1 == pytest.approx(0.0015, abs=1e-15)


def test_fit_of_symmetric_noise_is_the_middle_line():
    # +e and -e around a line at mirrored points leave the least-squares line unchanged
    frames = [1, 1, 3, 3]
    c0, c1 = slo.fit_latency(frames, [1.0 + 0.1, 1.0 - 0.1, 2.0 + 0.1, 2.0 - 0.1])
    assert c0 == pytest.approx(0.5, abs=1e-14) and c1 == pytest.approx(0.5, abs=1e-14)


def test_constant_latency_takes_the_most_frames_and_breaks_ties_by_latency_then_b():
    # L = 10 ms for every (B, T'): f = 100 B T', highest at B T' = 8.  Latencies at f_target =
    # 100: (8,1) 0.08, (4,2) 0.04 + 0.01 = 0.05, (2,4) 0.02 + 0.03 = 0.05, (1,8) 0.01 + 0.07 =
    # 0.08 -> tie between (4,2) and (2,4) -> smaller B.
    best = slo.select(0.01, 0.0, 100.0, 1.0, frames_ready=8, max_batch=8, max_chunk=8)
    assert (best["B"], best["T"], best["feasible"]) == (2, 4, True)
    assert best["fps"] == pytest.approx(800.0) and best["latency"] == pytest.approx(0.05)


def test_deadline_and_ready_frames_bind():
    # L = 2 ms + 1 ms * B T'.  f rises with B T' (B T' = 8: 8 / 0.010 = 800 fps).  A 25 ms
    # deadline at f_target = 100 rules out B = 4, T' = 2 (4 * 10 ms + 10 ms = 50 ms) and every
    # B T' = 8 choice except (1, 8): 10 ms + 70 ms = 80 ms, also out.  B T' = 6: (1,6) 8 + 50 =
    # 58, (2,3) 16 + 20 = 36, (3,2) 24 + 10 = 34, (6,1) 48 -> out.  B T' = 4: (1,4) 6 + 30 = 36,
    # (2,2) 12 + 10 = 22 ms ok, (4,1) 24 ms ok -> f = 4 / 6 ms = 667 fps, tie -> lower latency (2,2).
    best = slo.select(0.002, 0.001, 100.0, 0.025, frames_ready=8, max_batch=8, max_chunk=8)
    assert (best["B"], best["T"], best["feasible"]) == (2, 2, True)
    # only 3 frames collected: B T' <= 3, and (1,3) 5 + 20 = 25 ms, (3,1) 15 ms -> (3,1)
    best = slo.select(0.002, 0.001, 100.0, 0.025, frames_ready=3, max_batch=8, max_chunk=8)
    assert (best["B"], best["T"]) == (3, 1)


def test_unreachable_target_returns_the_fastest_candidate_flagged():
    best = slo.select(0.01, 0.0, 1e6, 1.0, frames_ready=8, max_batch=2, max_chunk=2)
    assert (best["B"], best["T"], best["feasible"]) == (2, 2, False)
