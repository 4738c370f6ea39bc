"""SLO-aware choice of stream batch B and chunk size T', float64.  Test infrastructure only.

Source: [WT] method section, "SLO感知的批處理調度器" (SLO-aware batching scheduler).  The page
models the latency of one step as L(T', B) ~ (A(T', B) + P_model) / (eta * BW) with an
activation term A that grows linearly in B*T' under FlashAttention, asks that B*T' not exceed
the frames already collected, and gives the processing frequency f = B*T' / L(T', B).

Readings (the formulas on the page are stripped):
* L = c0 + c1 * B * T', c0 and c1 fitted by least squares to measured step latencies;
* a frame's latency is B * L (its chunk is in flight for B steps) plus (T' - 1) / f_target
  (waiting for the rest of its chunk's frames);
* feasible: f >= f_target and latency <= deadline; the choice is the feasible candidate of
  highest f (f within a relative 1e-12 counts as equal; ties: lower latency, then smaller B),
  else the highest-f candidate overall, flagged infeasible.
"""
from __future__ import annotations

import numpy as np

REL_TIE = 1e-12


def fit_latency(frames, latency):
    """Least-squares line latency = c0 + c1 * frames (frames = B * T' per step)."""
    x = np.asarray(frames, np.float64)
    y = np.asarray(latency, np.float64)
    A = np.stack([np.ones_like(x), x], axis=1)
    (c0, c1), *_ = np.linalg.lstsq(A, y, rcond=None)
    return float(c0), float(c1)


def candidates(c0, c1, target_fps, frames_ready, max_batch, max_chunk, limit=8):
    out = []
    for B in range(1, max_batch + 1):
        for T in range(1, max_chunk + 1):
            if B * T > min(frames_ready, limit):
                continue
            L = c0 + c1 * B * T
            out.append({"B": B, "T": T, "L": L, "fps": B * T / L,
                        "latency": B * L + (T - 1) / target_fps})
    return out


def select(c0, c1, target_fps, deadline, frames_ready, max_batch, max_chunk, limit=8):
    cands = candidates(c0, c1, target_fps, frames_ready, max_batch, max_chunk, limit)
    feasible = [c for c in cands if c["fps"] >= target_fps and c["latency"] <= deadline]
    pool = feasible if feasible else cands
    best = pool[0]
    for c in pool[1:]:
        if c["fps"] > best["fps"] * (1 + REL_TIE):
            best = c
        elif c["fps"] >= best["fps"] * (1 - REL_TIE):           # equal throughput
            if c["latency"] < best["latency"] or (c["latency"] == best["latency"] and c["B"] < best["B"]):
                best = c
    return dict(best, feasible=bool(feasible))
