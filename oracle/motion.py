"""Motion estimate and motion-aware noise rate, float64.  Test infrastructure only.

[NEWS] algorithm item 2: motion strength from the L2 distance between adjacent frames; more
motion -> less noise, less motion -> more noise.  [WT] "運動感知的噪聲調度器": the distance
between consecutive latent frames, normalised by a statistical scale factor over a short
k-frame window and clipped to [0, 1], then an EMA with update rate lambda in (0, 1) between
the bounds s_min and s_max.  Readings (formulas stripped):

* d_t = sqrt(sum (x_t - x_{t-1})^2 / n)          (root-mean-square distance, t >= 1)
* dhat_t = min(1, max_{i in [max(1, t-k+1), t]} d_i / sigma)
* target_t = s_max - (s_max - s_min) * dhat_t
* s_t = lambda * target_t + (1 - lambda) * s_{t-1},   s_0 = s_max (initial noise scale)
"""
from __future__ import annotations

import numpy as np


def frame_distances(frames: np.ndarray) -> np.ndarray:
    """d_t for t = 1..F from frames[F+1, ...]; float64 [F]."""
    x = np.asarray(frames, np.float64).reshape(len(frames), -1)
    diff = x[1:] - x[:-1]
    return np.sqrt(np.sum(diff * diff, axis=1) / x.shape[1])


def normalised(d: np.ndarray, sigma: float, k: int) -> np.ndarray:
    """dhat for d[0] = d_1 ... : max over the last k distances / sigma, clipped to 1."""
    out = np.empty(len(d))
    for i in range(len(d)):
        out[i] = min(1.0, max(d[max(0, i - k + 1):i + 1]) / sigma)
    return out


def noise_schedule(d: np.ndarray, sigma: float, k: int, lam: float, s_min: float,
                   s_max: float, s0: float | None = None) -> np.ndarray:
    """Noise rates s_1..s_F for distances d_1..d_F."""
    dhat = normalised(d, sigma, k)
    s = s_max if s0 is None else s0
    out = np.empty(len(d))
    for i, dh in enumerate(dhat):
        target = s_max - (s_max - s_min) * dh
        s = lam * target + (1.0 - lam) * s
        out[i] = s
    return out
