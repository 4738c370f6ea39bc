"""Softmax attention of one head, float64.  Test infrastructure only.

Textbook definition (the pages name FlashAttention only as the exact tiled form of it, [WT]
"SLO感知的批處理調度器"): z = scale * Q K^T, P = exp(z - max_row z) / sum_row, O = P V.
"""
from __future__ import annotations

import numpy as np


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              key_mask: np.ndarray | None = None):
    """O[M, d] and P[M, L] for q[M, d], k[L, d], v[L, d]; key_mask[M, L] True = attend."""
    z = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    if key_mask is not None:
        z = np.where(key_mask, z, -np.inf)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ np.asarray(v, np.float64), p
