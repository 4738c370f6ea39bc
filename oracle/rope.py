"""Three-axis rotary position embedding (RoPE), float64.  Test infrastructure only.

[WT] "自適應的sink和RoPE刷新" names a RoPE phase per frame index and a periodic phase reset,
but prints no RoPE formula (stripped).  Reading adopted: the standard rotary embedding
(RoFormer) applied per axis of a (t, h, w) token grid, as in Wan2.1-style video DiTs:

* head_dim d is split into d_t + d_h + d_w (all even); pairs are interleaved adjacent
  elements (x_{2i}, x_{2i+1});
* pair i of axis a (i restarting at 0 in each axis) turns by phi = pos_a * omega_{a,i} with
  omega_{a,i} = theta ** (-2 i / d_a);
* a rotation by phi maps (x, y) -> (x cos phi - y sin phi, x sin phi + y cos phi);
* token n of a frame sits at row h = n // grid_w, column w = n % grid_w (row-major);
* the temporal position of frame f is p = f - b0, where b0 is the RoPE base that the refresh
  advances.
"""
from __future__ import annotations

import numpy as np


def axis_frequencies(dim_axis: int, theta: float) -> np.ndarray:
    """omega_i = theta ** (-2 i / dim_axis) for i in [0, dim_axis / 2)."""
    i = np.arange(dim_axis // 2, dtype=np.float64)
    return theta ** (-2.0 * i / dim_axis)


def token_grid(grid_h: int, grid_w: int) -> tuple[np.ndarray, np.ndarray]:
    """(row, column) of every token of a frame, row-major."""
    n = np.arange(grid_h * grid_w)
    return n // grid_w, n % grid_w


def angles(cfg, t_pos, h_pos, w_pos) -> np.ndarray:
    """Rotation angle of every pair: [..., d/2] for broadcastable position arrays."""
    t = np.asarray(t_pos, dtype=np.float64)[..., None]
    h = np.asarray(h_pos, dtype=np.float64)[..., None]
    w = np.asarray(w_pos, dtype=np.float64)[..., None]
    at = t * axis_frequencies(cfg.rope_dim_t, cfg.rope_theta)
    ah = h * axis_frequencies(cfg.rope_dim_h, cfg.rope_theta)
    aw = w * axis_frequencies(cfg.rope_dim_w, cfg.rope_theta)
    shape = np.broadcast_shapes(at.shape[:-1], ah.shape[:-1], aw.shape[:-1])
    return np.concatenate([np.broadcast_to(at, shape + at.shape[-1:]),
                           np.broadcast_to(ah, shape + ah.shape[-1:]),
                           np.broadcast_to(aw, shape + aw.shape[-1:])], axis=-1)


def rotate_pairs(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs of x[..., d] by phi[..., d/2]."""
    x = np.asarray(x, dtype=np.float64)
    a, b = x[..., 0::2], x[..., 1::2]
    c, s = np.cos(phi), np.sin(phi)
    out = np.empty(np.broadcast_shapes(x.shape, phi.shape[:-1] + (x.shape[-1],)))
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def rope_frame(cfg, x: np.ndarray, t_pos: float) -> np.ndarray:
    """RoPE of one frame's tokens x[N, H, d] at temporal position t_pos."""
    gh, gw = token_grid(cfg.grid_h, cfg.grid_w)
    phi = angles(cfg, np.full(gh.shape, float(t_pos)), gh, gw)      # [N, d/2]
    return rotate_pairs(x, phi[:, None, :])
