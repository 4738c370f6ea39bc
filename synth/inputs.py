"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

Every array is drawn from ``numpy.random.SeedSequence([0, cfg_id, *keys])`` with PCG64, in
float32, then rounded once to the workload's storage dtype.  bf16 arrays are returned as their
raw 16-bit patterns (``uint16``) so that both sides consume exactly the same rounded values;
each side decodes them itself.

Nothing here computes a step of the method (no RoPE, attention, cache bookkeeping, motion
statistic or sink decision); it only produces inputs of the pages' shapes.
"""
from __future__ import annotations

import numpy as np

from .configs import StreamConfig

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_EMBED, TENSOR_MOTION, TENSOR_SCENE = 0, 1, 2, 3, 4, 5


def rng(cfg_id: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, cfg_id, *keys])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite by construction (normal samples), so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def _storage(cfg: StreamConfig, x: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(x)
    if cfg.dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(cfg.dtype)


def qkv(cfg: StreamConfig, step: int, layer: int, elem: int):
    """Fresh q, k, v of one stream-batch element at one (step, layer): [T'*N, H, d] each.

    q is multiplied by ``cfg.q_prescale`` before rounding.  Returns storage arrays
    (uint16 bf16 bits or float32).
    """
    shape = (cfg.chunk_rows, cfg.num_heads, cfg.head_dim)
    out = []
    for t in (TENSOR_Q, TENSOR_K, TENSOR_V):
        x = rng(cfg.cfg_id, step, layer, elem, t).standard_normal(shape, dtype=np.float32)
        if t == TENSOR_Q and cfg.q_prescale != 1.0:
            x = x * np.float32(cfg.q_prescale)
        out.append(_storage(cfg, x))
    return tuple(out)


def _scene_of_chunk(cfg: StreamConfig) -> np.ndarray:
    cuts = rng(cfg.cfg_id, TENSOR_SCENE).random(cfg.num_chunks) < cfg.scene_change_prob
    cuts[0] = False
    return np.cumsum(cuts)


def chunk_embedding(cfg: StreamConfig, chunk: int) -> np.ndarray:
    """fp32 [D] embedding of one chunk.

    "iid": N(0,1) per component.  "scenes": a unit scene direction plus ``scene_noise`` times
    a unit random direction; a new scene starts at seeded cuts (probability
    ``scene_change_prob`` per chunk), so consecutive chunks are either nearly parallel or
    nearly orthogonal.
    """
    if cfg.embed_dim <= 0:
        raise ValueError("workload has no chunk embeddings")
    if cfg.embed_kind == "iid":
        return rng(cfg.cfg_id, chunk, TENSOR_EMBED).standard_normal(cfg.embed_dim, dtype=np.float32)
    if cfg.embed_kind == "scenes":
        scene = int(_scene_of_chunk(cfg)[chunk % cfg.num_chunks]) + (chunk // cfg.num_chunks) * 1000
        s = rng(cfg.cfg_id, TENSOR_SCENE, scene, 1).standard_normal(cfg.embed_dim)
        u = rng(cfg.cfg_id, chunk, TENSOR_EMBED).standard_normal(cfg.embed_dim)
        e = s / np.linalg.norm(s) + cfg.scene_noise * u / np.linalg.norm(u)
        return e.astype(np.float32)
    raise ValueError(cfg.embed_kind)


def motion_frames(cfg: StreamConfig, frames: int | None = None) -> np.ndarray:
    """fp32 latent frames [F+1, C, H, W]: smooth drift with seeded jumps.

    x_0 ~ N(0,1).  Drift: u_t = unit-RMS(u_{t-1} + 0.1 z_t), x_t = x_{t-1} + delta*u_t.
    With probability ``jump_prob`` a frame is instead a fresh N(0,1) sample (a scene cut).
    """
    m = cfg.motion
    if m is None:
        raise ValueError("workload has no motion path")
    n = m.frames if frames is None else frames
    shape = (m.channels, m.height, m.width)
    g = rng(cfg.cfg_id, TENSOR_MOTION)
    jumps = g.random(n) < m.jump_prob
    out = np.empty((n,) + shape, dtype=np.float32)
    x = g.standard_normal(shape).astype(np.float32)
    u = g.standard_normal(shape)
    u /= np.sqrt(np.mean(u * u))
    out[0] = x
    for t in range(1, n):
        z = g.standard_normal(shape)
        if jumps[t]:
            x = z.astype(np.float32)
        else:
            u = u + 0.1 * z
            u /= np.sqrt(np.mean(u * u))
            x = (x + np.float32(m.delta) * u.astype(np.float32)).astype(np.float32)
        out[t] = x
    return out
