"""Seeded random small stream configurations across the library's limits, for parity sweeps:
activation and cache types (fp32, bf16, bf16 with an e4m3 cache), head_dim 64 or 128, random
even RoPE splits, frames from 1 token to four key tiles, S in [0, 3], W in [1, 6], T' in
[1, 3], B in [1, 4] with B T' <= 8, RoPE refresh, pinned sinks, sink refresh and key scaling
on or off.  The streams run long enough to fill the window and wrap it."""
from __future__ import annotations

import math

import numpy as np

from synth import configs


def random_config(seed: int):
    r = np.random.default_rng(1000 + seed)
    kind = str(r.choice(["fp32", "bf16", "e4m3"], p=[0.15, 0.55, 0.3]))
    d = 128 if kind == "e4m3" else int(r.choice([64, 128], p=[0.3, 0.7]))
    dt = 2 * int(r.integers(0, min(32, d // 2) + 1))
    dh = 2 * int(r.integers(0, (d - dt) // 2 + 1))
    dw = d - dt - dh
    gh, gw = (1, 1) if seed % 8 == 0 else (int(r.integers(1, 15)), int(r.integers(1, 15)))   # one token a frame
    S, W, T = int(r.integers(0, 4)), int(r.integers(1, 7)), int(r.integers(1, 4))
    B = int(r.integers(1, 8 // T + 1)) if T > 1 else int(r.integers(1, 5))
    B = min(B, 4)
    refresh = int(r.choice([0, 0, 2, 3, 5, 7]))
    sink_refresh = S >= 1 and bool(r.integers(2))
    scale = 1.0 / math.sqrt(d) if r.integers(2) else 1.0
    return configs.TINY_FP32.with_(
        name=f"random_{seed}", cfg_id=100 + seed, num_layers=int(r.integers(1, 3)), num_heads=int(r.integers(1, 5)),
        head_dim=d, grid_h=gh, grid_w=gw, sink_frames=S, window_frames=W, chunk_frames=T, stream_batch=B,
        rope_dim_t=dt, rope_dim_h=dh, rope_dim_w=dw, rope_refresh_period=refresh,
        dtype="fp32" if kind == "fp32" else "bf16", kv_fp8=kind == "e4m3",
        num_chunks=(S + W) // T + 3 + B, q_prescale=1.0 if scale < 1 else 1.0 / math.sqrt(d), softmax_scale=scale,
        embed_dim=16 if sink_refresh else 0, sink_threshold=float(r.choice([0.2, 0.5])) if sink_refresh else None,
        embed_kind="iid" if sink_refresh else None, rope_pin_sinks=S >= 1 and bool(r.integers(2)),
        scaled_keys=bool(r.integers(3)) or kind == "e4m3")   # (the e4m3 cache needs its key scale)


def forced_splits(seed: int):
    """A split-KV count forced on the stream (the SDV2_NSPLIT knob) for some bf16 head_dim-128
    configurations, else None (the work plan's own choice)."""
    c = random_config(seed)
    if c.dtype != "bf16" or c.head_dim != 128:
        return None
    return [None, 2, 3, 5][seed % 4]


SEEDS = list(range(100))
