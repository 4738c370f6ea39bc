"""Named workloads for the sink + rolling-KV chunk-attention path.

Plain data: shapes, stream lengths and constants of each synthetic workload.  Nothing here
computes any step of the method; both the oracle and the GPU path read these fields.

Shapes follow the pages' models: Wan2.1 1.3B (dim 1536 = 12 heads x 128) and 14B (dim 5120 =
40 heads x 128); a 512x512 frame gives a 32x32 token grid per latent frame and 480x832 gives
30x52 (StreamDiffusionV2 MLSys 2026 wiki page, "Experiments and results" and "Design
trade-offs" - boundary conditions Wan-T2V 1.3B/14B, 512^2/480p).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class MotionConfig:
    """Latent frames for the motion estimate (VAE latent: channels x height x width, fp32)."""
    channels: int
    height: int
    width: int
    frames: int            # F + 1 latent frames x_0 .. x_F
    delta: float           # RMS step of the smooth drift
    jump_prob: float       # probability that a frame is a fresh N(0,1) "cut"
    sigma: float           # statistical scale factor of the normalisation
    window: int            # k, frames in the normalisation window
    lam: float             # EMA update rate
    s_min: float
    s_max: float

    @property
    def elems(self) -> int:
        return self.channels * self.height * self.width


@dataclass(frozen=True)
class StreamConfig:
    name: str
    cfg_id: int                       # seed component
    num_layers: int
    num_heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    sink_frames: int                  # S
    window_frames: int                # W
    chunk_frames: int                 # T'
    stream_batch: int                 # B
    rope_dim_t: int
    rope_dim_h: int
    rope_dim_w: int
    rope_theta: float
    rope_refresh_period: int          # T_reset, 0 = never
    dtype: str                        # "fp32" | "bf16"
    num_chunks: int                   # M chunks enter the pipeline
    q_prescale: float                 # q ~ N(0,1) * q_prescale before rounding
    softmax_scale: float
    embed_dim: int = 0                # D, 0 = no chunk embeddings
    sink_threshold: Optional[float] = None   # tau, None = sink refresh off
    embed_kind: Optional[str] = None         # "iid" | "scenes"
    scene_change_prob: float = 0.0
    scene_noise: float = 0.0
    motion: Optional[MotionConfig] = None
    rope_pin_sinks: bool = False      # refresh leaves the sinks' labels pinned (alternative reading)
    kv_fp8: bool = False              # bf16 activations with an OCP e4m3 KV cache
    scaled_keys: bool = True          # cache option: keys stored times the softmax scale (where allowed)

    @property
    def tokens(self) -> int:          # N tokens per latent frame
        return self.grid_h * self.grid_w

    @property
    def key_scale(self) -> float:     # the cache's key scale: the softmax scale, or 0 (keys as rotated)
        ok = self.scaled_keys and self.dtype == "bf16" and self.head_dim == 128
        return self.softmax_scale if ok else 0.0

    @property
    def chunk_rows(self) -> int:      # T' * N query rows per chunk
        return self.chunk_frames * self.tokens

    @property
    def num_steps(self) -> int:       # M chunks + (B - 1) drain steps
        return self.num_chunks + self.stream_batch - 1

    def with_(self, **kw) -> "StreamConfig":
        return replace(self, **kw)


def default_rope_split(head_dim: int) -> tuple[int, int, int]:
    """t/h/w split of head_dim: d_h = d_w = 2*floor(d/6), d_t = d - 2*d_h (44/42/42 at 128)."""
    dh = 2 * (head_dim // 6)
    return head_dim - 2 * dh, dh, dh


TINY_FP32 = StreamConfig(
    name="tiny_fp32", cfg_id=1, num_layers=1, num_heads=2, head_dim=64, grid_h=4, grid_w=4,
    sink_frames=1, window_frames=4, chunk_frames=1, stream_batch=1,
    rope_dim_t=24, rope_dim_h=20, rope_dim_w=20, rope_theta=10000.0, rope_refresh_period=8,
    dtype="fp32", num_chunks=12, q_prescale=1.0, softmax_scale=1.0 / math.sqrt(64),
    embed_dim=64, sink_threshold=0.9, embed_kind="iid")

WAN13B_1LAYER = StreamConfig(
    name="wan13b_512_1layer", cfg_id=2, num_layers=1, num_heads=12, head_dim=128, grid_h=32,
    grid_w=32, sink_frames=1, window_frames=8, chunk_frames=1, stream_batch=1,
    rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, rope_theta=10000.0, rope_refresh_period=32,
    dtype="bf16", num_chunks=64, q_prescale=1.0 / math.sqrt(128), softmax_scale=1.0)

WAN13B_30LAYER_B4 = StreamConfig(
    name="wan13b_512_30layer_b4", cfg_id=3, num_layers=30, num_heads=12, head_dim=128,
    grid_h=32, grid_w=32, sink_frames=1, window_frames=8, chunk_frames=1, stream_batch=4,
    rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, rope_theta=10000.0, rope_refresh_period=0,
    dtype="bf16", num_chunks=128, q_prescale=1.0, softmax_scale=1.0 / math.sqrt(128))

WAN13B_480P_B2 = StreamConfig(
    name="wan13b_480p_30layer_b2", cfg_id=4, num_layers=30, num_heads=12, head_dim=128,
    grid_h=30, grid_w=52, sink_frames=2, window_frames=6, chunk_frames=1, stream_batch=2,
    rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, rope_theta=10000.0, rope_refresh_period=24,
    dtype="bf16", num_chunks=128, q_prescale=1.0, softmax_scale=1.0 / math.sqrt(128),
    motion=MotionConfig(channels=16, height=60, width=104, frames=129, delta=0.05,
                        jump_prob=0.05, sigma=1.0, window=4, lam=0.9, s_min=0.25, s_max=1.0))

WAN14B_40LAYER_B4 = StreamConfig(
    name="wan14b_512_40layer_b4", cfg_id=5, num_layers=40, num_heads=40, head_dim=128,
    grid_h=32, grid_w=32, sink_frames=1, window_frames=8, chunk_frames=1, stream_batch=4,
    rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, rope_theta=10000.0, rope_refresh_period=0,
    dtype="bf16", num_chunks=96, q_prescale=1.0, softmax_scale=1.0 / math.sqrt(128),
    embed_dim=5120, sink_threshold=0.95, embed_kind="scenes", scene_change_prob=0.08,
    scene_noise=0.05)

# T' = 2 frames per chunk with B = 2: the same four frames per step as the B = 4 workload, with
# block-causal attention inside each chunk ([WT] SLO-aware batching scheduler: chunk size T' and
# stream batch B are the two latency knobs).
WAN13B_30LAYER_T2B2 = StreamConfig(
    name="wan13b_512_30layer_t2b2", cfg_id=6, num_layers=30, num_heads=12, head_dim=128,
    grid_h=32, grid_w=32, sink_frames=1, window_frames=8, chunk_frames=2, stream_batch=2,
    rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, rope_theta=10000.0, rope_refresh_period=0,
    dtype="bf16", num_chunks=64, q_prescale=1.0, softmax_scale=1.0 / math.sqrt(128))

ALL = [TINY_FP32, WAN13B_1LAYER, WAN13B_30LAYER_B4, WAN13B_480P_B2, WAN14B_40LAYER_B4,
       WAN13B_30LAYER_T2B2]
BY_NAME = {c.name: c for c in ALL}
