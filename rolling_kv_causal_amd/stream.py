"""Step-protocol driver over the C ABI: one stream step = refresh, per-layer append + attention,
commit of the finished element, sink refresh.

The schedule comes from sdv2_plan_step (stream batch B: chunks at different noise levels share
one call and the oldest finishes; nothing finishes while the pipeline fills - [NEWS] method,
system item 1; [REPO] quick example).  All compute runs in libsdv2.so; this module only orders
the calls and hands over torch device buffers.
"""
from __future__ import annotations

from typing import Callable, Optional

from . import sdv2


class StreamRunner:
    def __init__(self, cfg: sdv2.Config, num_chunks: int, scale: float, device="cuda"):
        import torch
        self.cfg = cfg
        self.num_chunks = num_chunks
        self.scale = scale
        self.cache = sdv2.Cache(cfg, device=device)
        self.dtype = torch.float32 if cfg.dtype == sdv2.SDV2_F32 else torch.bfloat16   # activations
        self.N = cfg.grid_h * cfg.grid_w
        self.rows = cfg.chunk_frames * self.N     # query rows per element: T' frames of N tokens
        self.out = torch.empty((cfg.num_layers, cfg.stream_batch, self.rows, cfg.num_heads, cfg.head_dim),
                               dtype=self.dtype, device=device)

    @property
    def num_steps(self) -> int:
        return self.num_chunks + self.cfg.stream_batch - 1

    def plan(self, step: int):
        return sdv2.sdv2_plan_step(self.cfg, self.num_chunks, step)

    def step(self, s: int, qkv: Callable[[int, int, int], tuple], embed: Optional[Callable] = None,
             latents: Optional[Callable] = None, stats=None, sink_sync: bool = True) -> dict:
        """Run step s.  qkv(s, layer, nbatch) -> (q, k, v) device tensors [nbatch][T'N][H][d]
        (q is rotated in place).  embed(chunk) -> fp32 device embedding or None.
        latents(frame) -> (previous, newest) fp32 device latent frames or None.  stats: fp64
        device tensor of 4 + 2S values receiving the chunk statistics, or None."""
        first, nb, commit, newest = self.plan(s)
        info = {"first": first, "nbatch": nb, "commit": commit, "refreshed": 0, "sink": None}
        if nb == 0:
            return info
        info["refreshed"] = self.cache.refresh(newest)
        for layer in range(self.cfg.num_layers):
            q, k, v = qkv(s, layer, nb)
            self.cache.append(layer, first, nb, q, k, v)
            self.cache.attention(layer, nb, q, self.out[layer, :nb], self.scale)
        if commit >= 0:
            self.cache.commit(commit)
            last = (commit + 1) * self.cfg.chunk_frames - 1   # the chunk's last frame
            e = embed(commit) if (embed is not None and self.cfg.embed_dim > 0) else None
            lat = latents(last) if latents is not None else None
            if e is not None or lat is not None or stats is not None:
                prev, cur = lat if lat is not None else (None, None)
                info["sink"] = self.cache.sink_replace(last, e, prev, cur, stats, sync=sink_sync)
        return info
