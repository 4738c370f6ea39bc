"""The sink + rolling-window stream, float64, step by step.  Test infrastructure only.

State is kept in the plainest form, independent of any device layout:

* raw (pre-RoPE) K and V of every cached frame plus an explicit temporal position label;
  RoPE is applied to keys at attention time;
* the sinks as a list of S entries and the window as a chronological list (oldest first),
  not a ring buffer.

Sources and readings:

* Sink frames + rolling window ([NEWS] algorithm item 1: the earliest frames' KV stay as sink
  tokens, the rest of the cache rolls; [REPO] core components: ring-buffer KV cache with
  sliding-window attention).  Keys of a chunk: every present sink, the last <= W committed
  non-sink frames, and the chunk's own frames (block-causal inside the chunk).  The window is
  kept as a list here; ring_slot() states where a ring of W + T' slots places each frame.
* Stream batch ([NEWS] system item 1, [WT] "可擴展的pipeline編排": B chunks at different noise
  levels in one call, one finished frame per call; [REPO] quick example: denoise returns
  nothing while the pipeline fills).  At step s the in-flight chunks are
  c in [max(0, s-B+1), min(s, M-1)], element b = c - max(0, s-B+1); element 0 is the oldest
  and is the one that finishes and is committed at the end of the step.
* RoPE refresh ([WT] "自適應的sink和RoPE刷新": when the frame index passes a threshold the RoPE
  phase is reset).  Reading: at the start of a step, while the newest in-flight frame f_new
  satisfies f_new - b0 >= T_reset, b0 += T_reset and every cached label drops by T_reset.
  Alternative reading (cfg.rope_pin_sinks; the same passage speaks of resetting the temporal
  anchors): only the window's labels drop, the sinks keep theirs, so the distance from the
  current frame to the sinks resets with the phase.
* Sink refresh (same sub-section: cosine similarity of the new chunk embedding against the
  sink set; the least similar sink is refreshed when the similarity is below a threshold).
  Reading: after the commit of frame f >= S, alpha_j = cos(h, e_j), j* = argmin (lowest index
  on ties); if alpha_j* < tau the sink j* takes frame f's (K, V, label) for all layers and
  e_j* = h.  Frame f also stays in the window.
* FP8 cache (cfg.kv_fp8; [REPO] future work and [WT] trade-offs name an FP8 KV cache without a
  format).  Reading: the cache holds what the exact stream would hold, each element rounded to
  OCP e4m3 (oracle.fp8): a key is rotated at its label and then rounded, a value is rounded;
  this covers the chunk's own frames as well, since they are read from the cache.  A RoPE
  refresh turns each stored key's temporal pairs by -T_reset and rounds again (the stored
  keys are all the cache has).  Queries, scores and outputs keep their own precision.
  With a key scale (cfg.key_scale > 0) the cache stores every key times the fp32 factor
  g = key_scale * log2(e) * 2^k, k = -floor(log2(key_scale * log2(e)) + 1/2) (so that the keys
  keep their O(1) range in e4m3), rounded after the product; attention divides g out again.
"""
from __future__ import annotations

import copy
from dataclasses import dataclass, field

import numpy as np

from . import fp8 as ofp8
from . import rope
from .attention import attention
from .sink import decide, similarity_terms


def decode(cfg, x: np.ndarray) -> np.ndarray:
    """Storage array (bf16 bit patterns or float32) -> float64 values."""
    if cfg.dtype == "bf16":
        return (np.asarray(x, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(x, np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 values -> the nearest bf16 values (via float32, then round half to even on the
    16 dropped bits), as float64.  Finite inputs only."""
    b = np.asarray(x, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def fp8_key_factor(key_scale: float) -> float:
    """The e4m3 cache's key factor g (module docstring): 1 without a key scale."""
    if not key_scale > 0:
        return 1.0
    c = key_scale * np.log2(np.e)
    k = -int(np.floor(np.log2(c) + 0.5))
    return float(np.float32(c * 2.0 ** k))


def schedule(cfg, s: int) -> dict:
    """Chunks in flight at step s (element order), the chunk committed at its end, f_new."""
    B, M, T = cfg.stream_batch, cfg.num_chunks, cfg.chunk_frames
    lo, hi = max(0, s - B + 1), min(s, M - 1)
    chunks = list(range(lo, hi + 1))
    c0 = s - B + 1
    return {"chunks": chunks,
            "commit": c0 if 0 <= c0 < M else None,
            "newest_frame": (hi + 1) * T - 1 if chunks else None}


def ring_slot(cfg, frame: int) -> int:
    """Cache slot of a frame once its chunk is appended: sinks are slots [0, S); frame f >= S
    lives in ring slot S + f mod (W + T').

    Reading ([REPO] core components: a ring-buffer KV cache with sliding-window attention;
    [NEWS] algorithm item 1): the step appends the new chunk's K/V into the ring while the
    chunk still attends the W committed frames before it, so the ring holds W + T' frames -
    the window plus the chunk being written - and a frame's slot is its index modulo that
    length.  The T' slots of chunk c hold frames c*T' - W - T' .. c*T' - W - 1, which left the
    window when chunk c - 1 was committed, so writing chunk c into its final slots disturbs no
    attended frame."""
    S, W, T = cfg.sink_frames, cfg.window_frames, cfg.chunk_frames
    return frame if frame < S else S + frame % (W + T)


@dataclass
class Entry:
    frame: int
    label: int                                   # temporal RoPE position of the cached frame
    # layer -> (K, V) float64 [N,H,d]: K raw (pre-RoPE), or rotated at `label` and e4m3 in FP8 mode
    kv: dict = field(default_factory=dict)


class OracleStream:
    def __init__(self, cfg, layers=None):
        self.cfg = cfg
        self.layers = list(range(cfg.num_layers)) if layers is None else list(layers)
        self.base = 0                                # b0
        self.sinks: list[Entry | None] = [None] * cfg.sink_frames
        self.sink_embed: list[np.ndarray | None] = [None] * cfg.sink_frames
        self.window: list[Entry] = []
        self.refresh_log: list[tuple[int, int]] = []          # (step, new b0)
        self.sink_log: list[dict] = []
        self.step = -1
        self.plan = None
        self.kv_fp8 = bool(getattr(cfg, "kv_fp8", False))
        self.key_mul = fp8_key_factor(getattr(cfg, "key_scale", 0.0)) if self.kv_fp8 else 1.0

    # ---- step start: schedule + RoPE refresh ---------------------------------------------
    def begin_step(self, s: int) -> dict:
        assert s == self.step + 1, "steps must be consecutive"
        self.step = s
        self.plan = schedule(self.cfg, s)
        T_reset = self.cfg.rope_refresh_period
        f_new = self.plan["newest_frame"]
        n = 0
        while T_reset > 0 and f_new is not None and f_new - self.base >= T_reset:
            self.base += T_reset
            n += 1
            self.refresh_log.append((s, self.base))
        if n:
            # one refresh event per step: when the newest frame passes several periods at once
            # (T' > T_reset), the labels drop by the whole n T_reset and stored e4m3 keys turn
            # back by it once, with one rounding
            moved = self.window if self.cfg.rope_pin_sinks else self.cached_entries()
            for e in moved:
                e.label -= n * T_reset
                if self.kv_fp8:
                    e.kv = {layer: (self._turn_back(K, n * T_reset), V) for layer, (K, V) in e.kv.items()}
        return self.plan

    def _turn_back(self, K: np.ndarray, delta: int) -> np.ndarray:
        """Stored (rotated, e4m3) keys of a frame whose label drops by delta: the temporal
        pairs turn by -delta * omega (the row and column pairs by angle 0), then round."""
        phi = rope.angles(self.cfg, -float(delta), 0.0, 0.0)
        return ofp8.round_fp8(rope.rotate_pairs(K, phi))

    def _stored(self, K_raw: np.ndarray, V: np.ndarray, label: int):
        """What the cache keeps for a frame at a label: raw K and V (exact mode, RoPE applied
        when attending), or the rotated key (times the key factor) and the value rounded to
        e4m3."""
        if self.kv_fp8:
            K = rope.rope_frame(self.cfg, K_raw, label) * self.key_mul
            return ofp8.round_fp8(K), ofp8.round_fp8(V)
        return K_raw, V

    def key_rot(self, e: Entry, layer: int, heads=slice(None)) -> np.ndarray:
        """Rotated key of a cached entry at its label (the given heads)."""
        K = e.kv[layer][0][:, heads]
        return K / self.key_mul if self.kv_fp8 else rope.rope_frame(self.cfg, K, e.label)

    def cached_entries(self) -> list[Entry]:
        """Distinct cached entries: present sinks, then the window (oldest first)."""
        return [e for e in self.sinks if e is not None] + list(self.window)

    # ---- attention of one element ---------------------------------------------------------
    def attend(self, layer: int, elem: int, q, k, v, rows=None, heads=None, rotated="exact",
               key_scale=0.0) -> np.ndarray:
        """Output rows of element `elem` at the current step: float64 [len(rows), len(heads), d].

        q, k, v are that element's fresh storage arrays [T'N, H, d] (pre-RoPE).  rotated="bf16"
        rounds the rotated queries and keys to bf16 before the product, as a bf16 path stores
        them (reading R13: q_rot and the cached keys are bf16 tensors); the default keeps them
        exact.  With rotated="bf16" and key_scale > 0 the keys are rounded after a product by
        the fp32 value of key_scale * log2(e), as a cache created with that key scale holds
        them, and the product is divided out again.
        """
        cfg = self.cfg
        N, T = cfg.tokens, cfg.chunk_frames
        chunk = self.plan["chunks"][elem]
        rows = np.arange(T * N) if rows is None else np.asarray(rows)
        heads = np.arange(cfg.num_heads) if heads is None else np.asarray(heads)
        # heads are independent: only the requested ones are formed
        qd, kd, vd = (decode(cfg, x)[:, heads] for x in (q, k, v))

        # keys: cached entries at their labels, then the own chunk's frames at f - b0
        k_parts, v_parts, key_frame = [], [], []
        for e in self.cached_entries():
            k_parts.append(self.key_rot(e, layer, heads))
            v_parts.append(e.kv[layer][1][:, heads])
            key_frame.append(np.full(N, -1))                     # always visible
        own_frames = [chunk * T + t for t in range(T)]
        for t, g in enumerate(own_frames):
            own = self._stored(kd[t * N:(t + 1) * N], vd[t * N:(t + 1) * N], g - self.base)
            k_parts.append(own[0] / self.key_mul if self.kv_fp8 else rope.rope_frame(cfg, own[0], g - self.base))
            v_parts.append(own[1])
            key_frame.append(np.full(N, g))
        K_all = np.concatenate(k_parts)                            # [L, H, d]
        if rotated == "bf16" and cfg.dtype == "bf16" and not self.kv_fp8:
            if key_scale > 0:
                kmul = float(np.float32(key_scale * np.log2(np.e)))
                K_all = round_bf16(K_all * kmul) / kmul
            else:
                K_all = round_bf16(K_all)
        V_all = np.concatenate(v_parts)
        key_frame = np.concatenate(key_frame)

        q_frame = chunk * T + rows // N
        gh, gw = rope.token_grid(cfg.grid_h, cfg.grid_w)
        phi = rope.angles(cfg, (q_frame - self.base).astype(np.float64), gh[rows % N], gw[rows % N])
        Q_rot = rope.rotate_pairs(qd[rows], phi[:, None, :])       # [R, H, d]
        if rotated == "bf16" and cfg.dtype == "bf16":
            Q_rot = round_bf16(Q_rot)
        mask = key_frame[None, :] <= q_frame[:, None]              # block-causal own chunk

        out = np.empty((len(rows), len(heads), cfg.head_dim))
        for i in range(len(heads)):
            out[:, i], _ = attention(Q_rot[:, i], K_all[:, i], V_all[:, i], cfg.softmax_scale, mask)
        return out

    # ---- step end: commit + sink refresh ---------------------------------------------------
    def end_step(self, commit_kv: dict | None = None, embedding=None):
        """commit_kv: layer -> (k, v) storage arrays of element 0 at this step."""
        cfg = self.cfg
        c0 = self.plan["commit"]
        if c0 is None:
            return None
        N, T, S, W = cfg.tokens, cfg.chunk_frames, cfg.sink_frames, cfg.window_frames
        h = None if embedding is None else np.asarray(embedding, np.float32).astype(np.float64)
        entry = None
        for t in range(T):
            f = c0 * T + t
            entry = Entry(frame=f, label=f - self.base)
            for layer in self.layers:
                k, v = commit_kv[layer]
                entry.kv[layer] = self._stored(decode(cfg, k)[t * N:(t + 1) * N],
                                               decode(cfg, v)[t * N:(t + 1) * N], entry.label)
            if f < S:
                self.sinks[f] = entry
                self.sink_embed[f] = h
            else:
                self.window.append(entry)
                if len(self.window) > W:
                    self.window.pop(0)
        decision = None
        if cfg.sink_threshold is not None and entry.frame >= S and S > 0:
            terms = similarity_terms(h, self.sink_embed)
            j, alpha, replace = decide(h, self.sink_embed, cfg.sink_threshold)
            if replace:
                self.sinks[j] = copy.deepcopy(entry)
                self.sink_embed[j] = h
            decision = {"step": self.step, "chunk": c0, "frame": entry.frame, "slot": j,
                        "alpha": alpha, "replaced": replace, "terms": terms}
            self.sink_log.append(decision)
        return decision
