"""Brute-force references used to pin the oracle (tests only).

Written separately from ``oracle/``: RoPE through complex multiplication instead of cos/sin
pair formulas, keys gathered from the full frame history by index arithmetic instead of a
cache, and attention through ``torch.nn.functional.scaled_dot_product_attention`` in float64.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from synth import inputs


def to_f64(cfg, x):
    if cfg.dtype == "bf16":
        return torch.from_numpy(np.asarray(x).view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    return np.asarray(x, np.float64)


def complex_rope(cfg, x, t_pos, h_pos, w_pos):
    """x[..., d] rotated: pair j of axis a is the complex number x_2j + i x_2j+1 times e^{i pos w_j}."""
    z = x[..., 0::2] + 1j * x[..., 1::2]
    parts = []
    for dim, pos in ((cfg.rope_dim_t, t_pos), (cfg.rope_dim_h, h_pos), (cfg.rope_dim_w, w_pos)):
        j = np.arange(dim // 2)
        freq = np.power(float(cfg.rope_theta), -(2.0 * j) / dim)
        parts.append(np.exp(1j * np.multiply.outer(np.asarray(pos, np.float64), freq)))
    rot = np.concatenate(parts, axis=-1)                # broadcasts against z's trailing axes
    zr = z * rot
    out = np.empty(x.shape)
    out[..., 0::2] = zr.real
    out[..., 1::2] = zr.imag
    return out


def frame_rope(cfg, x, t_pos):
    """x[N, H, d] of one frame at temporal position t_pos (complex route)."""
    n = np.arange(cfg.tokens)
    hh, ww = n // cfg.grid_w, n % cfg.grid_w
    rot_in = np.moveaxis(x, 1, 0)                       # [H, N, d]
    out = complex_rope(cfg, rot_in, np.full(cfg.tokens, t_pos), hh, ww)
    return np.moveaxis(out, 0, 1)


def sdpa(q, k, v, scale, mask=None):
    """float64 attention per head via torch: q[M,H,d], k/v[L,H,d], mask[M,L] True = attend."""
    qt = torch.from_numpy(np.ascontiguousarray(np.moveaxis(q, 1, 0)))
    kt = torch.from_numpy(np.ascontiguousarray(np.moveaxis(k, 1, 0)))
    vt = torch.from_numpy(np.ascontiguousarray(np.moveaxis(v, 1, 0)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return np.moveaxis(o.numpy(), 0, 1)


def round_e4m3(x):
    """Round to OCP e4m3 another way than oracle.fp8's table search: scale by the quantum of x's
    binade (3 mantissa bits; the subnormal quantum 2^-9 below 2^-6), round half to even,
    saturate at 448."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)                                  # |x| in [2^(e-1), 2^e)
    q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.clip(np.round(x / q) * q, -448.0, 448.0)


def committed_frame_kv(cfg, frame, layer):
    """K, V (float64 [N,H,d]) of a frame as committed: element 0's inputs at step c + B - 1."""
    T, N, B = cfg.chunk_frames, cfg.tokens, cfg.stream_batch
    c = frame // T
    _, k, v = inputs.qkv(cfg, c + B - 1, layer, 0)
    r = (frame % T) * N
    return to_f64(cfg, k)[r:r + N], to_f64(cfg, v)[r:r + N]


def refresh_base(cfg, step):
    """RoPE base b0 at a step, from the schedule alone: the largest multiple of T_reset not
    above the newest in-flight frame (0 without refresh)."""
    T_reset = cfg.rope_refresh_period
    if T_reset == 0:
        return 0
    f_new = (min(step, cfg.num_chunks - 1) + 1) * cfg.chunk_frames - 1
    return T_reset * (f_new // T_reset)


def history_output(cfg, s, elem, layer, sink_frames=None, pinned_sinks=False, fp8=False):
    """Output of one element at step s from the frame history.

    Keys: sinks = the first S frames (or the frames listed in sink_frames), window = the last W
    committed non-sink frames, own chunk block-causal; every frame rotated at its absolute
    index.  Without pinned_sinks the stream has no refresh.  With pinned_sinks the stream may
    refresh and the sinks keep the label they had when committed, f - b0(commit step); since
    scores depend only on position differences, that is a sink placed at absolute position
    f - b0(commit step) + b0(s) against everything else at its absolute index.

    fp8: the e4m3 cache, where rounding makes scores depend on the labels themselves, so every
    position is taken relative to b0(s).  A cached key is rotated at its commit-time label
    f - b0(commit step), rounded, then turned back by T_reset and rounded once per refresh
    since; values and the own chunk's keys are rounded once.
    """
    if fp8:
        assert not pinned_sinks
        return _history_output_fp8(cfg, s, elem, layer, sink_frames)
    assert pinned_sinks or cfg.rope_refresh_period == 0
    T, N, B, S, W = cfg.chunk_frames, cfg.tokens, cfg.stream_batch, cfg.sink_frames, cfg.window_frames
    chunk = max(0, s - B + 1) + elem
    n_committed = max(0, s - B + 1) * T                    # frames of chunks already committed
    sinks = list(range(min(S, n_committed))) if sink_frames is None else list(sink_frames)
    frames = sinks + list(range(max(S, n_committed - W), n_committed))
    k_parts, v_parts, kf = [], [], []
    for i, f in enumerate(frames):
        k, v = committed_frame_kv(cfg, f, layer)
        pos = f
        if pinned_sinks and i < len(sinks):
            pos = f - refresh_base(cfg, f // T + B - 1) + refresh_base(cfg, s)
        k_parts.append(frame_rope(cfg, k, pos))
        v_parts.append(v)
        kf.append(np.full(N, -1))
    q, k, v = (to_f64(cfg, a) for a in inputs.qkv(cfg, s, layer, elem))
    for t in range(T):
        g = chunk * T + t
        k_parts.append(frame_rope(cfg, k[t * N:(t + 1) * N], g))
        v_parts.append(v[t * N:(t + 1) * N])
        kf.append(np.full(N, g))
    q_rot = np.concatenate([frame_rope(cfg, q[t * N:(t + 1) * N], chunk * T + t) for t in range(T)])
    qf = chunk * T + np.arange(T * N) // N
    mask = np.concatenate(kf)[None, :] <= qf[:, None]
    return sdpa(q_rot, np.concatenate(k_parts), np.concatenate(v_parts), cfg.softmax_scale, mask)


def e4m3_key_factor(cfg):
    """The documented key factor of a key-scaled e4m3 cache, from its definition: c =
    key_scale * log2(e), k = -floor(log2(c) + 1/2), g = fp32(c * 2^k); 1 without a key scale."""
    ks = getattr(cfg, "key_scale", 0.0)
    if not ks > 0:
        return 1.0
    c = ks * math.log2(math.e)
    k = -math.floor(math.log2(c) + 0.5)
    return float(np.float32(math.ldexp(c, k)))


def _history_output_fp8(cfg, s, elem, layer, sink_frames):
    T, N, B, S, W = cfg.chunk_frames, cfg.tokens, cfg.stream_batch, cfg.sink_frames, cfg.window_frames
    T_reset = cfg.rope_refresh_period
    chunk = max(0, s - B + 1) + elem
    n_committed = max(0, s - B + 1) * T
    sinks = list(range(min(S, n_committed))) if sink_frames is None else list(sink_frames)
    frames = sinks + list(range(max(S, n_committed - W), n_committed))
    b_s = refresh_base(cfg, s)
    gk = e4m3_key_factor(cfg)                 # keys are stored times gk and read back divided
    k_parts, v_parts, kf = [], [], []
    for f in frames:
        k, v = committed_frame_kv(cfg, f, layer)
        c_step = f // T + B - 1                   # the step that committed frame f
        b_c = refresh_base(cfg, c_step)
        key = round_e4m3(gk * frame_rope(cfg, k, f - b_c))
        # each later step whose base moved turns the stored key back by that step's move, once
        for s2 in range(c_step + 1, s + 1):
            d = refresh_base(cfg, s2) - refresh_base(cfg, s2 - 1)
            if d:
                key = round_e4m3(complex_rope(cfg, key, -d, 0, 0))
        k_parts.append(key / gk)
        v_parts.append(round_e4m3(v))
        kf.append(np.full(N, -1))
    q, k, v = (to_f64(cfg, a) for a in inputs.qkv(cfg, s, layer, elem))
    for t in range(T):
        g = chunk * T + t
        k_parts.append(round_e4m3(gk * frame_rope(cfg, k[t * N:(t + 1) * N], g - b_s)) / gk)
        v_parts.append(round_e4m3(v[t * N:(t + 1) * N]))
        kf.append(np.full(N, g))
    q_rot = np.concatenate([frame_rope(cfg, q[t * N:(t + 1) * N], chunk * T + t - b_s) for t in range(T)])
    qf = chunk * T + np.arange(T * N) // N
    mask = np.concatenate(kf)[None, :] <= qf[:, None]
    return sdpa(q_rot, np.concatenate(k_parts), np.concatenate(v_parts), cfg.softmax_scale, mask)


def run_oracle(cfg, steps=None, layers=(0,), embeddings=False, embed_fn=None):
    """Drive the oracle stream on the seeded inputs; returns (stream, outputs[(s, layer, elem)]).

    Chunk embeddings come from embed_fn(chunk) when given, else from the seeded generator when
    `embeddings` is set.
    """
    import oracle.stream as ost
    st = ost.OracleStream(cfg, layers=layers)
    outs = {}
    for s in range(cfg.num_steps if steps is None else steps):
        plan = st.begin_step(s)
        kv0 = {}
        for layer in layers:
            for b in range(len(plan["chunks"])):
                q, k, v = inputs.qkv(cfg, s, layer, b)
                outs[(s, layer, b)] = st.attend(layer, b, q, k, v)
                if b == 0:
                    kv0[layer] = (k, v)
        emb = None
        if plan["commit"] is not None:
            if embed_fn is not None:
                emb = embed_fn(plan["commit"])
            elif embeddings:
                emb = inputs.chunk_embedding(cfg, plan["commit"])
        st.end_step(kv0, emb)
    return st, outs
