"""Pins of the oracle's attention and cache semantics against brute force and special cases."""
import numpy as np
import pytest

import brute
from oracle import attention as oatt
from oracle import stream as ost
from synth import inputs
from synth.configs import TINY_FP32


def tiny(**kw):
    base = dict(rope_refresh_period=0, sink_threshold=None, embed_dim=0, embed_kind=None)
    base.update(kw)
    return TINY_FP32.with_(**base)


def test_attention_matches_torch_sdpa_with_mask():
    g = np.random.default_rng(0)
    q, k, v = g.standard_normal((3, 9, 3, 16))
    q, k, v = q[:7], k, v
    mask = g.random((7, 9)) < 0.7
    mask[:, 0] = True
    want = brute.sdpa(q, k, v, 0.3, mask)
    for h in range(3):
        o, p = oatt.attention(q[:, h], k[:, h], v[:, h], 0.3, mask)
        np.testing.assert_allclose(o, want[:, h], atol=1e-12)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        assert np.all(p[~mask] == 0.0)


def test_attention_special_cases():
    g = np.random.default_rng(1)
    q, k = g.standard_normal((2, 11, 8))
    v = np.full((11, 8), 2.5)
    o, _ = oatt.attention(q, k, v, 1.0)
    np.testing.assert_allclose(o, 2.5, atol=1e-12)                 # V const -> O const
    v = g.standard_normal((11, 8))
    o, p = oatt.attention(np.zeros((4, 8)), k, v, 1.0)
    np.testing.assert_allclose(p, 1.0 / 11, atol=1e-15)            # Q = 0 -> uniform weights
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-12)


@pytest.mark.parametrize("B,T", [(1, 1), (3, 1), (2, 2)])
def test_no_eviction_equals_full_causal_history(B, T):
    # S = 0 and a window longer than the stream: the cache never evicts, so every element must
    # see exactly all committed frames plus its own chunk (block-causal) - plain attention over
    # the history.
    cfg = tiny(sink_frames=0, window_frames=64, stream_batch=B, chunk_frames=T, num_chunks=6)
    st, outs = brute.run_oracle(cfg)
    for s in range(cfg.num_steps):
        for b in range(len(ost.schedule(cfg, s)["chunks"])):
            np.testing.assert_allclose(outs[(s, 0, b)], brute.history_output(cfg, s, b, 0), atol=1e-12)


@pytest.mark.parametrize("S,W,B,T", [(1, 4, 1, 1), (2, 3, 2, 1), (1, 2, 4, 1), (0, 3, 1, 1), (3, 1, 2, 1),
                                     (2, 3, 2, 2), (1, 2, 2, 3), (2, 4, 1, 3)])
def test_sink_and_window_match_history(S, W, B, T):
    # keys = the first S frames + the last W committed non-sink frames + own chunk (block-causal);
    # T > 1 covers a window shorter than the chunk and a chunk straddling the sink boundary
    cfg = tiny(sink_frames=S, window_frames=W, stream_batch=B, chunk_frames=T, num_chunks=11 if T == 1 else 7)
    st, outs = brute.run_oracle(cfg)
    for s in range(cfg.num_steps):
        for b in range(len(ost.schedule(cfg, s)["chunks"])):
            np.testing.assert_allclose(outs[(s, 0, b)], brute.history_output(cfg, s, b, 0), atol=1e-12)


def test_frame0_attends_only_to_itself():
    cfg = tiny()
    st = ost.OracleStream(cfg)
    st.begin_step(0)
    q, k, v = inputs.qkv(cfg, 0, 0, 0)
    out = st.attend(0, 0, q, k, v)
    kr = brute.frame_rope(cfg, brute.to_f64(cfg, k), 0)
    qr = brute.frame_rope(cfg, brute.to_f64(cfg, q), 0)
    np.testing.assert_allclose(out, brute.sdpa(qr, kr, brute.to_f64(cfg, v), cfg.softmax_scale), atol=1e-12)


def test_elements_do_not_see_each_other():
    # element 0's output must not change when element 1's k/v change
    cfg = tiny(stream_batch=2, num_chunks=5)
    st, _ = brute.run_oracle(cfg, steps=3)
    plan = st.begin_step(3)
    q0, k0, v0 = inputs.qkv(cfg, 3, 0, 0)
    a = st.attend(0, 0, q0, k0, v0)
    b = st.attend(0, 0, q0, k0, v0)
    np.testing.assert_array_equal(a, b)
    q1, k1, v1 = inputs.qkv(cfg, 3, 0, 1)
    o1 = st.attend(0, 1, q1, k1, v1)
    o1b = st.attend(0, 1, q1, k1 * np.float32(2.0), v1 + np.float32(1.0))
    assert np.max(np.abs(o1 - o1b)) > 1e-3
    np.testing.assert_array_equal(st.attend(0, 0, q0, k0, v0), a)


def test_row_and_head_subsets_match_full():
    cfg = tiny(num_chunks=4)
    st, _ = brute.run_oracle(cfg, steps=3)
    st.begin_step(3)
    q, k, v = inputs.qkv(cfg, 3, 0, 0)
    full = st.attend(0, 0, q, k, v)
    rows, heads = [0, 5, 15], [1]
    np.testing.assert_allclose(st.attend(0, 0, q, k, v, rows=rows, heads=heads), full[rows][:, heads], atol=1e-13)
