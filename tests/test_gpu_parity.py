"""GPU parity: the HIP path against the float64 oracle on the same seeded inputs.

Bars: bit-exact slot table, V bytes, refresh events and sink decisions; outputs and cached K
within max-abs 1e-5 (fp32) or max-abs 2e-2 and mean-abs 2e-3 (bf16, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import Harness, assert_close, host64, log, sample_rows
from oracle import motion as omotion
from rolling_kv_causal_amd import sdv2
from synth import configs, inputs

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(rope_refresh_period=0, sink_threshold=None, embed_dim=0, embed_kind=None)
    base.update(kw)
    return configs.TINY_FP32.with_(**base)


def _stream(cfg, steps, layers=(0,), check=lambda s: True, rows=None, cache_check=lambda s: True):
    h = Harness(cfg, layers)
    worst = 0.0
    for s in range(steps):
        full = check(s)
        h.step(s, full=full)
        if full:
            worst = max(worst, h.check_outputs(rows=rows))
        h.finish_step()
        if cache_check(s):
            h.check_cache()
    log(f"{cfg.name}: {steps} steps, worst max-abs {worst:.3g}, refreshes {h.st.refresh_log}")
    return h


def test_tiny_fp32_full_stream():
    # 12 chunks: the ring wraps twice, refresh at frame 8, the sink refreshed by cosine rule
    cfg = configs.TINY_FP32
    h = _stream(cfg, cfg.num_steps)
    assert h.st.refresh_log == [(8, 8)]
    assert len(h.decisions) == cfg.num_chunks - cfg.sink_frames


def _keys_times_8(steps):
    """inputs.qkv with the keys of the chunks entering at `steps` scaled by 8 (exact in bf16)."""
    orig = inputs.qkv

    def qkv(cfg, step, layer, elem):
        q, k, v = orig(cfg, step, layer, elem)
        if step in steps:
            assert k.dtype == np.uint16
            f = (k.astype(np.uint32) << 16).view(np.float32) * np.float32(8.0)
            k = (f.view(np.uint32) >> 16).astype(np.uint16)
        return q, k, v
    return qkv


@pytest.mark.parametrize("grid", [(5, 13), (8, 16)], ids=["ragged-tiles", "full-tiles"])
def test_score_jump_rescales_mid_walk(monkeypatch, grid):
    # The keys of two committed frames are scaled by 8, so their scores rise far above the
    # running maximum of the tiles walked before them: the lazy rescale (row maximum, O and l
    # scaled, P recomputed) runs at tiles in the middle of the walk, in the masked variant too
    # when the tiles are ragged (65 tokens per frame), not only at the first tile.
    # Scores 8x larger also make the bf16 rounding of the rotated q and k (R13) 8x larger in
    # the scores, which the tolerance does not cover, so the oracle rounds them as the path
    # stores them; what is left to differ is the kernel's own arithmetic.  The attention is
    # then peaked, outputs reach |V| (up to about 4), and the bf16 bars apply relative to the
    # largest output magnitude of the element (bf16 carries relative precision).
    monkeypatch.setattr(inputs, "qkv", _keys_times_8({2, 5}))
    cfg = _small(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
                 grid_h=grid[0], grid_w=grid[1], num_heads=2, sink_frames=1, window_frames=4,
                 stream_batch=2, num_chunks=10, softmax_scale=128 ** -0.5)
    h = Harness(cfg, [0])
    worst = 0.0
    for s in range(cfg.num_steps):
        h.step(s, full=True)
        for b in range(len(h.st.plan["chunks"])):
            q, k, v = h.np_inputs[(0, b)]
            ref = h.st.attend(0, b, q, k, v, rotated="bf16")
            got = host64(h.run.out[0, b])
            scale = max(1.0, float(np.abs(ref).max()))
            worst = max(worst, assert_close(cfg, got, ref, f"out step {s} elem {b}", scale) / scale)
        h.finish_step()
    log(f"score jump {grid}: worst max-abs relative to max |out| {worst:.3g}")


@pytest.mark.parametrize("kw", [
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=5, grid_w=13,
         num_heads=3, sink_frames=2, window_frames=3, stream_batch=3, rope_refresh_period=5, num_chunks=14,
         softmax_scale=128 ** -0.5),
    dict(dtype="bf16", head_dim=64, grid_h=9, grid_w=11, num_heads=2, sink_frames=0, window_frames=2,
         stream_batch=2, num_chunks=9, num_layers=2),
    dict(dtype="fp32", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=3, grid_w=7,
         num_heads=2, sink_frames=1, window_frames=1, stream_batch=4, rope_refresh_period=3, num_chunks=10),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=12, grid_w=25,
         num_heads=4, sink_frames=3, window_frames=2, stream_batch=1, num_chunks=9, embed_dim=16,
         sink_threshold=0.2, embed_kind="iid", softmax_scale=128 ** -0.5),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=11, grid_w=13,
         num_heads=2, sink_frames=1, window_frames=2, stream_batch=2, num_chunks=8,
         softmax_scale=128 ** -0.5),
], ids=["bf16-ragged-B3-refresh", "bf16-d64-S0", "fp32-d128-W1-B4", "bf16-sinks-iid", "bf16-3-tiles-per-frame"])
def test_small_ragged_streams(kw):
    # token counts that are not multiples of the 64-key tile or the 128-row query tile,
    # degenerate windows (W = 1, S = 0), B up to 4, and several layers; 143 tokens give three
    # key tiles per frame, so the key walks have 3, 6 and 9 tiles (every phase of the 64-row
    # kernel's four-slot ring ends a walk)
    cfg = _small(**kw)
    _stream(cfg, cfg.num_steps, layers=range(cfg.num_layers))


def test_split_without_visible_keys_for_some_rows(monkeypatch):
    # Four splits forced over a T' = 2 chunk of 81 tokens (two tiles per frame) with one sink
    # and a window of one: at steady state the walk of the query tile is 8 tiles, and the last
    # split holds only own frame 1, which the rows of own frame 0 may not see.  Those rows keep
    # no maximum through that split (they go through the rescale every tile and end with l = 0
    # and m = -inf), and the combine must give that split no weight.
    monkeypatch.setenv("SDV2_NSPLIT", "4")
    cfg = _small(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, chunk_frames=2,
                 grid_h=9, grid_w=9, num_heads=2, sink_frames=1, window_frames=1, stream_batch=2,
                 num_chunks=7, softmax_scale=128 ** -0.5)
    assert sdv2.sdv2_cache_size(sdv2.config_of(cfg))[2] > 0     # the forced splits are in effect
    _stream(cfg, cfg.num_steps)


@pytest.mark.parametrize("kw", [
    dict(dtype="fp32", chunk_frames=2, grid_h=5, grid_w=7, num_heads=2, sink_frames=1, window_frames=3,
         stream_batch=2, rope_refresh_period=5, num_chunks=8, num_layers=2),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, chunk_frames=3, grid_h=6,
         grid_w=13, num_heads=3, sink_frames=2, window_frames=4, stream_batch=2, num_chunks=10, embed_dim=16,
         sink_threshold=0.2, embed_kind="iid", softmax_scale=128 ** -0.5),
    dict(dtype="bf16", chunk_frames=4, grid_h=9, grid_w=9, num_heads=2, sink_frames=0, window_frames=2,
         stream_batch=2, num_chunks=7),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, chunk_frames=2, grid_h=12,
         grid_w=12, num_heads=4, sink_frames=1, window_frames=2, stream_batch=4, rope_refresh_period=3,
         num_chunks=9, softmax_scale=128 ** -0.5),
], ids=["fp32-T2-B2-refresh", "bf16-T3-sinks-straddle", "bf16-T4-W2-S0", "bf16-T2-B4-refresh"])
def test_block_causal_chunks(kw):
    # T' frames per chunk: block-causal own chunk, T' frames per append and commit, a chunk that
    # straddles the sink boundary, a window shorter than the chunk, B * T' at its limit of 8
    cfg = _small(**kw)
    h = _stream(cfg, cfg.num_steps, layers=range(cfg.num_layers))
    if cfg.sink_threshold is not None:
        assert len(h.decisions) == cfg.num_chunks


@pytest.mark.parametrize("kw", [
    dict(dtype="fp32", rope_refresh_period=3, sink_frames=2, window_frames=3, stream_batch=2, num_chunks=12,
         rope_pin_sinks=True),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=5, grid_w=13,
         num_heads=3, sink_frames=1, window_frames=3, stream_batch=2, chunk_frames=2, rope_refresh_period=4,
         num_chunks=10, embed_dim=16, sink_threshold=0.2, embed_kind="iid", softmax_scale=128 ** -0.5,
         rope_pin_sinks=True),
], ids=["fp32-pinned-refresh", "bf16-pinned-T2-sink-refresh"])
def test_pinned_sink_refresh(kw):
    # refresh rebases only the window; the sinks' labels (checked in the slot table) stay
    cfg = _small(**kw)
    h = _stream(cfg, cfg.num_steps, layers=range(cfg.num_layers))
    assert len(h.st.refresh_log) >= 2


_D128 = dict(dtype="bf16", kv_fp8=True, head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
             softmax_scale=128 ** -0.5)


@pytest.mark.parametrize("kw", [
    dict(grid_h=5, grid_w=13, num_heads=3, sink_frames=2, window_frames=3, stream_batch=3,
         rope_refresh_period=5, num_chunks=14),
    dict(chunk_frames=2, grid_h=12, grid_w=12, num_heads=4, sink_frames=1, window_frames=2, stream_batch=4,
         rope_refresh_period=3, num_chunks=9, num_layers=2),
    dict(chunk_frames=3, grid_h=6, grid_w=13, num_heads=3, sink_frames=2, window_frames=4, stream_batch=2,
         num_chunks=10, embed_dim=16, sink_threshold=0.2, embed_kind="iid"),
    dict(grid_h=7, grid_w=9, num_heads=2, sink_frames=1, window_frames=3, stream_batch=2, chunk_frames=2,
         rope_refresh_period=4, num_chunks=10, rope_pin_sinks=True),
], ids=["ragged-B3-refresh", "T2-B4-refresh", "T3-sink-refresh", "pinned-T2"])
def test_fp8_kv_cache(kw):
    # e4m3 cache: token counts off the 32-token byte-permutation blocks, refresh re-rounding,
    # block-causal chunks, sink replacement (a byte copy) and pinned sinks
    cfg = _small(**dict(_D128, **kw))
    h = _stream(cfg, cfg.num_steps, layers=range(cfg.num_layers))
    assert len(h.st.refresh_log) >= (2 if cfg.rope_refresh_period else 0)


def test_fp8_kv_wan13b_single_layer_full_size():
    # the headline shape with an e4m3 cache, through the refresh at frame 32
    cfg = configs.WAN13B_1LAYER.with_(kv_fp8=True)
    checked = {1, 9, 31, 32, 33}
    rows = sample_rows(cfg.tokens, n=48, seed=5)
    h = _stream(cfg, 34, check=lambda s: s in checked, rows=rows, cache_check=lambda s: s in checked)
    assert h.st.refresh_log == [(32, 32)]


def test_fp8_kv_wan14b_40layer_b4_full_size():
    cfg = configs.WAN14B_40LAYER_B4.with_(kv_fp8=True, sink_threshold=None, embed_dim=0, embed_kind=None)
    rows = sample_rows(cfg.tokens, n=16, seed=6)
    h = Harness(cfg, layers=(39,))                       # the last layer: largest cache offsets
    for s in range(12):
        full = s in (3, 11)
        h.step(s, full=full)
        if full:
            h.check_outputs(rows=rows, heads=np.arange(0, 40, 3))
        h.finish_step()
        if full:
            h.check_cache()


def test_wan13b_30layer_t2b2_full_size():
    # split-KV with block-causal query tiles: splits of frame-0 rows end before own frame 1
    cfg = configs.WAN13B_30LAYER_T2B2
    checked = {1, 9, 10}
    rows = sample_rows(cfg.chunk_rows, n=32, seed=4)
    _stream(cfg, 11, layers=(0, 29), check=lambda s: s in checked, rows=rows,
            cache_check=lambda s: s in checked)


def test_wan13b_single_layer_full_size():
    cfg = configs.WAN13B_1LAYER
    checked = {0, 1, 8, 9, 10, 31, 32, 33, cfg.num_steps - 1}
    rows = sample_rows(cfg.tokens, n=48)
    h = _stream(cfg, cfg.num_steps, check=lambda s: s in checked, rows=rows,
                cache_check=lambda s: s in checked)
    assert h.st.refresh_log == [(32, 32)]


def test_wan13b_30layer_b4_full_size():
    cfg = configs.WAN13B_30LAYER_B4
    checked = {3, 12, 13}
    rows = sample_rows(cfg.tokens, n=24, seed=1)
    _stream(cfg, 14, layers=(0, 29), check=lambda s: s in checked, rows=rows,
            cache_check=lambda s: s in checked)


def test_wan13b_480p_b2_full_size_with_refresh():
    cfg = configs.WAN13B_480P_B2
    checked = {2, 10, 24, 25}
    rows = sample_rows(cfg.tokens, n=24, seed=2)
    h = _stream(cfg, 26, layers=(0,), check=lambda s: s in checked, rows=rows,
                cache_check=lambda s: s in checked)
    assert h.st.refresh_log == [(24, 24)]


def test_wan14b_40layer_b4_full_size_with_sink_refresh():
    cfg = configs.WAN14B_40LAYER_B4
    steps = 40
    rows = sample_rows(cfg.tokens, n=16, seed=3)
    h = Harness(cfg, layers=(0,))
    replaced = kept = 0
    for s in range(steps):
        full = s in (12, steps - 1)
        h.step(s, full=full)
        if full:
            h.check_outputs(rows=rows, heads=np.arange(0, 40, 3))
        dec = h.finish_step()
        if dec is not None:
            replaced += dec["replaced"]
            kept += not dec["replaced"]
        if full:
            h.check_cache()
    log(f"{cfg.name}: sink decisions replaced {replaced} kept {kept}")
    assert replaced >= 1 and kept >= 1


def test_motion_l2_and_noise_schedule():
    cfg = configs.WAN13B_480P_B2
    m = cfg.motion
    frames = inputs.motion_frames(cfg)
    x = torch.from_numpy(frames).cuda()
    F = m.frames - 1
    dist = torch.empty(F, dtype=torch.float64, device="cuda")
    ws = torch.empty(sdv2.sdv2_motion_workspace_size(m.frames, m.elems), dtype=torch.uint8, device="cuda")
    sdv2.sdv2_motion_l2(x, m.frames, m.elems, dist, ws)
    got = dist.cpu().numpy()
    want = omotion.frame_distances(frames)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
    rate = sdv2.sdv2_noise_schedule(list(got), m.sigma, m.window, m.lam, m.s_min, m.s_max, m.s_max)
    np.testing.assert_allclose(rate, omotion.noise_schedule(want, m.sigma, m.window, m.lam, m.s_min, m.s_max),
                               rtol=1e-12)
    # odd element count and unaligned base take the scalar path
    sdv2.sdv2_motion_l2(x.view(-1)[1:1 + 3 * 1001], 3, 1001, dist, ws)
    want2 = omotion.frame_distances(frames.reshape(-1)[1:1 + 3 * 1001].reshape(3, 1001))
    np.testing.assert_allclose(dist[:2].cpu().numpy(), want2, rtol=1e-12)


def test_repeat_runs_are_bitwise_identical():
    cfg = configs.WAN13B_1LAYER.with_(num_chunks=12)
    outs = []
    for _ in range(2):
        h = Harness(cfg, layers=(0,))
        for s in range(cfg.num_steps):
            h.step(s)
            h.finish_step()
        outs.append(h.run.out.clone())
    assert torch.equal(outs[0], outs[1])
