"""GPU parity: the HIP path against the float64 oracle on the same seeded inputs.

Bars: bit-exact slot table, V bytes, refresh events and sink decisions; outputs and cached K
within max-abs 1e-5 (fp32) or max-abs 2e-2 and mean-abs 2e-3 (bf16, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import random_configs
from gpu_helpers import Harness, assert_close, dev, host64, log, sample_rows
from oracle import motion as omotion
from oracle import stream as ost
from rolling_kv_causal_amd import sdv2
from rolling_kv_causal_amd.stream import StreamRunner
from synth import configs, inputs

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(rope_refresh_period=0, sink_threshold=None, embed_dim=0, embed_kind=None)
    base.update(kw)
    return configs.TINY_FP32.with_(**base)


def _stream(cfg, steps, layers=(0,), check=lambda s: True, rows=None, cache_check=lambda s: True,
            all_rows_at=()):
    """Run both sides for `steps` steps; outputs checked at steps where check(s) holds (on the
    sampled rows, or on every row and head at the steps in all_rows_at)."""
    h = Harness(cfg, layers)
    worst = 0.0
    for s in range(steps):
        full = check(s) or s in all_rows_at
        h.step(s, full=full)
        if full:
            worst = max(worst, h.check_outputs(rows=None if s in all_rows_at else rows))
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


@pytest.mark.parametrize("scaled", [True, False], ids=["scaled-keys", "plain-keys"])
@pytest.mark.parametrize("grid", [(5, 13), (8, 16)], ids=["ragged-tiles", "full-tiles"])
def test_score_jump_rescales_mid_walk(monkeypatch, grid, scaled):
    # The keys of two committed frames are scaled by 8, so their scores rise far above the
    # running maximum of the tiles walked before them: the lazy rescale (row maximum, O and l
    # scaled, P recomputed) runs at tiles in the middle of the walk, in the masked variant too
    # when the tiles are ragged (65 tokens per frame), not only at the first tile.
    # Scores 8x larger make the bf16 rounding of the stored rotated q and k 8x larger in the
    # scores, so the oracle rounds them as the path stores them (rotated="bf16").  What is left
    # is the kernel's own arithmetic: fp32 sums, and the bf16 rounding of each weight P, of a
    # split's partial output and of the output.  With M the element's largest output (about
    # the largest value of V it attends, the attention being peaked), that allows 2^-9 M for
    # the output, 2^-9 M for a partial and 2 * 2^-9 M for the weights (a weighted mean of V
    # with weights perturbed by 2^-9 each moves by at most 2^-9 * 2 max|V|): max-abs 2^-7 M,
    # and a mean-abs of 2^-9 M.
    monkeypatch.setattr(inputs, "qkv", _keys_times_8({2, 5}))
    # (scaled: the cache holds K times the softmax scale (key_scale), rounded after the product,
    # and the oracle's storage mode rounds it the same way)
    cfg = _small(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
                 grid_h=grid[0], grid_w=grid[1], num_heads=2, sink_frames=1, window_frames=4,
                 stream_batch=2, num_chunks=10, softmax_scale=128 ** -0.5, scaled_keys=scaled)
    assert (cfg.key_scale > 0) == scaled
    h = Harness(cfg, [0])
    worst_rel = worst_abs = 0.0
    for s in range(cfg.num_steps):
        h.step(s, full=True)
        for b in range(len(h.st.plan["chunks"])):
            q, k, v = h.np_inputs[(0, b)]
            ref = h.st.attend(0, b, q, k, v, rotated="bf16", key_scale=cfg.key_scale)
            got = host64(h.run.out[0, b])
            M = max(1.0, float(np.abs(ref).max()))
            err = np.abs(got - ref)
            assert err.max() <= 2.0 ** -7 * M, f"step {s} elem {b}: max-abs {err.max():.3g}, M {M:.3g}"
            assert err.mean() <= 2.0 ** -9 * M, f"step {s} elem {b}: mean-abs {err.mean():.3g}, M {M:.3g}"
            worst_rel = max(worst_rel, float(err.max()) / M)
            worst_abs = max(worst_abs, float(err.max()))
        h.finish_step()
    log(f"score jump {grid}: worst max-abs {worst_abs:.3g}, relative to the largest output {worst_rel:.3g}")


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
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=5, grid_w=13,
         num_heads=3, sink_frames=2, window_frames=3, stream_batch=3, rope_refresh_period=5, num_chunks=14,
         softmax_scale=128 ** -0.5, scaled_keys=False),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=11, grid_w=13,
         num_heads=2, sink_frames=1, window_frames=2, stream_batch=2, num_chunks=8,
         softmax_scale=128 ** -0.5, scaled_keys=False),
], ids=["bf16-ragged-B3-refresh", "bf16-d64-S0", "fp32-d128-W1-B4", "bf16-sinks-iid", "bf16-3-tiles-per-frame",
        "bf16-ragged-B3-refresh-plain-keys", "bf16-3-tiles-per-frame-plain-keys"])
def test_small_ragged_streams(kw):
    # token counts that are not multiples of the 64-key tile or the 128-row query tile,
    # degenerate windows (W = 1, S = 0), B up to 4, and several layers; 143 tokens give three
    # key tiles per frame, so the key walks have 3, 6 and 9 tiles (every phase of the 64-row
    # kernel's four-slot ring ends a walk)
    cfg = _small(**kw)
    _stream(cfg, cfg.num_steps, layers=range(cfg.num_layers))


def test_sink_decisions_left_on_the_device():
    # sdv2_sink_replace with h_slot NULL (no host synchronisation): the decision and the copy
    # happen on the device only.  Every output matches the oracle, whose sinks follow its own
    # decisions; the fp64 statistics (alpha included) are checked at every commit; the cache
    # holds the oracle's sink bytes while the library reports the sink slots as unknown.
    cfg = _small(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=5,
                 grid_w=13, num_heads=2, sink_frames=2, window_frames=3, stream_batch=2, num_chunks=14,
                 embed_dim=16, sink_threshold=0.2, embed_kind="iid", rope_refresh_period=5,
                 softmax_scale=128 ** -0.5)
    h = Harness(cfg, [0], sink_sync=False)
    replaced = 0
    for s in range(cfg.num_steps):
        h.step(s, full=True)
        h.check_outputs()
        dec = h.finish_step()
        replaced += bool(dec and dec["replaced"])
        h.check_cache()
    assert h.sinks_unknown and replaced >= 2
    assert all(h.run.cache.slot_info(j)[0] == -2 for j in range(cfg.sink_frames))


@pytest.mark.parametrize("S,W,T", [(3, 60, 1), (2, 60, 2)], ids=["S3-W60-T1", "S2-W60-T2"])
def test_sixty_four_attended_frames(S, W, T):
    # the library's limit S + W + T' = 64 (the attended frames' slots fill one 64-lane register):
    # 65 tokens per frame (two key tiles, the second ragged), the window filled and wrapped, a
    # refresh every 20 frames; every output of every step, the cache at fill, wrap and the end
    cfg = _small(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=5, grid_w=13,
                 num_heads=2, sink_frames=S, window_frames=W, chunk_frames=T, stream_batch=2,
                 num_chunks=(S + W) // T + 12, rope_refresh_period=20, softmax_scale=128 ** -0.5)
    assert S + W + T == 64
    fill = (S + W) // T
    _stream(cfg, cfg.num_steps, cache_check=lambda s: s in (fill - 1, fill + 5, cfg.num_steps - 1))


@pytest.mark.parametrize("kv_fp8", [False, True], ids=["bf16", "e4m3"])
def test_sixteen_sinks_widest_temporal_rope_and_full_batch(kv_fp8):
    # the other limits at once: S = 16 sinks (the most the library takes) under sink refresh,
    # rope_dim_t = 64 (32 temporal pairs, the most) with a refresh every 5 frames, B T' = 8
    # (B = 4, T' = 2); every output of every step, the cache at fill, after refreshes and at the end
    cfg = _small(dtype="bf16", head_dim=128, rope_dim_t=64, rope_dim_h=32, rope_dim_w=32, grid_h=6, grid_w=11,
                 num_heads=2, sink_frames=16, window_frames=3, chunk_frames=2, stream_batch=4, kv_fp8=kv_fp8,
                 num_chunks=16, rope_refresh_period=5, embed_dim=16, sink_threshold=0.5, embed_kind="iid",
                 softmax_scale=128 ** -0.5)
    h = _stream(cfg, cfg.num_steps, cache_check=lambda s: s in (8, 12, cfg.num_steps - 1))
    assert len(h.st.refresh_log) >= 4
    assert sum(1 for d, _ in h.decisions.values() if d["replaced"]) >= 1


@pytest.mark.parametrize("kv_fp8,heads", [(False, 255), (True, 510)], ids=["bf16", "e4m3"])
def test_layer_block_at_the_4gib_limit(kv_fp8, heads):
    # 64 slots (S + W + T' = 1 + 62 + 1) of `heads` x 1024 tokens x 128 dims: a layer's K block
    # of 4.28e9 bytes, just under the library's 2^32 limit, so once the ring has filled the tile
    # loop's 32-bit slot offsets pass 2^31, and the refreshes at frames 32 and 64 rebase the
    # whole block.  The first, middle and last heads carry the seeded inputs the oracle sees
    # (a 3-head stream: heads are independent); the others are random on the device.  Every row
    # of those heads at the fill step, after the wrap (the second refresh) and at the end.
    base = configs.WAN13B_1LAYER.with_(sink_frames=1, window_frames=62, num_chunks=70, kv_fp8=kv_fp8)
    big, small = base.with_(num_heads=heads), base.with_(num_heads=3)
    ccfg = sdv2.config_of(big)
    lay = sdv2.sdv2_cache_layout(ccfg)
    block = lay.slots * lay.slot_stride * lay.elem_bytes
    assert lay.slots == 64 and 2 ** 31 + 2 ** 30 < block < 2 ** 32, block
    hsel = [0, heads // 2, heads - 1]
    run = StreamRunner(ccfg, big.num_chunks, big.softmax_scale)
    st = ost.OracleStream(small, layers=[0])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    worst = 0.0
    for s in range(big.num_steps):
        plan = st.begin_step(s)
        q, k, v = inputs.qkv(small, s, 0, 0)

        def qkv(s_, layer, nb):
            out = []
            for x in (q, k, v):
                t = torch.randn((nb, big.chunk_rows, heads, big.head_dim), generator=gen, device="cuda")
                t = (t * (big.q_prescale if x is q else 1.0)).to(torch.bfloat16)
                t[0][:, hsel] = dev(small, x)
                out.append(t)
            return tuple(out)

        info = run.step(s, qkv)
        assert info["refreshed"] == sum(1 for (s_, _) in st.refresh_log if s_ == s)
        if s in (62, 64, big.num_steps - 1):
            log(f"4 GiB block ({'e4m3' if kv_fp8 else 'bf16'}, {heads} heads): step {s}, every row of heads {hsel}")
            ref = st.attend(0, 0, q, k, v)
            worst = max(worst, assert_close(small, host64(run.out[0, 0][:, hsel]), ref, f"out step {s}"))
        st.end_step({0: (k, v)})
    assert [f for (_, f) in st.refresh_log] == [32, 64]
    log(f"4 GiB block: worst max-abs {worst:.3g}")


@pytest.mark.parametrize("seed", random_configs.SEEDS)
def test_random_small_streams(seed, monkeypatch):
    # seeded random configurations across the library's limits (tests/random_configs.py), some
    # with a forced split-KV count: every output of every step, the cache at the end
    cfg = random_configs.random_config(seed)
    nsplit = random_configs.forced_splits(seed)
    if nsplit:
        monkeypatch.setenv("SDV2_NSPLIT", str(nsplit))
    log(f"{cfg.name}: {cfg.dtype}{' e4m3 cache' if cfg.kv_fp8 else ''} d {cfg.head_dim} rope "
        f"{cfg.rope_dim_t}/{cfg.rope_dim_h}/{cfg.rope_dim_w} grid {cfg.grid_h}x{cfg.grid_w} H {cfg.num_heads} "
        f"layers {cfg.num_layers} S {cfg.sink_frames} W {cfg.window_frames} T' {cfg.chunk_frames} "
        f"B {cfg.stream_batch} refresh {cfg.rope_refresh_period} pinned {cfg.rope_pin_sinks} "
        f"tau {cfg.sink_threshold} key scale {cfg.key_scale:.3g} forced splits {nsplit}")
    _stream(cfg, cfg.num_steps, cache_check=lambda s: s == cfg.num_steps - 1)


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
    # the single-layer shape with an e4m3 cache, through the refresh at frame 32; every row and
    # head at the step after it
    cfg = configs.WAN13B_1LAYER.with_(kv_fp8=True)
    checked = {1, 9, 31, 32, 33}
    rows = sample_rows(cfg.tokens, n=48, seed=5)
    h = _stream(cfg, 34, check=lambda s: s in checked, rows=rows, cache_check=lambda s: s in checked,
                all_rows_at={33})
    assert h.st.refresh_log == [(32, 32)]


def test_fp8_kv_wan14b_40layer_b4_full_size():
    cfg = configs.WAN14B_40LAYER_B4.with_(kv_fp8=True, sink_threshold=None, embed_dim=0, embed_kind=None)
    rows = sample_rows(cfg.tokens, n=16, seed=6)
    h = Harness(cfg, layers=(39,))                       # the last layer: largest cache offsets
    for s in range(12):
        full = s in (3, 11)
        h.step(s, full=full)
        if s == 3:
            h.check_outputs(rows=rows, heads=np.arange(0, 40, 3))
        elif full:
            log(f"{cfg.name} e4m3: step {s}, all rows, heads and elements of layer 39")
            h.check_outputs()
        h.finish_step()
        if full:
            h.check_cache()


def test_wan13b_30layer_t2b2_full_size():
    # split-KV with block-causal query tiles: splits of frame-0 rows end before own frame 1;
    # every row, head and element (2 x 2048 x 12) of layers 0 and 29 at the last step
    cfg = configs.WAN13B_30LAYER_T2B2
    checked = {1, 9, 10}
    rows = sample_rows(cfg.chunk_rows, n=32, seed=4)
    _stream(cfg, 11, layers=(0, 29), check=lambda s: s in checked, rows=rows,
            cache_check=lambda s: s in checked, all_rows_at={10})


def test_wan13b_single_layer_full_size():
    # sampled rows through fill, wrap and refresh; every row and head (1024 x 12) at step 33,
    # the first steady step after the refresh
    cfg = configs.WAN13B_1LAYER
    checked = {0, 1, 8, 9, 10, 31, 32, cfg.num_steps - 1}
    rows = sample_rows(cfg.tokens, n=48)
    h = _stream(cfg, cfg.num_steps, check=lambda s: s in checked, rows=rows,
                cache_check=lambda s: s in checked | {33}, all_rows_at={33})
    assert h.st.refresh_log == [(32, 32)]


def test_wan13b_30layer_b4_full_size():
    # sampled rows; every row, head and element (4 x 1024 x 12) of layers 0 and 29 at the last step
    cfg = configs.WAN13B_30LAYER_B4
    checked = {3, 12, 13}
    rows = sample_rows(cfg.tokens, n=24, seed=1)
    _stream(cfg, 14, layers=(0, 29), check=lambda s: s in checked, rows=rows,
            cache_check=lambda s: s in checked, all_rows_at={13})


def test_wan13b_480p_b2_full_size_with_refresh():
    # sampled rows through the refresh; every row, head and element (2 x 1560 x 12) of layers 0
    # and 29 at the first step after it
    cfg = configs.WAN13B_480P_B2
    checked = {2, 10, 24, 25}
    rows = sample_rows(cfg.tokens, n=24, seed=2)
    h = _stream(cfg, 26, layers=(0, 29), check=lambda s: s in checked, rows=rows,
                cache_check=lambda s: s in checked, all_rows_at={25})
    assert h.st.refresh_log == [(24, 24)]
    assert h.stats_checked == 24                # the motion term of commits 1..24 (frame 0 has none)


@pytest.mark.timeout(900)
def test_wan14b_40layer_b4_full_size_with_sink_refresh():
    # layers 0 and 39 (the largest cache offsets); sampled rows and heads at step 12, every row,
    # head and element (4 x 1024 x 40) at the last step
    cfg = configs.WAN14B_40LAYER_B4
    steps = 40
    rows = sample_rows(cfg.tokens, n=16, seed=3)
    h = Harness(cfg, layers=(0, 39))
    replaced = kept = 0
    for s in range(steps):
        full = s in (12, steps - 1)
        h.step(s, full=full)
        if s == 12:
            h.check_outputs(rows=rows, heads=np.arange(0, 40, 3))
        elif full:
            log(f"{cfg.name}: step {s}, all rows, heads and elements of layers 0 and 39")
            h.check_outputs()
        dec = h.finish_step()
        if dec is not None:
            replaced += dec["replaced"]
            kept += not dec["replaced"]
        if full:
            h.check_cache()
    log(f"{cfg.name}: sink decisions replaced {replaced} kept {kept}")
    assert replaced >= 1 and kept >= 1


def test_fused_chunk_stats_over_the_480p_latent_series_and_14b_embeddings():
    # One sdv2_sink_replace per commit reduces the newest 16x60x104 latent frame against the one
    # before it and the 5120-d chunk embedding against the sink (the 14B workload's scene
    # generator, tau 0.95), in one statistics launch.  All 128 commits of the 129-frame series:
    # distances and similarity terms against oracle.motion / oracle.sink at rtol 1e-12, every
    # decision bit-exact (a tiny attention shape keeps the stream cheap).
    c5 = configs.WAN14B_40LAYER_B4
    cfg = _small(cfg_id=c5.cfg_id, num_chunks=128, embed_dim=c5.embed_dim, sink_threshold=c5.sink_threshold,
                 embed_kind=c5.embed_kind, scene_change_prob=c5.scene_change_prob, scene_noise=c5.scene_noise)
    h = Harness(cfg, [0], motion_cfg=configs.WAN13B_480P_B2)
    replaced = kept = 0
    for s in range(cfg.num_steps):
        h.step(s)
        dec = h.finish_step()
        if dec is not None:
            replaced += dec["replaced"]
            kept += not dec["replaced"]
    assert h.stats_checked == 2 * (cfg.num_chunks - 1)
    assert replaced >= 3 and kept >= 3
    log(f"fused stats: {h.stats_checked} checks, replaced {replaced} kept {kept}")


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


def test_motion_l2_long_series():
    """1025 frames of 16x60x104 (the measured series): 32 runs of 32 pairs; 70 frames: a last
    run of 5 pairs; each frame's last part of 1536 elements takes the tail loads.  The scalar
    path (unaligned base, 5001 elements: a part of 905) over 40 frames; one pair, frames of a
    single tail part (100 and 3 elements) and of one element.  Two calls give identical bits
    (fixed reduction order)."""
    cfg = configs.WAN13B_480P_B2
    m = cfg.motion
    frames = inputs.motion_frames(cfg, frames=1025)
    x = torch.from_numpy(frames).cuda()
    for nf in (1025, 70):
        log(f"motion_l2: {nf} frames of {m.elems} elements")
        dist = torch.empty(nf - 1, dtype=torch.float64, device="cuda")
        ws = torch.empty(sdv2.sdv2_motion_workspace_size(nf, m.elems), dtype=torch.uint8, device="cuda")
        sdv2.sdv2_motion_l2(x[:nf], nf, m.elems, dist, ws)
        got = dist.cpu().numpy()
        np.testing.assert_allclose(got, omotion.frame_distances(frames[:nf]), rtol=1e-12, atol=0)
        sdv2.sdv2_motion_l2(x[:nf], nf, m.elems, dist, ws)
        assert np.array_equal(dist.cpu().numpy(), got)
    # degenerate sizes: one pair; one part that is all tail (100 and 3 elements); one element
    for nf, ne, off in ((2, 99840, 0), (5, 100, 0), (4, 3, 1), (3, 1, 0)):
        log(f"motion_l2: {nf} frames of {ne} elements, offset {off}")
        flat = frames.reshape(-1)[off:off + nf * ne].reshape(nf, ne)
        dist = torch.empty(nf - 1, dtype=torch.float64, device="cuda")
        ws = torch.empty(sdv2.sdv2_motion_workspace_size(nf, ne), dtype=torch.uint8, device="cuda")
        sdv2.sdv2_motion_l2(x.view(-1)[off:off + nf * ne], nf, ne, dist, ws)
        np.testing.assert_allclose(dist.cpu().numpy(), omotion.frame_distances(flat), rtol=1e-12, atol=0)
    nf, ne = 40, 5001
    log(f"motion_l2: {nf} frames of {ne} elements, unaligned")
    flat = frames.reshape(-1)[1:1 + nf * ne].reshape(nf, ne)
    dist = torch.empty(nf - 1, dtype=torch.float64, device="cuda")
    ws = torch.empty(sdv2.sdv2_motion_workspace_size(nf, ne), dtype=torch.uint8, device="cuda")
    sdv2.sdv2_motion_l2(x.view(-1)[1:1 + nf * ne], nf, ne, dist, ws)
    np.testing.assert_allclose(dist.cpu().numpy(), omotion.frame_distances(flat), rtol=1e-12, atol=0)


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
