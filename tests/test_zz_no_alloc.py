"""sdv2_chunk_attention_static (no allocation, static device scratch) against
sdv2_chunk_attention (create-time workspace): same kernels and split count, so the outputs must
be bitwise equal.  Two calls in a row, the second on a smaller input; the size limit; and
replays of the call from a captured HIP graph."""
import numpy as np
import pytest
import torch

from gpu_helpers import log
from rolling_kv_causal_amd import sdv2
from rolling_kv_causal_amd.stream import StreamRunner
from synth import configs

pytestmark = pytest.mark.gpu


def _steady(cfg, steps, seed):
    """A stream of cfg run for `steps` steps (device-side random inputs), then one more step
    opened and appended on every layer; returns the runner and that step's rotated q."""
    run = StreamRunner(sdv2.config_of(cfg), 1 << 20, cfg.softmax_scale)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    shape = (cfg.stream_batch, cfg.chunk_rows, cfg.num_heads, cfg.head_dim)

    def qkv(s, layer, nb):
        return tuple(torch.randn(shape, generator=g, device="cuda").to(run.dtype)[:nb] for _ in range(3))

    for s in range(steps):
        run.step(s, qkv)
    first, nb, commit, newest = run.plan(steps)
    run.cache.refresh(newest)
    qs = []
    for layer in range(cfg.num_layers):
        q, k, v = qkv(steps, layer, nb)
        run.cache.append(layer, first, nb, q, k, v)
        qs.append(q)
    return run, nb, qs


def _compare(cfg, steps, seed):
    run, nb, qs = _steady(cfg, steps, seed)
    for layer, q in enumerate(qs):
        ref = torch.empty_like(q)
        got = torch.full_like(q, float("nan"))
        sdv2.sdv2_chunk_attention(run.cache.handle, layer, nb, q, ref, cfg.softmax_scale)
        sdv2.sdv2_chunk_attention_static(run.cache.handle, layer, nb, q, got, cfg.softmax_scale)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{cfg.name} layer {layer}: static-scratch output differs"
    run.cache.close()
    return nb


def test_static_scratch_matches_workspace_then_a_smaller_call(monkeypatch):
    # 1.3B single layer: five splits (16 MB of partials), then a smaller ragged stream (65
    # tokens, B = 3, four splits forced) on the same GPU's array
    big = configs.WAN13B_1LAYER
    kv, meta, ws = sdv2.sdv2_cache_size(sdv2.config_of(big))
    assert ws > 0, "the workload must use split-KV partials"
    log(f"no-alloc: {big.name} workspace {ws} bytes")
    _compare(big, 12, 1)
    small = configs.TINY_FP32.with_(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
                                    grid_h=5, grid_w=13, num_heads=3, sink_frames=2, window_frames=3,
                                    stream_batch=3, rope_refresh_period=0, sink_threshold=None, embed_dim=0,
                                    embed_kind=None, softmax_scale=128 ** -0.5, name="small_b3")
    monkeypatch.setenv("SDV2_NSPLIT", "4")
    assert 0 < sdv2.sdv2_cache_size(sdv2.config_of(small))[2] < ws
    _compare(small, 8, 2)


def test_static_scratch_refuses_partials_beyond_its_size(monkeypatch):
    # sixteen forced splits of the 14B shape (one layer, B = 4) need 692 MB of partials: the
    # static entry point returns ENOSPC and launches nothing; the workspace entry point runs
    monkeypatch.setenv("SDV2_NSPLIT", "16")
    cfg = configs.WAN14B_40LAYER_B4.with_(num_layers=1, sink_threshold=None, embed_dim=0, embed_kind=None)
    run, nb, qs = _steady(cfg, 6, 3)
    out = torch.zeros_like(qs[0])
    with pytest.raises(sdv2.SDV2Error) as e:
        sdv2.sdv2_chunk_attention_static(run.cache.handle, 0, nb, qs[0], out, cfg.softmax_scale)
    assert e.value.code == sdv2.SDV2_ENOSPC and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    sdv2.sdv2_chunk_attention(run.cache.handle, 0, nb, qs[0], out, cfg.softmax_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.count_nonzero(out) > 0
    run.cache.close()


def test_static_entry_point_replays_from_a_hip_graph(monkeypatch):
    # The callers the entry point is for: one chunk-attention call (split-KV: attention and
    # combine launches, partials in the static array) captured into a HIP graph and replayed.
    # Before each replay the output is set to NaN and an eager call of its own runs on the same
    # array, with the program synchronising in between; every replay equals the eager result
    # of the workspace entry point bit for bit.
    cfg = configs.TINY_FP32.with_(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
                                  grid_h=5, grid_w=13, num_heads=3, sink_frames=2, window_frames=3,
                                  stream_batch=3, rope_refresh_period=0, sink_threshold=None, embed_dim=0,
                                  embed_kind=None, softmax_scale=128 ** -0.5, name="graph_b3")
    monkeypatch.setenv("SDV2_NSPLIT", "4")                        # four splits forced
    assert sdv2.sdv2_cache_size(sdv2.config_of(cfg))[2] > 0, "the call must use split-KV partials"
    run, nb, qs = _steady(cfg, 8, 4)
    q, h, scale = qs[0], run.cache.handle, cfg.softmax_scale
    ref = torch.empty_like(q)
    sdv2.sdv2_chunk_attention(h, 0, nb, q, ref, scale)
    first = torch.empty_like(q)
    sdv2.sdv2_chunk_attention_static(h, 0, nb, q, first, scale)     # set-up outside the capture
    torch.cuda.synchronize()
    assert torch.equal(first, ref)
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sdv2.sdv2_chunk_attention_static(h, 0, nb, q, out, scale)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        other = torch.full_like(q, float("nan"))
        sdv2.sdv2_chunk_attention_static(h, 0, nb, q, other, scale)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(other, ref), f"eager call before replay {i}"
        assert torch.equal(out, ref), f"replay {i}"
    log(f"graph replays of {cfg.name}: 4 equal to the eager result")
    del g
    run.cache.close()
