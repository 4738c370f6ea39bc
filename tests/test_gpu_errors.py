"""Error paths through the C ABI on the GPU.

Out-of-protocol calls return SDV2_ESTATE and change neither the RoPE base, the committed count
nor any slot; a HIP failure at an entry point's first launch (injected with
sdv2_debug_fail_hip_call) returns SDV2_EHIP, launches nothing and leaves the bookkeeping as it
was, so the call can simply be made again and the stream still matches the oracle.
"""
import collections

import numpy as np
import pytest
import torch

from gpu_helpers import Harness, log
from rolling_kv_causal_amd import sdv2
from rolling_kv_causal_amd.stream import StreamRunner
from synth import configs, inputs

pytestmark = pytest.mark.gpu


def snapshot(cache):
    return cache.state(), tuple(cache.slot_info(s) for s in range(cache.layout.slots))


def expect(code, fn, *a, **k):
    with pytest.raises(sdv2.SDV2Error) as e:
        fn(*a, **k)
    assert e.value.code == code, str(e.value)
    return str(e.value)


def test_out_of_protocol_calls_change_nothing():
    cfg = configs.TINY_FP32.with_(num_layers=2)
    run = StreamRunner(sdv2.config_of(cfg), cfg.num_chunks, cfg.softmax_scale)
    c = run.cache
    shape = (1, cfg.chunk_rows, cfg.num_heads, cfg.head_dim)
    q, k, v = (torch.randn(shape, device="cuda") for _ in range(3))
    out = torch.empty_like(q)
    emb = torch.from_numpy(inputs.chunk_embedding(cfg, 0)).cuda()
    ES = sdv2.SDV2_ESTATE

    def no_change(fn, *a, code=ES):
        before = snapshot(c)
        msg = expect(code, fn, *a)
        assert snapshot(c) == before, msg
        return msg

    # nothing before the step opens
    no_change(c.append, 0, 0, 1, q, k, v)
    no_change(c.attention, 0, 1, q, out, cfg.softmax_scale)
    no_change(c.commit, 0)
    no_change(c.sink_replace, 0, emb)
    c.refresh(0)
    no_change(c.attention, 0, 1, q, out, cfg.softmax_scale)         # layer 0 not appended
    no_change(c.commit, 0)                                           # no layer appended
    no_change(c.append, 0, 1, 1, q, k, v)                            # first chunk must be 0
    c.append(0, 0, 1, q, k, v)
    no_change(c.append, 0, 0, 1, q, k, v)                            # layer 0 twice
    no_change(c.commit, 0)                                           # layer 1 not appended
    c.append(1, 0, 1, q, k, v)
    c.attention(0, 1, q, out, cfg.softmax_scale)
    no_change(c.commit, 1)                                           # only element 0's chunk
    no_change(c.sink_replace, 0, emb)                                # before the commit
    c.commit(0)
    no_change(c.commit, 0)                                           # twice in one step
    no_change(c.append, 0, 1, 1, q, k, v)                            # after the commit
    no_change(c.sink_replace, 5, emb)                                # not the committed frame
    c.sink_replace(0, emb)
    no_change(c.refresh, 0)                                          # frame 0 is committed
    no_change(c.refresh, -1, code=sdv2.SDV2_EINVAL)
    c.refresh(1)
    no_change(c.refresh, 0)                                          # newest frame went back
    assert c.state() == (0, 1, 0)
    assert c.slot_info(0) == (0, 0)                                  # frame 0 is the sink


def test_scaled_key_cache_refuses_another_scale():
    # a cache created with a key scale holds its keys times it: an attention call with any other
    # scale returns SDV2_EINVAL, launches nothing and changes nothing; the matching call runs
    cfg = configs.TINY_FP32.with_(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
                                  rope_refresh_period=0, sink_threshold=None, embed_dim=0, embed_kind=None,
                                  softmax_scale=128 ** -0.5)
    assert cfg.key_scale == cfg.softmax_scale
    run = StreamRunner(sdv2.config_of(cfg), cfg.num_chunks, cfg.softmax_scale)
    c = run.cache
    shape = (1, cfg.chunk_rows, cfg.num_heads, cfg.head_dim)
    q, k, v = (torch.randn(shape, device="cuda").to(torch.bfloat16) for _ in range(3))
    out = torch.zeros_like(q)
    c.refresh(0)
    c.append(0, 0, 1, q, k, v)
    before = snapshot(c)
    msg = expect(sdv2.SDV2_EINVAL, c.attention, 0, 1, q, out, 2 * cfg.softmax_scale)
    assert "key_scale" in msg and snapshot(c) == before
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    c.attention(0, 1, q, out, cfg.softmax_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.count_nonzero(out) > 0
    run.cache.close()


def test_create_fails_cleanly_on_an_injected_hip_error():
    cfg = sdv2.config_of(configs.TINY_FP32)
    kv, meta, ws = sdv2.sdv2_cache_size(cfg)
    bufs = [torch.empty(max(n, 256), dtype=torch.uint8, device="cuda") for n in (kv, meta, ws)]
    sdv2.sdv2_debug_fail_hip_call(0)
    try:
        msg = expect(sdv2.SDV2_EHIP, sdv2.sdv2_cache_create, cfg, *bufs)
    finally:
        sdv2.sdv2_debug_fail_hip_call(-1)
    assert "injected" in msg
    h = sdv2.sdv2_cache_create(cfg, *bufs)
    sdv2.sdv2_cache_destroy(h)


class FailFirst:
    """Proxy of a Cache: every refresh, append, attention and sink_replace is first made with
    its first HIP call failing; the call must return SDV2_EHIP with the bookkeeping unchanged,
    and is then made again."""

    def __init__(self, cache):
        self._c = cache
        self.fired = collections.Counter()

    def __getattr__(self, name):
        f = getattr(self._c, name)
        if name not in ("refresh", "append", "attention", "commit", "sink_replace"):
            return f

        def wrapped(*a, **k):
            before = snapshot(self._c)
            sdv2.sdv2_debug_fail_hip_call(0)
            try:
                r = f(*a, **k)
                failed = None
            except sdv2.SDV2Error as e:
                failed = e
            finally:
                sdv2.sdv2_debug_fail_hip_call(-1)
            if failed is None:                 # the call made no HIP call (commit; refresh not due)
                return r
            assert failed.code == sdv2.SDV2_EHIP and "injected" in str(failed), str(failed)
            assert snapshot(self._c) == before, name
            self.fired[name] += 1
            return f(*a, **k)
        return wrapped


def test_injected_hip_failures_leave_the_stream_intact(monkeypatch):
    # bf16, two layers, refresh every 3 frames, sink refresh with i.i.d. embeddings, B = 2 and
    # split-KV (three splits forced: attention and combine launches): every entry point that
    # launches fails once per call, then succeeds; outputs, cache, decisions and statistics
    # still match the oracle at every step
    monkeypatch.setenv("SDV2_NSPLIT", "3")
    cfg = configs.TINY_FP32.with_(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
                                  grid_h=5, grid_w=13, num_heads=2, num_layers=2, sink_frames=1,
                                  window_frames=2, stream_batch=2, rope_refresh_period=3, num_chunks=8,
                                  embed_dim=16, sink_threshold=0.2, embed_kind="iid",
                                  softmax_scale=128 ** -0.5)
    assert sdv2.sdv2_cache_size(sdv2.config_of(cfg))[2] > 0      # the forced splits are in effect
    h = Harness(cfg, range(cfg.num_layers))
    proxy = FailFirst(h.run.cache)
    h.run.cache = proxy
    for s in range(cfg.num_steps):
        h.step(s, full=True)
        h.check_outputs()
        h.finish_step()
        h.check_cache()
    log(f"injected failures: {dict(proxy.fired)}")
    assert proxy.fired["append"] == cfg.num_layers * cfg.num_steps
    assert proxy.fired["attention"] == cfg.num_layers * cfg.num_steps
    assert proxy.fired["refresh"] >= 2 and proxy.fired["sink_replace"] == cfg.num_chunks
    assert proxy.fired["commit"] == 0
