"""Pins of the oracle's stream bookkeeping: schedule, ring model, RoPE refresh."""
import numpy as np
import pytest

import brute
from oracle import rope
from oracle import stream as ost
from oracle.attention import attention
from synth import inputs
from synth.configs import TINY_FP32, WAN13B_1LAYER, WAN13B_480P_B2


def tiny(**kw):
    base = dict(rope_refresh_period=0, sink_threshold=None, embed_dim=0, embed_kind=None)
    base.update(kw)
    return TINY_FP32.with_(**base)


def test_schedule_fill_steady_drain():
    # B = 4, M = 6: the pipeline fills for B-1 steps (nothing finishes), then one chunk
    # finishes per step; after the last chunk enters, B-1 drain steps finish the rest.
    cfg = tiny(stream_batch=4, num_chunks=6)
    got = [ost.schedule(cfg, s) for s in range(cfg.num_steps)]
    assert cfg.num_steps == 9
    assert [g["chunks"] for g in got] == [[0], [0, 1], [0, 1, 2], [0, 1, 2, 3], [1, 2, 3, 4],
                                          [2, 3, 4, 5], [3, 4, 5], [4, 5], [5]]
    assert [g["commit"] for g in got] == [None, None, None, 0, 1, 2, 3, 4, 5]
    assert [g["newest_frame"] for g in got] == [0, 1, 2, 3, 4, 5, 5, 5, 5]
    cfg2 = tiny(stream_batch=2, num_chunks=3, chunk_frames=2)
    assert [ost.schedule(cfg2, s)["newest_frame"] for s in range(4)] == [1, 3, 5, 5]


@pytest.mark.parametrize("S,W,T", [(1, 8, 1), (2, 6, 1), (1, 4, 1), (0, 3, 1), (3, 1, 1),
                                   (1, 8, 2), (2, 3, 3), (0, 2, 4), (3, 1, 2), (1, 5, 8)])
def test_ring_slots_hold_exactly_the_window(S, W, T):
    # Stream chunks of T frames through the oracle's chronological window (the last W committed
    # non-sink frames) and place every frame in a ring by ring_slot():
    #  - sinks keep slots [0, S); every other frame lands in [S, S + W + T);
    #  - after every commit the ring slots of the window frames are distinct and the slot of
    #    each window frame still holds it (nothing later overwrote it);
    #  - the T slots the next chunk is written to hold no window frame, so appending that chunk
    #    in place leaves every frame it attends intact.
    cfg = tiny(sink_frames=S, window_frames=W, chunk_frames=T, num_chunks=6 * (W + T) + S + 3)
    st = ost.OracleStream(cfg, layers=[])
    ring = {}
    for s_ in range(cfg.num_chunks):
        st.begin_step(s_)
        c = st.plan["chunks"][0]
        window = [e.frame for e in st.window]
        nxt = [ost.ring_slot(cfg, c * T + t) for t in range(T)]
        # the chunk's own slots do not hold a frame the chunk attends
        assert not set(nxt) & {ost.ring_slot(cfg, f) for f in window}
        for t, slot in enumerate(nxt):
            f = c * T + t
            assert slot == f if f < S else S <= slot < S + W + T
            ring[slot] = f                        # the append writes the frame to its final slot
        st.end_step({}, None)
        window = [e.frame for e in st.window]
        slots = [ost.ring_slot(cfg, f) for f in window]
        assert len(set(slots)) == len(slots)
        assert all(ring[ost.ring_slot(cfg, f)] == f for f in window)
        assert [ring[j] for j in range(S) if j in ring] == [e.frame for e in st.sinks if e is not None]


def test_ring_order_attention_equals_chronological():
    # after wraparound, attention over the keys in ring-slot order equals chronological order
    cfg = tiny(sink_frames=1, window_frames=4, num_chunks=12)
    st, outs = brute.run_oracle(cfg, steps=11)
    st.begin_step(11)
    q, k, v = inputs.qkv(cfg, 11, 0, 0)
    want = st.attend(0, 0, q, k, v)
    entries = sorted(st.cached_entries(), key=lambda e: ost.ring_slot(cfg, e.frame))
    assert [e.frame for e in st.window] == [7, 8, 9, 10]
    # a ring of W + T' = 5 slots after the sink: frame f in slot 1 + f mod 5; slot 2 is the
    # one the chunk of frame 11 is written to
    assert [ost.ring_slot(cfg, e.frame) for e in entries] == [0, 1, 3, 4, 5]
    assert [e.frame for e in entries] == [0, 10, 7, 8, 9]
    assert ost.ring_slot(cfg, 11) == 2
    ks = [rope.rope_frame(cfg, e.kv[0][0], e.label) for e in entries]
    vs = [e.kv[0][1] for e in entries]
    ks.append(rope.rope_frame(cfg, brute.to_f64(cfg, k), 11))
    vs.append(brute.to_f64(cfg, v))
    qr = rope.rope_frame(cfg, brute.to_f64(cfg, q), 11)
    K, V = np.concatenate(ks), np.concatenate(vs)
    for h in range(cfg.num_heads):
        o, _ = attention(qr[:, h], K[:, h], V[:, h], cfg.softmax_scale)
        np.testing.assert_allclose(o, want[:, h], atol=1e-12)


@pytest.mark.parametrize("period,B,M,expect", [
    (8, 1, 12, [(8, 8)]),                                   # tiny fp32 workload: frame index 8
    (32, 1, 64, [(32, 32)]),                                # Wan-1.3B single layer: every 32
    (24, 2, 128, [(24, 24), (48, 48), (72, 72), (96, 96), (120, 120)]),   # 480p, B = 2
    (4, 3, 10, [(4, 4), (8, 8)]),
])
def test_refresh_events(period, B, M, expect):
    cfg = tiny(rope_refresh_period=period, stream_batch=B, num_chunks=M)
    st = ost.OracleStream(cfg, layers=[])
    for s in range(cfg.num_steps):
        st.begin_step(s)
        st.end_step({}, None)                               # no layers tracked: labels only
    assert st.refresh_log == expect


def test_refresh_makes_new_frame_position_zero_and_shifts_labels():
    cfg = tiny(rope_refresh_period=8, num_chunks=12)
    st, _ = brute.run_oracle(cfg, steps=8)
    before = {e.frame: e.label for e in st.cached_entries()}
    assert before == {0: 0, 4: 4, 5: 5, 6: 6, 7: 7}
    st.begin_step(8)
    after = {e.frame: e.label for e in st.cached_entries()}
    assert st.base == 8
    assert after == {f: p - 8 for f, p in before.items()}


@pytest.mark.parametrize("B,period", [(1, 3), (2, 4), (3, 5)])
def test_refresh_leaves_outputs_unchanged(B, period):
    # rebasing every cached label and the query by the same constant leaves every score, hence
    # every output, unchanged: the same stream with and without refresh must agree.
    cfg = tiny(stream_batch=B, num_chunks=13)
    _, plain = brute.run_oracle(cfg)
    st, refreshed = brute.run_oracle(cfg.with_(rope_refresh_period=period))
    assert len(st.refresh_log) >= 2
    for key in plain:
        np.testing.assert_allclose(refreshed[key], plain[key], atol=1e-12)


def test_commit_labels_and_window_contents_over_a_stream():
    cfg = tiny(sink_frames=2, window_frames=3, stream_batch=2, num_chunks=9, rope_refresh_period=4)
    st = ost.OracleStream(cfg, layers=[0])
    for s in range(cfg.num_steps):
        plan = st.begin_step(s)
        _, k, v = inputs.qkv(cfg, s, 0, 0)
        st.end_step({0: (k, v)})
        c0 = plan["commit"]
        if c0 is not None:
            committed = list(range(c0 + 1))
            assert [e.frame for e in st.sinks if e] == committed[:2]
            assert [e.frame for e in st.window] == [f for f in committed if f >= 2][-3:]
            for e in st.cached_entries():
                assert e.label == e.frame - st.base


@pytest.mark.parametrize("S,B,T,period", [(1, 1, 1, 3), (2, 2, 1, 4), (2, 2, 2, 3), (1, 3, 1, 2)])
def test_pinned_sinks_match_history(S, B, T, period):
    # alternative refresh reading: the sinks keep their labels across refreshes.  Outputs must
    # equal the history brute force with each sink placed at f - b0(commit step) + b0(step).
    cfg = tiny(sink_frames=S, window_frames=3, stream_batch=B, chunk_frames=T, num_chunks=10,
               rope_refresh_period=period, rope_pin_sinks=True)
    st, outs = brute.run_oracle(cfg)
    assert len(st.refresh_log) >= 2
    for e in st.sinks:                            # the label at commit, never moved since
        assert e.label == e.frame - brute.refresh_base(cfg, e.frame // T + B - 1)
    for s in range(cfg.num_steps):
        for b in range(len(ost.schedule(cfg, s)["chunks"])):
            np.testing.assert_allclose(outs[(s, 0, b)], brute.history_output(cfg, s, b, 0, pinned_sinks=True),
                                       atol=1e-12)


def test_pinned_sinks_equal_rebased_sinks_without_refresh():
    cfg = tiny(sink_frames=2, window_frames=3, stream_batch=2, num_chunks=8)
    _, a = brute.run_oracle(cfg)
    _, b = brute.run_oracle(cfg.with_(rope_pin_sinks=True))
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_pinned_and_rebased_sinks_part_at_the_first_refresh():
    # the two readings agree until the first refresh (step 3: frame 3 reaches T_reset = 3) and
    # differ afterwards, when the pinned sinks sit closer to the query
    cfg = tiny(sink_frames=1, window_frames=3, num_chunks=10, rope_refresh_period=3)
    _, a = brute.run_oracle(cfg)
    _, b = brute.run_oracle(cfg.with_(rope_pin_sinks=True))
    differ = sorted(k[0] for k in a if not np.allclose(a[k], b[k], atol=1e-9))
    assert differ and differ[0] == 3


def test_round_bf16_pins():
    # exact values stay; ties (half a bf16 quantum, 2^-8 at 1.0) go to the even neighbour;
    # anything above a tie goes up; the float32 step keeps the sign and handles tiny values
    from oracle.stream import round_bf16
    q = 2.0 ** -7                                     # bf16 quantum in [1, 2)
    x = np.array([1.0, 1.0 + q, 1.0 + q / 2, 1.0 + 3 * q / 2, 1.0 + q / 2 + 2.0 ** -20,
                  -3.0 - q / 2, 2.0 ** -130, 65280.0 + 128.0])
    want = np.array([1.0, 1.0 + q, 1.0, 1.0 + 2 * q, 1.0 + q, -3.0, 2.0 ** -130, 65536.0])
    np.testing.assert_array_equal(round_bf16(x), want)


def test_bf16_storage_mode_with_a_key_scale():
    # rotated="bf16" with key_scale rounds the keys after a product by the fp32 value of
    # key_scale * log2(e) and divides it out again.  With key_scale = 4 / log2(e) that product is
    # exactly 4 in fp32, and rounding commutes with a power of two: the outputs equal those of the
    # unscaled storage mode bit for bit.  With 1/sqrt(128) the keys round at other values: the
    # outputs differ from the unscaled mode, by no more than the bf16 rounding of the keys moves
    # them (both stay within that of the exact outputs).
    cfg = tiny(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, num_heads=2,
               stream_batch=2, num_chunks=8, softmax_scale=128 ** -0.5)
    st = ost.OracleStream(cfg, layers=[0])
    assert float(np.float32(4.0 / np.log2(np.e) * np.log2(np.e))) == 4.0
    checked = 0
    for s in range(cfg.num_steps):
        plan = st.begin_step(s)
        kv0 = {}
        for b in range(len(plan["chunks"])):
            q, k, v = inputs.qkv(cfg, s, 0, b)
            exact = st.attend(0, b, q, k, v)
            plain = st.attend(0, b, q, k, v, rotated="bf16")
            four = st.attend(0, b, q, k, v, rotated="bf16", key_scale=4.0 / np.log2(np.e))
            scaled = st.attend(0, b, q, k, v, rotated="bf16", key_scale=128 ** -0.5)
            np.testing.assert_array_equal(four, plain)
            if s >= 4:
                assert not np.array_equal(scaled, plain)
                checked += 1
            for out in (plain, scaled):
                assert np.abs(out - exact).max() <= 2e-2
            if b == 0:
                kv0[0] = (k, v)
        st.end_step(kv0, None)
    assert checked >= 4
