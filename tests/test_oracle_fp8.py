"""Pins of the OCP E4M3 encoding: values fixed by the format's definition."""
import numpy as np

from oracle import fp8


def test_known_codes():
    assert fp8.decode_code(0x38) == 1.0                 # exponent 7 = bias, mantissa 0
    assert fp8.decode_code(0x7E) == 448.0               # largest finite: 2^8 * 1.75
    assert np.isnan(fp8.decode_code(0x7F)) and np.isnan(fp8.decode_code(0xFF))
    assert fp8.decode_code(0x01) == 2.0 ** -9           # smallest subnormal: 2^-6 / 8
    assert fp8.decode_code(0x08) == 2.0 ** -6           # smallest normal
    assert fp8.decode_code(0xC0) == -2.0
    assert fp8.decode_code(0x80) == 0.0 and np.signbit(fp8.decode_code(0x80))


def test_every_finite_value_round_trips_and_is_a_bf16():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = fp8.decode(codes)
    assert np.array_equal(fp8.encode(vals), codes)
    # 3 mantissa bits and exponents 2^-9 .. 2^8 fit bf16 (7 bits, 8-bit exponent) exactly
    f32 = vals.astype(np.float32)
    assert np.array_equal(f32.view(np.uint32) & 0xFFFF, np.zeros(len(codes), np.uint32))


def test_round_to_nearest_even_and_saturation():
    # 1 + 1/16 lies halfway between 1 (0x38, even) and 1.125 (0x39): to the even code
    assert fp8.encode([1.0625])[0] == 0x38
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even)
    assert fp8.encode([1.1875])[0] == 0x3A
    assert fp8.encode([1.07])[0] == 0x39                # just above the midpoint
    assert fp8.encode([2.0 ** -10])[0] == 0x00          # half the smallest subnormal: tie to 0
    assert fp8.encode([3 * 2.0 ** -11])[0] == 0x01      # above it: the subnormal
    assert list(fp8.encode([448.0, 460.0, 1e6, -1e9])) == [0x7E, 0x7E, 0x7E, 0xFE]
    assert fp8.encode([-0.0])[0] == 0x80


def test_relative_error_bound():
    x = np.random.default_rng(0).standard_normal(100000) * 4
    big = np.abs(x) >= 2.0 ** -6                        # normal range: half an ulp = 2^-4 relative
    r = fp8.round_fp8(x)
    assert np.all(np.abs(r[big] - x[big]) <= np.abs(x[big]) * 2.0 ** -4 * (1 + 1e-12))


# ---- the FP8 cache mode of the oracle stream -------------------------------------------------

import pytest

import brute
from oracle import rope
from synth.configs import TINY_FP32


def _fp8_cfg(**kw):
    base = dict(dtype="bf16", kv_fp8=True, sink_threshold=None, embed_dim=0, embed_kind=None,
                sink_frames=1, window_frames=3, rope_refresh_period=3, num_chunks=10)
    base.update(kw)
    return TINY_FP32.with_(**base)


def _fp8_scaled_cfg(**kw):
    # head_dim 128 with the softmax scale as key scale: keys stored times the factor g
    base = dict(head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, softmax_scale=128 ** -0.5)
    base.update(kw)
    cfg = _fp8_cfg(**base)
    assert cfg.key_scale == cfg.softmax_scale
    return cfg


def test_key_factor_has_its_documented_form():
    # g = key_scale * log2(e) * 2^k with k = -floor(log2(key_scale * log2(e)) + 1/2): g in
    # [2^-1/2, 2^1/2] and key_scale * log2(e) / g a power of two; 4 / log2(e) gives g = 1 and
    # no key scale gives 1
    from oracle.stream import fp8_key_factor
    assert fp8_key_factor(0.0) == 1.0
    assert fp8_key_factor(4.0 / np.log2(np.e)) == 1.0
    for ks in (128 ** -0.5, 64 ** -0.5, 1.0, 0.3, 5.0, 1e-3):
        g = fp8_key_factor(ks)
        c = ks * np.log2(np.e)
        assert 2 ** -0.5 <= g <= 2 ** 0.5, (ks, g)
        e = np.log2(c / g)
        assert abs(e - np.round(e)) < 1e-6, (ks, g)           # a power of two up to fp32 rounding of g
        assert g == brute.e4m3_key_factor(TINY_FP32.with_(dtype="bf16", head_dim=128, rope_dim_t=44,
                                                           rope_dim_h=42, rope_dim_w=42, softmax_scale=ks))


def test_brute_rounding_agrees_with_the_table_encoder():
    # two routes to e4m3 rounding (binade quantum vs nearest-table search) on values that
    # include every midpoint, both signs, subnormals and saturation
    vals = fp8.decode(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8))
    pos = np.sort(vals[vals > 0])
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([vals, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), [460., 500., -1e6],
                        np.random.default_rng(1).standard_normal(20000) * 8])
    np.testing.assert_array_equal(brute.round_e4m3(x), fp8.round_fp8(x))


@pytest.mark.parametrize("T,B,period,scaled", [(1, 1, 3, False), (1, 2, 3, False), (2, 2, 4, False),
                                               (1, 3, 0, False), (1, 2, 3, True), (2, 2, 4, True),
                                               (3, 2, 2, False), (3, 1, 2, True)])
def test_fp8_stream_equals_history_fold(T, B, period, scaled):
    # every output at every step equals attention over keys rebuilt from the frame history:
    # commit-time rounding, then one turn-back and rounding for each later step whose base
    # moved, by that step's move (T' > T_reset: some steps pass two periods at once), all
    # relative to b0(s) (scaled: each key times the key factor before its roundings, divided
    # out when attending)
    cfg = (_fp8_scaled_cfg if scaled else _fp8_cfg)(chunk_frames=T, stream_batch=B, rope_refresh_period=period)
    st, outs = brute.run_oracle(cfg)
    assert (len(st.refresh_log) > 2) == (period > 0)
    for s in range(cfg.num_steps):
        for b in range(len(ost_schedule(cfg, s)["chunks"])):
            np.testing.assert_allclose(outs[(s, 0, b)], brute.history_output(cfg, s, b, 0, fp8=True),
                                       atol=1e-12, err_msg=f"step {s} elem {b}")


def ost_schedule(cfg, s):
    from oracle import stream as ost
    return ost.schedule(cfg, s)


@pytest.mark.parametrize("scaled", [False, True])
def test_fp8_cached_keys_are_e4m3_and_near_the_exact_rotation(scaled):
    # stored keys and values are e4m3 values; each key pair is within the rounding errors of
    # its commit and of each refresh since of the exact rotation at the current label (scaled:
    # of the exact rotation times the key factor g)
    cfg = (_fp8_scaled_cfg if scaled else _fp8_cfg)(window_frames=4, rope_refresh_period=2, num_chunks=12)
    g = brute.e4m3_key_factor(cfg)
    assert (g != 1.0) == scaled
    st, _ = brute.run_oracle(cfg)
    r = len(st.refresh_log)
    assert r >= 4
    for e in st.cached_entries():
        K, V = e.kv[0]
        assert np.array_equal(fp8.round_fp8(K), K) and np.array_equal(fp8.round_fp8(V), V)
        k_raw, v_raw = brute.committed_frame_kv(cfg, e.frame, 0)
        np.testing.assert_array_equal(V, fp8.round_fp8(v_raw))
        exact = g * brute.frame_rope(cfg, k_raw, e.label)
        err = np.hypot(K[..., 0::2] - exact[..., 0::2], K[..., 1::2] - exact[..., 1::2])
        norm = np.hypot(exact[..., 0::2], exact[..., 1::2])
        assert np.all(err <= (r + 1) * (2.0 ** -4 * 1.1 * norm + 2.0 ** -9)), e.frame


def test_fp8_outputs_stay_near_the_exact_stream():
    # the e4m3 cache perturbs outputs but only at the level its rounding allows
    cfg = _fp8_cfg()
    _, a = brute.run_oracle(cfg)
    _, b = brute.run_oracle(cfg.with_(kv_fp8=False))
    d = np.array([np.abs(a[k] - b[k]).max() for k in a])
    assert 0 < d.max() <= 0.1
