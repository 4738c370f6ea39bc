"""Pins of the oracle's sink refresh (oracle/sink.py and the stream's use of it)."""
import json
import math
import pathlib

import numpy as np
import pytest

import brute
from oracle import sink
from oracle import stream as ost
from synth.configs import TINY_FP32

GOLDEN = json.loads((pathlib.Path(__file__).parent / "golden" / "sink_script.json").read_text())


@pytest.mark.parametrize("phi,replace", [(0.4, False), (0.45, False), (0.46, True), (0.5, True)])
def test_constructed_angle_either_side_of_threshold(phi, replace):
    # e = (1, 0, ...), h = (cos phi, sin phi, 0, ...) -> similarity cos phi; tau = 0.9 sits
    # between cos 0.45 = 0.9004 and cos 0.46 = 0.8961.
    e = np.zeros(64, np.float32)
    e[0] = 1
    h = np.zeros(64, np.float32)
    h[0], h[1] = math.cos(phi), math.sin(phi)
    j, alpha, rep = sink.decide(h, [e], 0.9)
    assert j == 0 and rep is replace
    assert alpha == pytest.approx(math.cos(phi), abs=1e-7)


def test_least_similar_sink_is_chosen():
    e0, e1, e2 = np.eye(3)
    h = np.array([math.cos(0.5), math.sin(0.5), 0.0])
    j, alpha, rep = sink.decide(h, [e0, e1, e2], 0.9)
    assert j == 2 and alpha == 0.0 and rep                   # orthogonal to e2
    j, alpha, _ = sink.decide(h, [e0, e1], 0.9)
    assert j == 1 and alpha == pytest.approx(math.sin(0.5), abs=1e-15)


def test_ties_zero_norm_and_strictness():
    e = np.array([1.0, 0.0, 0.0, 0.0])
    assert sink.decide(e, [e, e, e], 0.5) == (0, 1.0, False)
    assert sink.cosine(np.zeros(4), e) == 0.0
    c = GOLDEN["strict_threshold_case"]
    j, alpha, rep = sink.decide(np.array(c["embedding"], float), [np.array(c["sink"], float)], c["tau"])
    assert alpha == c["alpha"] and rep is c["replaced"]


def _script_cfg():
    return TINY_FP32.with_(sink_frames=GOLDEN["sink_frames"], window_frames=GOLDEN["window_frames"],
                           sink_threshold=GOLDEN["tau"], embed_dim=4, rope_refresh_period=0,
                           num_chunks=len(GOLDEN["embeddings"]))


def test_scripted_sequence_matches_hand_derivation():
    cfg = _script_cfg()
    emb = [np.array(e, np.float32) for e in GOLDEN["embeddings"]]
    st = ost.OracleStream(cfg, layers=[0])
    from synth import inputs
    for s in range(cfg.num_steps):
        plan = st.begin_step(s)
        _, k, v = inputs.qkv(cfg, s, 0, 0)
        st.end_step({0: (k, v)}, emb[plan["commit"]])
        want = GOLDEN["sink_frames_after_chunk"][plan["commit"]]
        assert [None if e is None else e.frame for e in st.sinks] == want
    got = [{"chunk": d["chunk"], "slot": d["slot"], "replaced": d["replaced"]} for d in st.sink_log]
    want = [{"chunk": d["chunk"], "slot": d["slot"], "replaced": d["replaced"]} for d in GOLDEN["decisions"]]
    assert got == want
    for d, g in zip(st.sink_log, GOLDEN["decisions"]):
        assert d["alpha"] == pytest.approx(g["alpha"], abs=1e-7)


def test_replaced_sink_carries_the_frame_into_attention():
    # after each replacement the keys are [the scripted sink frames | window | own chunk]
    cfg = _script_cfg()
    emb = [np.array(e, np.float32) for e in GOLDEN["embeddings"]]
    st, outs = brute.run_oracle(cfg, embed_fn=lambda c: emb[c])
    for s in range(1, cfg.num_steps):
        sinks = [f for f in GOLDEN["sink_frames_after_chunk"][s - 1] if f is not None]
        np.testing.assert_allclose(outs[(s, 0, 0)], brute.history_output(cfg, s, 0, 0, sink_frames=sinks),
                                   atol=1e-12)


def test_chunk_of_two_frames_decides_on_its_last_frame():
    # T' = 2, S = 1: chunk 0 = frames 0, 1.  Frame 0 becomes the sink with e_0 = h_0; the decision
    # on frame 1 compares h_0 with itself (alpha = 1, kept).  Chunk 1 (frames 2, 3) has h_1
    # orthogonal to h_0 (alpha = 0 < tau): sink 0 takes frame 3, the chunk's last frame.  Chunk 2
    # repeats h_1 (alpha = 1, kept).  Attention must then use frame 3 as the sink.
    D = 8
    h0 = np.zeros(D, np.float32); h0[0] = 1.0
    h1 = np.zeros(D, np.float32); h1[1] = 1.0
    emb = [h0, h1, h1, h1, h1]
    cfg = TINY_FP32.with_(chunk_frames=2, stream_batch=1, sink_frames=1, window_frames=3, num_chunks=5,
                          rope_refresh_period=0, embed_dim=D, sink_threshold=0.5, embed_kind="iid")
    st, outs = brute.run_oracle(cfg, embed_fn=lambda c: emb[c])
    got = [(d["chunk"], d["frame"], d["replaced"], d["alpha"]) for d in st.sink_log]
    assert got == [(0, 1, False, 1.0), (1, 3, True, 0.0), (2, 5, False, 1.0), (3, 7, False, 1.0),
                   (4, 9, False, 1.0)]
    assert st.sinks[0].frame == 3
    np.testing.assert_allclose(st.sink_embed[0], h1)
    for s in range(2, cfg.num_steps):
        np.testing.assert_allclose(outs[(s, 0, 0)], brute.history_output(cfg, s, 0, 0, sink_frames=[3]),
                                   atol=1e-12)


def test_similarity_terms_on_hand_computed_vectors():
    # h = (3, 4, 0), e0 = (4, 3, 0), e1 = (0, 0, 2), e2 = 0: h.h = 25, e.e = 25, 4, 0;
    # h.e = 24, 0, 0; alpha = 24/25, 0 (orthogonal), 0 (zero norm).
    h = np.array([3.0, 4.0, 0.0])
    t = sink.similarity_terms(h, [np.array([4.0, 3.0, 0.0]), np.array([0.0, 0.0, 2.0]), np.zeros(3)])
    assert t["hh"] == 25.0
    assert t["ee"] == [25.0, 4.0, 0.0]
    assert t["he"] == [24.0, 0.0, 0.0]
    assert t["alphas"] == [24.0 / 25.0, 0.0, 0.0]
    # a negative dot product: e = (-3, -4, 0) is antiparallel, alpha = -1 exactly
    t2 = sink.similarity_terms(h, [np.array([-3.0, -4.0, 0.0])])
    assert t2["he"] == [-25.0] and t2["alphas"] == [-1.0]
