"""The seeded input generators: rounding, determinism and the structure the workloads need."""
import numpy as np
import torch

from oracle import sink
from synth import configs, inputs


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -1.0, 0.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 3.0e38, -1e-40], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(inputs.f32_to_bf16_bits(x), want)


def test_qkv_deterministic_and_distinct():
    cfg = configs.TINY_FP32
    a = inputs.qkv(cfg, 3, 0, 0)
    b = inputs.qkv(cfg, 3, 0, 0)
    c = inputs.qkv(cfg, 4, 0, 0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[1], c[1])
    assert a[0].shape == (16, 2, 64) and a[0].dtype == np.float32


def test_bf16_workload_prescale():
    cfg = configs.WAN13B_1LAYER
    q, k, v = inputs.qkv(cfg, 0, 0, 0)
    assert q.dtype == np.uint16 and q.shape == (1024, 12, 128)
    qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).float().numpy()
    kf = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(qf.std() * np.sqrt(128) - 1) < 0.01 and abs(kf.std() - 1) < 0.01


def test_scene_embeddings_have_both_outcomes_with_margin():
    cfg = configs.WAN14B_40LAYER_B4
    emb = [inputs.chunk_embedding(cfg, c) for c in range(cfg.num_chunks)]
    cos = [sink.cosine(emb[c], emb[c - 1]) for c in range(1, cfg.num_chunks)]
    tau = cfg.sink_threshold
    assert min(abs(c - tau) for c in cos) > 1e-3
    assert any(c < tau for c in cos) and any(c > tau for c in cos)


def test_motion_frames_drift_and_jumps():
    cfg = configs.WAN13B_480P_B2
    x = inputs.motion_frames(cfg, frames=40)
    assert x.shape == (40, 16, 60, 104) and x.dtype == np.float32
    d = np.sqrt(np.mean((x[1:].astype(np.float64) - x[:-1]) ** 2, axis=(1, 2, 3)))
    drift = np.abs(d - 0.05) < 1e-4
    jump = d > 1.0                      # a fresh N(0,1) frame against a drifted one
    assert np.all(drift | jump) and drift.sum() > 20 and jump.sum() >= 1
