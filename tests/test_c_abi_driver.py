"""The C ABI driven from plain C: tests/c_abi_driver.c (gcc, hipMalloc'd buffers, one HIP stream,
no Python or torch in the loop) runs whole small streams through sdv2_plan_step, refresh,
append, attention, commit and the sink refresh; every output of every step, layer and element
is compared with the oracle on the same seeded inputs, every sink decision bit for bit."""
import ctypes
import pathlib
import shutil
import subprocess

import numpy as np
import pytest

from gpu_helpers import assert_close, log
from oracle import stream as ost
from rolling_kv_causal_amd import sdv2
from synth import configs, inputs

pytestmark = pytest.mark.gpu

ROOT = pathlib.Path(__file__).resolve().parents[1]
LIB = ROOT / "rolling_kv_causal_amd"


def _build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not installed")
    exe = tmp_path / "c_abi_driver"
    cmd = [gcc, "-std=c11", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", str(ROOT / "include"), str(ROOT / "tests" / "c_abi_driver.c"), "-o", str(exe),
           "-L", str(LIB), "-lsdv2", f"-Wl,-rpath,{LIB}", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def _encode(cfg, x):
    """A storage array of the input generator (bf16 bit patterns or float32) as raw bytes."""
    return np.ascontiguousarray(x, np.uint16 if cfg.dtype == "bf16" else np.float32).tobytes()


def _decode(cfg, raw, shape):
    if cfg.dtype == "bf16":
        bits = np.frombuffer(raw, np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64).reshape(shape)
    return np.frombuffer(raw, np.float32).astype(np.float64).reshape(shape)


@pytest.mark.parametrize("kw", [
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=5, grid_w=13,
         num_heads=3, sink_frames=2, window_frames=3, stream_batch=3, rope_refresh_period=5, num_chunks=12,
         softmax_scale=128 ** -0.5, num_layers=2),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=7, grid_w=9,
         num_heads=2, sink_frames=1, window_frames=3, stream_batch=2, chunk_frames=2, rope_refresh_period=4,
         num_chunks=8, softmax_scale=128 ** -0.5, num_layers=2),
    dict(dtype="fp32", head_dim=64, grid_h=3, grid_w=7, num_heads=2, sink_frames=1, window_frames=2,
         stream_batch=2, rope_refresh_period=3, num_chunks=8),
    dict(dtype="bf16", kv_fp8=True, head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=5,
         grid_w=13, num_heads=2, sink_frames=1, window_frames=3, stream_batch=2, rope_refresh_period=4,
         num_chunks=10, softmax_scale=128 ** -0.5, num_layers=2),
    dict(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42, grid_h=12, grid_w=25,
         num_heads=4, sink_frames=3, window_frames=2, stream_batch=2, num_chunks=10, embed_dim=16,
         sink_threshold=0.2, embed_kind="iid", softmax_scale=128 ** -0.5),
], ids=["bf16-B3-refresh", "bf16-T2-block-causal", "fp32-d64", "e4m3-cache", "bf16-sink-refresh"])
def test_stream_from_plain_c_matches_the_oracle(kw, tmp_path):
    base = dict(rope_refresh_period=0, sink_threshold=None, embed_dim=0, embed_kind=None)
    base.update(kw)
    cfg = configs.TINY_FP32.with_(**base)
    exe = _build(tmp_path)
    ccfg = sdv2.config_of(cfg)
    L, rows, H, d = cfg.num_layers, cfg.chunk_rows, cfg.num_heads, cfg.head_dim
    st = ost.OracleStream(cfg, layers=list(range(L)))
    plans = []
    with open(tmp_path / "in.bin", "wb") as f:
        f.write(ctypes.string_at(ctypes.addressof(ccfg), ctypes.sizeof(ccfg)))
        f.write(np.int64(cfg.num_chunks).tobytes())
        f.write(np.float32(cfg.softmax_scale).tobytes())
        for s in range(cfg.num_steps):
            nb = len(ost.schedule(cfg, s)["chunks"])
            plans.append(nb)
            for layer in range(L):
                x = [inputs.qkv(cfg, s, layer, b) for b in range(nb)]
                for j in range(3):
                    for b in range(nb):
                        f.write(_encode(cfg, x[b][j]))
            commit = ost.schedule(cfg, s)["commit"]
            if commit is not None and cfg.embed_dim > 0:
                f.write(np.ascontiguousarray(inputs.chunk_embedding(cfg, commit), np.float32).tobytes())
    log(f"c_abi_driver {cfg.name}: {cfg.num_steps} steps")
    r = subprocess.run([str(exe), str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    raw = (tmp_path / "out.bin").read_bytes()
    eb = 2 if cfg.dtype == "bf16" else 4
    per_elem = rows * H * d * eb
    decisions = sum(1 for s in range(cfg.num_steps) if ost.schedule(cfg, s)["commit"] is not None) \
        if cfg.embed_dim > 0 else 0
    assert len(raw) == sum(nb * L * per_elem for nb in plans) + 16 * decisions
    pos, worst, replaced = 0, 0.0, 0
    for s, nb in enumerate(plans):
        plan = st.begin_step(s)
        assert len(plan["chunks"]) == nb
        x = {}
        for layer in range(L):
            got = _decode(cfg, raw[pos:pos + nb * per_elem], (nb, rows, H, d))
            pos += nb * per_elem
            for b in range(nb):
                x[(layer, b)] = inputs.qkv(cfg, s, layer, b)
                ref = st.attend(layer, b, *x[(layer, b)])
                worst = max(worst, assert_close(cfg, got[b], ref, f"C driver step {s} layer {layer} elem {b}"))
        commit = plan["commit"]
        h = inputs.chunk_embedding(cfg, commit) if (commit is not None and cfg.embed_dim > 0) else None
        dec = st.end_step({layer: x[(layer, 0)][1:] for layer in range(L)}, h)
        if h is not None:
            slot = int(np.frombuffer(raw[pos:pos + 8], np.int64)[0])
            alpha = float(np.frombuffer(raw[pos + 8:pos + 16], np.float64)[0])
            pos += 16
            if dec is None:
                assert (slot, alpha) == (-1, 1.0), (s, slot, alpha)
            else:
                assert slot == (dec["slot"] if dec["replaced"] else -1), (s, slot, dec)
                assert abs(alpha - dec["alpha"]) <= 1e-9, (s, alpha, dec["alpha"])
                replaced += dec["replaced"]
    assert pos == len(raw)
    if cfg.embed_dim > 0:
        assert replaced >= 1, "the stream should replace a sink at least once"
    log(f"c_abi_driver {cfg.name}: every output of {len(plans)} steps ok, worst max-abs {worst:.3g}, "
        f"sinks replaced {replaced}")
