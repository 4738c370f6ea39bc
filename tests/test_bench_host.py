"""Host-side logic of bench.py (no GPU): the one-GPU guard, the workloads' algorithmic FLOPs and
bytes, and the rule that a committed profile is used only for the sources it was taken on."""
import pathlib
import subprocess
import sys

import pytest

import bench
from synth import configs

ROOT = pathlib.Path(bench.__file__).resolve().parent


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and r.stdout == ""
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("c,gflop", [(configs.WAN13B_1LAYER, 64.4), (configs.WAN13B_30LAYER_B4, 257.7),
                                     (configs.WAN13B_480P_B2, 269.1), (configs.WAN14B_40LAYER_B4, 859.0)],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_attention_flops_per_layer_at_t1(c, gflop):
    # 4 B H N L d per layer with L = (S + W + 1) N keys (one frame per chunk): the figures the
    # hot-path scope table gives for these workloads
    N = c.tokens
    want = 4 * c.stream_batch * c.num_heads * N * (c.sink_frames + c.window_frames + 1) * N * c.head_dim
    got = bench.workload_numbers(c)["flops_per_layer"]
    assert got == want
    assert round(got / 1e9, 1) == gflop


def test_block_causal_flops_count_each_frame_of_the_chunk_over_its_own_keys():
    # T' = 2: frame t of the chunk attends over S + W + t + 1 frames of keys
    c = configs.WAN13B_30LAYER_T2B2
    N = c.tokens
    frames = sum(c.sink_frames + c.window_frames + t + 1 for t in range(c.chunk_frames))
    assert bench.workload_numbers(c)["flops_per_layer"] == 4 * c.stream_batch * c.num_heads * N * frames * N * c.head_dim


def test_attention_bytes_read_the_shared_cache_once():
    # Q and O of every element, the sinks' and window's K and V once, each element's own K and V
    c = configs.WAN14B_40LAYER_B4
    N, H, d, B = c.tokens, c.num_heads, c.head_dim, c.stream_batch
    want = 2 * B * N * H * d * 2 + 2 * (c.sink_frames + c.window_frames) * N * H * d * 2 + 2 * B * N * H * d * 2
    assert bench.workload_numbers(c)["attn_bytes_per_layer"] == want == 356515840
    f8 = bench.workload_numbers(c.with_(kv_fp8=True))["attn_bytes_per_layer"]
    assert f8 == 2 * B * N * H * d * 2 + (want - 2 * B * N * H * d * 2) // 2


def test_profiles_are_used_only_for_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    csrc = tmp_path / "rolling_kv_causal_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.ATTN_SOURCES:
        (csrc / name).write_text(f"// {name}\n")
    h = bench.attn_source_hash()
    (prof / "attn_traffic_w.md").write_text(f"# x\n\nbytes_per_call: 123\nattn_sources_sha256_16: {h}\n")
    assert bench.load_traffic("w") == 123
    (csrc / bench.ATTN_SOURCES[0]).write_text("// changed\n")
    assert bench.attn_source_hash() != h
    assert bench.load_traffic("w") is None
    assert bench.load_traffic("missing") is None

