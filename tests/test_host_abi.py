"""CPU tests of the C ABI: the library loads and exports every declared symbol, and its
host-only entry points (validation, layout, schedule, noise schedule) behave as documented.
No kernel is launched here."""
import math
import pathlib
import re

import numpy as np
import pytest

from oracle import motion as omotion
from oracle import stream as ost
from rolling_kv_causal_amd import sdv2
from synth import configs

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "sdv2.h"


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(sdv2_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 17
    L = sdv2.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # the binding exposes the same names
    assert all(hasattr(sdv2, n) for n in names)


def test_struct_layout_matches_header():
    # field order and types of sdv2_config / sdv2_layout as declared in the header
    text = HEADER.read_text()
    body = re.search(r"typedef struct sdv2_config \{(.*?)\} sdv2_config;", text, re.S).group(1)
    fields = re.findall(r"(int32_t|double)\s+([^;]+);", body)
    names = []
    for ty, decl in fields:
        names += [(ty, n.strip()) for n in decl.split(",")]
    want = [(("double" if f[1] is sdv2.ctypes.c_double else "int32_t"), f[0]) for f in sdv2.Config._fields_]
    assert names == want


@pytest.mark.parametrize("c", configs.ALL, ids=lambda c: c.name)
def test_workload_configs_validate_and_size(c):
    cfg = sdv2.config_of(c)
    sdv2.sdv2_config_validate(cfg)
    kv, meta, ws = sdv2.sdv2_cache_size(cfg)
    L = sdv2.sdv2_cache_layout(cfg)
    N = c.grid_h * c.grid_w
    assert L.tokens_padded % 64 == 0 and N <= L.tokens_padded < N + 64
    assert L.slots == c.sink_frames + c.window_frames + c.stream_batch * c.chunk_frames
    assert L.layer_stride == 2 * L.slots * c.num_heads * L.tokens_padded * c.head_dim
    assert kv == c.num_layers * L.layer_stride * (2 if c.dtype == "bf16" else 4)
    assert meta > 0 and ws >= 0


def test_wan14b_cache_is_about_8_4_gb_plus_staging():
    # 40 layers x (1 sink + 8 window + 1 chunk) frames x 1024 tokens x 40 heads x 128 x 2 (K, V)
    # x 2 bytes = 8.39 GB; the cache also holds B = 4 staging frames.
    c = configs.WAN14B_40LAYER_B4
    kv, _, _ = sdv2.sdv2_cache_size(sdv2.config_of(c))
    per_frame = 40 * 1024 * 40 * 128 * 2 * 2
    assert kv == per_frame * (1 + 8 + 4)
    assert abs(per_frame * 10 / 1e9 - 8.39) < 0.01


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, sdv2.SDV2_EINVAL), ("num_layers", 0, sdv2.SDV2_EINVAL),
    ("window_frames", 0, sdv2.SDV2_EINVAL), ("chunk_frames", 0, sdv2.SDV2_EINVAL),
    ("chunk_frames", 9, sdv2.SDV2_EINVAL), ("window_frames", 63, sdv2.SDV2_EINVAL),
    ("stream_batch", 9, sdv2.SDV2_EINVAL), ("rope_dim_t", 46, sdv2.SDV2_EINVAL),
    ("rope_dim_h", 41, sdv2.SDV2_EINVAL), ("rope_theta", 1.0, sdv2.SDV2_EINVAL),
    ("dtype", 7, sdv2.SDV2_EINVAL), ("sink_frames", 17, sdv2.SDV2_EINVAL),
    ("rope_refresh_period", -1, sdv2.SDV2_EINVAL), ("grid_w", 0, sdv2.SDV2_EINVAL),
])
def test_invalid_configs_are_rejected(field, value, code):
    cfg = sdv2.config_of(configs.WAN13B_1LAYER)
    setattr(cfg, field, value)
    with pytest.raises(sdv2.SDV2Error) as e:
        sdv2.sdv2_config_validate(cfg)
    assert e.value.code == code and sdv2.sdv2_last_error()


def test_fp8_cache_config():
    # e4m3 cache: dtype code 2, one byte per element, head_dim 128 only
    c = configs.WAN14B_40LAYER_B4.with_(kv_fp8=True)
    cfg = sdv2.config_of(c)
    assert cfg.dtype == sdv2.SDV2_BF16_KV_FP8
    sdv2.sdv2_config_validate(cfg)
    kv, _, _ = sdv2.sdv2_cache_size(cfg)
    assert kv == sdv2.sdv2_cache_size(sdv2.config_of(configs.WAN14B_40LAYER_B4))[0] // 2
    assert sdv2.config_of(c.with_(dtype="fp32")).dtype == sdv2.SDV2_F32      # fp32 runs keep fp32
    cfg = sdv2.config_of(configs.TINY_FP32.with_(dtype="bf16", kv_fp8=True))  # head_dim 64
    with pytest.raises(sdv2.SDV2Error) as e:
        sdv2.sdv2_config_validate(cfg)
    assert e.value.code == sdv2.SDV2_EINVAL and "128" in sdv2.sdv2_last_error()


def test_sink_threshold_needs_embeddings():
    cfg = sdv2.config_of(configs.WAN13B_1LAYER)
    cfg.sink_threshold = 0.5
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_config_validate(cfg)
    cfg.embed_dim = 8
    sdv2.sdv2_config_validate(cfg)
    cfg.sink_threshold = -math.inf              # off again
    cfg.embed_dim = 0
    sdv2.sdv2_config_validate(cfg)


def test_chunk_frames_limits():
    # B * T' <= 8 and S + W + T' <= 64; T' > 1 sizes T' slots per element
    c = configs.WAN13B_1LAYER.with_(chunk_frames=2, stream_batch=4)
    cfg = sdv2.config_of(c)
    sdv2.sdv2_config_validate(cfg)
    assert sdv2.sdv2_cache_layout(cfg).slots == 1 + 8 + 4 * 2
    cfg.stream_batch = 5
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_config_validate(cfg)
    cfg = sdv2.config_of(configs.WAN13B_1LAYER.with_(chunk_frames=8, window_frames=55, sink_frames=1))
    sdv2.sdv2_config_validate(cfg)
    cfg.window_frames = 56
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_config_validate(cfg)


@pytest.mark.parametrize("B,M,T", [(1, 5, 1), (2, 7, 1), (4, 6, 1), (4, 2, 1), (8, 11, 1),
                                   (1, 5, 2), (2, 7, 3), (4, 6, 2), (2, 3, 4)])
def test_plan_step_matches_oracle_schedule(B, M, T):
    c = configs.WAN13B_1LAYER.with_(stream_batch=B, num_chunks=M, chunk_frames=T)
    cfg = sdv2.config_of(c)
    for s in range(M + B + 1):
        first, nb, commit, newest = sdv2.sdv2_plan_step(cfg, M, s)
        want = ost.schedule(c, s)
        assert nb == len(want["chunks"])
        if nb:
            assert list(range(first, first + nb)) == want["chunks"]
            assert newest == want["newest_frame"]
        assert commit == (want["commit"] if want["commit"] is not None else -1)


def test_noise_schedule_matches_oracle():
    g = np.random.default_rng(0)
    d = np.abs(g.standard_normal(50)) * 0.4
    for sigma, k, lam in [(1.0, 4, 0.9), (0.3, 1, 0.5), (2.0, 7, 1.0)]:
        got = sdv2.sdv2_noise_schedule(list(d), sigma, k, lam, 0.25, 1.0, 1.0)
        np.testing.assert_allclose(got, omotion.noise_schedule(d, sigma, k, lam, 0.25, 1.0), rtol=1e-14)
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_noise_schedule([0.1], 0.0, 4, 0.9, 0.25, 1.0, 1.0)


def test_motion_workspace_size_and_errors():
    assert sdv2.sdv2_motion_workspace_size(129, 99840) == 128 * 7 * 8
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_motion_workspace_size(1, 10)


def test_null_handle_and_bad_arguments_fail_cleanly():
    with pytest.raises(sdv2.SDV2Error) as e:
        sdv2.sdv2_cache_slot_info(None, 0)
    assert e.value.code == sdv2.SDV2_EINVAL
    sdv2.sdv2_cache_destroy(None)


def test_latency_fit_and_slo_select_match_the_oracle():
    from oracle import slo
    g = np.random.default_rng(7)
    for _ in range(300):
        n = int(g.integers(2, 9))
        frames = [int(x) for x in g.integers(1, 9, n)]
        if len(set(frames)) < 2:
            frames[-1] = frames[0] % 8 + 1
        lat = [0.002 + 0.001 * x + float(g.normal(0, 2e-4)) for x in frames]
        c0, c1 = sdv2.sdv2_latency_fit(frames, lat)
        o0, o1 = slo.fit_latency(frames, lat)
        assert c0 == pytest.approx(o0, abs=1e-12) and c1 == pytest.approx(o1, abs=1e-12)
        c0, c1 = abs(c0) + 1e-4, abs(c1)
        args = (float(g.uniform(10, 2000)), float(g.uniform(0.005, 0.2)), int(g.integers(1, 10)),
                int(g.integers(1, 9)), int(g.integers(1, 9)))
        got = sdv2.sdv2_slo_select(c0, c1, *args)
        want = slo.select(c0, c1, *args)
        assert (got["B"], got["T"], got["feasible"]) == (want["B"], want["T"], want["feasible"])
        assert got["fps"] == pytest.approx(want["fps"], rel=1e-12)
        assert got["latency"] == pytest.approx(want["latency"], rel=1e-12)


def test_slo_select_errors():
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_latency_fit([2, 2, 2], [0.1, 0.2, 0.3])         # one distinct frame count
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_slo_select(-0.01, 0.001, 100.0, 1.0, 8, 8, 8)    # L <= 0 for small B T'
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_slo_select(0.01, 0.001, 0.0, 1.0, 8, 8, 8)       # target_fps <= 0
    with pytest.raises(sdv2.SDV2Error):
        sdv2.sdv2_slo_select(0.01, 0.001, 100.0, 1.0, 0, 8, 8)     # no frames ready


def test_generated_attention_asm_is_current():
    # attn_w64_asm.h is the output of gen_attn_w64.py (which also checks its hazard rules)
    import pathlib
    import subprocess
    import sys
    csrc = pathlib.Path(sdv2.__file__).resolve().parent / "csrc"
    out = subprocess.run([sys.executable, "gen_attn_w64.py"], cwd=csrc, capture_output=True, text=True, check=True)
    assert out.stdout == (csrc / "attn_w64_asm.h").read_text()


def _asm_register_set(spec):
    """Registers named by one constraint or clobber string: v12, a[0:31], s84 ..."""
    import re
    m = re.match(r"^([vas])\[(\d+):(\d+)\]$", spec)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {spec} if re.match(r"^[vas]\d+$", spec) else set()


def test_generated_asm_writes_only_declared_registers():
    # every register the tile-loop programs write is an output or a clobber of the asm statement
    # that runs them (an undeclared write corrupts whatever the compiler keeps there)
    import importlib.util
    import pathlib
    import re
    csrc = pathlib.Path(sdv2.__file__).resolve().parent / "csrc"
    src = (csrc / "k_attention_w64.hip").read_text()
    spec = importlib.util.spec_from_file_location("gen_attn_w64_test", csrc / "gen_attn_w64.py")
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)

    def macro(name):
        # the #define line and its backslash-continued lines
        lines = src[src.index(f"#define {name}"):].split("\n")
        out = []
        for line in lines:
            out.append(line)
            if not line.rstrip().endswith("\\"):
                break
        return "\n".join(out)

    shared = "".join(macro(m) for m in re.findall(r"#define (SDV2_W64_\w*(?:OUTPUTS|CLOBBERS))\b", src))
    for prog_name, f8 in (("SDV2_W64_LOOP_FP8", True), ("SDV2_W64_LOOP\n", False)):
        i = src.index(f"asm volatile({prog_name}")
        stmt = src[i:src.index(");", i)]
        declared = set()
        for text in (shared, stmt):
            for c in re.findall(r'"[=+]&?\{([^}]*)\}"', text):
                declared |= _asm_register_set(c)
            for c in re.findall(r'"([vas]\d+)"', text):
                declared |= _asm_register_set(c)
        gen.F8 = f8
        written = set()
        for line in gen.loop_program():
            t = line.replace(",", " ").split()
            if not t or t[0].startswith(".") or t[0] in ("s_waitcnt", "s_nop", "s_barrier", "s_branch") or \
                    t[0].startswith(("s_cbranch", "s_cmp", "global_load", "ds_write", "v_cmp_")):
                continue
            written |= _asm_register_set(t[1])
        assert not written - declared, (prog_name.strip(), sorted(written - declared))


def test_forced_split_count_sizes_the_workspace(monkeypatch):
    # SDV2_NSPLIT forces the split-KV count: a small bf16 stream whose cost model keeps one
    # split (no workspace) needs partials for four when forced, clamped to the shortest walk
    from synth import configs
    c = configs.TINY_FP32.with_(dtype="bf16", head_dim=128, rope_dim_t=44, rope_dim_h=42, rope_dim_w=42,
                                chunk_frames=2, grid_h=9, grid_w=9, num_heads=2, sink_frames=1,
                                window_frames=1, stream_batch=2, rope_refresh_period=0, sink_threshold=None,
                                embed_dim=0, embed_kind=None)
    cfg = sdv2.config_of(c)
    monkeypatch.delenv("SDV2_NSPLIT", raising=False)
    ws_model = sdv2.sdv2_cache_size(cfg)[2]
    monkeypatch.setenv("SDV2_NSPLIT", "4")
    ws4 = sdv2.sdv2_cache_size(cfg)[2]
    monkeypatch.setenv("SDV2_NSPLIT", "64")
    ws_big = sdv2.sdv2_cache_size(cfg)[2]
    rows = 2 * 2 * 2 * 81                       # elements x heads x T' x tokens, per split
    assert ws_model == 0
    assert ws4 >= 4 * rows * (128 * 2 + 8)
    assert ws4 <= ws_big <= 16 * rows * (128 * 2 + 8) + 4096


def test_generator_hazard_check_rejects_an_early_softmax():
    # the generator's hazard check is live: starting the exponentials at the 17th MFMA reads
    # S^T of key block 0 fewer than 12 instructions after the MFMA that writes it
    import importlib.util
    import pathlib
    csrc = pathlib.Path(sdv2.__file__).resolve().parent / "csrc"
    spec = importlib.util.spec_from_file_location("gen_attn_w64_hz", csrc / "gen_attn_w64.py")
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    gen.emit("X", gen.loop_program())          # the committed schedule passes
    gen.SM_FROM = 17
    with pytest.raises(AssertionError):
        gen.emit("X", gen.loop_program())


def test_generator_hazard_check_rejects_a_missing_lds_wait():
    # dropping the second LDS wait of the first tile stream leaves an MFMA reading a fragment
    # whose ds_read may still be in flight: the check must reject the program
    import importlib.util
    import pathlib
    csrc = pathlib.Path(sdv2.__file__).resolve().parent / "csrc"
    spec = importlib.util.spec_from_file_location("gen_attn_w64_lds", csrc / "gen_attn_w64.py")
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    lines = [l for l in gen.loop_program() if not l.startswith(".L")]
    gen.check_hazards(lines)
    first_read = next(i for i, l in enumerate(lines) if l.startswith("ds_read_b128"))
    waits = [i for i, l in enumerate(lines) if i > first_read and l.startswith("s_waitcnt lgkmcnt")]
    with pytest.raises(AssertionError):
        gen.check_hazards(lines[:waits[1]] + lines[waits[1] + 1:])
