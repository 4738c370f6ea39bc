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
    assert sdv2.sdv2_motion_workspace_size(129, 99840) == 128 * 25 * 8    # 25 parts of 4096 elements per pair
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
    for prog_name, f8, scaled in (("SDV2_W64_LOOP_FP8", True, True), ("SDV2_W64_LOOP_SK", False, True),
                                  ("SDV2_W64_LOOP\n", False, False)):
        i = src.index(f"asm volatile({prog_name}")
        stmt = src[i:src.index(");", i)]
        declared = set()
        for text in (shared, stmt):
            for c in re.findall(r'"[=+]&?\{([^}]*)\}"', text):
                declared |= _asm_register_set(c)
            for c in re.findall(r'"([vas]\d+)"', text):
                declared |= _asm_register_set(c)
        gen.set_mode(f8, scaled)
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


def test_random_stream_configs_are_valid(monkeypatch):
    # the seeded random configurations of the GPU parity sweep are inside the library's limits,
    # and every work plan their streams reach (with the forced split counts) covers each key
    # tile once
    import random_configs
    for seed in random_configs.SEEDS:
        c = random_configs.random_config(seed)
        cfg = sdv2.config_of(c)
        sdv2.sdv2_config_validate(cfg)
        nsplit = random_configs.forced_splits(seed)
        if nsplit:
            monkeypatch.setenv("SDV2_NSPLIT", str(nsplit))
        else:
            monkeypatch.delenv("SDV2_NSPLIT", raising=False)
        for nb in range(1, c.stream_batch + 1):
            for shared in range(c.sink_frames + c.window_frames + 1):
                if c.dtype == "bf16" and c.head_dim == 128:
                    sdv2.sdv2_debug_check_plan(cfg, nb, shared)


def test_generator_staging_check_rejects_planted_mistakes():
    # The e4m3 program widens each staged tile in the stream of the iteration after its loads;
    # check_staging runs one wave's loads, waits and LDS traffic.  It passes the committed
    # program and rejects: a vmcnt wait one load short, the widening reading the other staging
    # slot, K(t+1) widened into the ring slot K(t) is being read from, and a widened write of
    # registers whose conversion comes later.
    import importlib.util
    import pathlib
    csrc = pathlib.Path(sdv2.__file__).resolve().parent / "csrc"
    spec = importlib.util.spec_from_file_location("gen_attn_w64_stage", csrc / "gen_attn_w64.py")
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    gen.set_mode(True, scaled=True)
    gen.check_staging()
    resolve, units = gen.resolve_waits, gen.widen_units

    def short_wait(out):
        return [f"s_waitcnt vmcnt({int(l.split('(')[1].rstrip(')')) + 1})" if l.startswith("s_waitcnt vmcnt") else l
                for l in resolve(out)]

    def edit_units(fix):
        def f(ph, pc):
            return [(g, [fix(ph, x) for x in u]) for g, u in units(ph, pc)]
        return f

    def other_stage(ph, x):
        line = x[0] if isinstance(x, tuple) else x
        if line.startswith("ds_read_b128") and (f"v{gen.SK}" in line or f"v{gen.SV}" in line):
            off = int(line.split("offset:")[1])
            line = line.split("offset:")[0] + f"offset:{off ^ gen.STAGE}"
        return (line, x[1]) if isinstance(x, tuple) else line

    def early_write(ph, x):
        # K0's low half written from the registers of V1, whose conversions come later
        if isinstance(x, str) and x.startswith(f"ds_write_b128 v{gen.TMP},"):
            lo = int(x.split("v[")[1].split(":")[0])
            return x.replace(f"v[{lo}:{lo + 3}]", f"v[{lo + 24}:{lo + 27}]")
        return x

    def k_into_read_slot(ph, x):
        if isinstance(x, str) and x.startswith("ds_write_b128") and int(x.split()[1].rstrip(",")[1:]) < gen.TMP + 4:
            return x.split("offset:")[0] + f"offset:{(ph % gen.NSLOT) * gen.KTILE}"
        return x

    for name, attr, plant in (("short vmcnt", "resolve_waits", short_wait),
                              ("other staging slot", "widen_units", edit_units(other_stage)),
                              ("K over the slot being read", "widen_units", edit_units(k_into_read_slot)),
                              ("a write before its conversion", "widen_units", edit_units(early_write))):
        setattr(gen, attr, plant)
        with pytest.raises(AssertionError):
            gen.check_staging()
        setattr(gen, attr, resolve if attr == "resolve_waits" else units)
    gen.check_staging()


def test_generator_ring_check_rejects_planted_mistakes():
    # The bf16 programs load each K and V^T tile straight into an LDS ring slot two iterations
    # ahead; check_ring runs one wave's loads, waits, barriers and fragment reads.  It passes
    # both committed bf16 programs and rejects: the iteration's vmcnt wait one load short, the
    # barrier left out, K(t+2) loaded into the slot K(t+1) is about to be read from, V^T(t+1)
    # loaded into the slot V^T(t-1) is being read from, and the stream's last fragment read moved
    # after its final LDS wait (still in flight at the next barrier).
    import importlib.util
    import pathlib
    csrc = pathlib.Path(sdv2.__file__).resolve().parent / "csrc"
    spec = importlib.util.spec_from_file_location("gen_attn_w64_ring", csrc / "gen_attn_w64.py")
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    for scaled in (False, True):
        gen.set_mode(False, scaled=scaled)
        gen.check_ring()
    iteration, loads, resolve = gen.iteration, gen.tile_loads, gen.resolve_waits

    def short_wait(ph):
        return [l.replace("vmcnt(8)", "vmcnt(9)") for l in iteration(ph)]

    def no_barrier(ph):
        return [l for l in iteration(ph) if l != "s_barrier"]

    def slot_shift(kind, delta):
        def f(ph):
            base = "%[mk]" if kind == "K" else "%[mv]"
            d = {}
            for i, (setup, load) in loads(ph).items():
                if setup.startswith(f"s_add_u32 m0, {base},"):
                    off = int(setup.split(",")[-1])
                    setup = f"s_add_u32 m0, {base}, {(off + delta * gen.KTILE) % (gen.NSLOT * gen.KTILE)}"
                d[i] = (setup, load)
            return d
        return f

    def read_after_last_wait(out):
        lines = resolve(out)
        last = max(i for i, l in enumerate(lines) if l.startswith("ds_read_b128"))
        return lines[:last] + lines[last + 1:] + [lines[last]]

    for name, attr, plant in (("short vmcnt", "iteration", short_wait),
                              ("no barrier", "iteration", no_barrier),
                              ("K one slot early", "tile_loads", slot_shift("K", -1)),
                              ("V^T two slots late", "tile_loads", slot_shift("V", 2)),
                              ("a read in flight at the barrier", "resolve_waits", read_after_last_wait)):
        setattr(gen, attr, plant)
        with pytest.raises(AssertionError):
            gen.check_ring()
        setattr(gen, attr, {"iteration": iteration, "tile_loads": loads, "resolve_waits": resolve}[attr])
    gen.check_ring()


def test_layer_blocks_over_the_32_bit_offset_range_are_rejected():
    # The attention tile loop forms offsets inside a layer's K or V block in 32 bits: a layer
    # block of 4 GiB or more, or a slot of 2 GiB or more, is refused at validation.
    big = sdv2.config_of(configs.WAN14B_40LAYER_B4.with_(grid_h=128, grid_w=128, sink_frames=16,
                                                         window_frames=40, stream_batch=8,
                                                         sink_threshold=None, embed_dim=0))
    with pytest.raises(sdv2.SDV2Error) as e:
        sdv2.sdv2_config_validate(big)
    assert e.value.code == sdv2.SDV2_EINVAL and "4 GiB" in str(e.value)
    slot = sdv2.config_of(configs.WAN13B_1LAYER.with_(grid_h=1024, grid_w=1024, num_heads=8))
    with pytest.raises(sdv2.SDV2Error) as e:
        sdv2.sdv2_config_validate(slot)
    assert "2 GiB" in str(e.value)
    # the largest workload is far inside: 13 slots x 10.5 MB
    sdv2.sdv2_config_validate(sdv2.config_of(configs.WAN14B_40LAYER_B4))


def test_create_with_short_buffers_is_enospc_before_any_device_work():
    # the size checks come before any HIP call, so (aligned, never touched) stand-in addresses
    # are enough: each buffer one byte short gives SDV2_ENOSPC and no handle
    import ctypes
    cfg = sdv2.config_of(configs.WAN13B_1LAYER)
    kv, meta, ws = sdv2.sdv2_cache_size(cfg)
    assert ws > 0
    L = sdv2.lib()
    fake = 1 << 20
    for sizes in ((kv - 1, meta, ws), (kv, meta - 1, ws), (kv, meta, ws - 1)):
        h = ctypes.c_void_p()
        rc = L.sdv2_cache_create(ctypes.byref(cfg), fake, sizes[0], fake, sizes[1], fake, sizes[2], None,
                                 ctypes.byref(h))
        assert rc == sdv2.SDV2_ENOSPC and h.value is None, (sizes, rc)
        assert "bytes" in sdv2.sdv2_last_error()
    # misaligned buffers are EINVAL, also before any device work
    h = ctypes.c_void_p()
    assert L.sdv2_cache_create(ctypes.byref(cfg), fake + 16, kv, fake, meta, fake, ws, None,
                               ctypes.byref(h)) == sdv2.SDV2_EINVAL


def test_fault_injection_hook_arms_and_disarms():
    # host-only: arming and disarming the injection makes no HIP call
    sdv2.sdv2_debug_fail_hip_call(3)
    sdv2.sdv2_debug_fail_hip_call(-1)
    sdv2.sdv2_config_validate(sdv2.config_of(configs.TINY_FP32))


def test_asm_program_scalar_operands_are_sgprs(tmp_path):
    # Every named operand of the generated tile-loop program is scalar ("s").  The compiler may
    # satisfy an "s" operand whose value it computed in a VGPR with that VGPR, which the program
    # then reads while it overwrites the register for its own state (a scale computed in the
    # kernel once landed in an S^T register).  Compile the kernel to gfx950 assembly and check
    # that every %[name] of every program line was substituted with an SGPR.
    import re
    import subprocess
    csrc = pathlib.Path(__file__).resolve().parents[1] / "rolling_kv_causal_amd" / "csrc"
    out = tmp_path / "w64.s"
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
                        "-S", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", str(csrc.parents[1] / "include"), "-I", str(csrc),
                        str(csrc / "k_attention_w64.hip"), "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    header = (csrc / "attn_w64_asm.h").read_text()
    programs = {}
    for name, body in re.findall(r"#define (SDV2_W64_LOOP\w*) \\\n(.*?)(?:\n\n|\Z)", header, re.S):
        programs[name] = [ln for ln in re.findall(r'"(.*?)\\n\\t"', body)]
    assert set(programs) == {"SDV2_W64_LOOP", "SDV2_W64_LOOP_SK", "SDV2_W64_LOOP_FP8"}
    asm = out.read_text()
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", asm, re.S)
    blocks = [[ln.strip() for ln in b.splitlines() if ln.strip() and not ln.strip().startswith(";")] for b in blocks]
    blocks = [b for b in blocks if len(b) > 1000]
    assert len(blocks) == 3, [len(b) for b in blocks]

    def pattern(tmpl):
        parts = re.split(r"(%\[\w+\]|%=)", tmpl.strip())
        rx, names = "", []
        for part in parts:
            if part == "%=":
                rx += r"\d+"
            elif part.startswith("%["):
                rx += r"(\S+?)"
                names.append(part[2:-1])
            else:
                rx += re.escape(part).replace(r"\ ", r"\s+")
        return re.compile(rx + r"$"), names

    checked = 0
    for prog in programs.values():
        blk = next(b for b in blocks if len(b) == len(prog))
        for tmpl, line in zip(prog, blk):
            if "%[" not in tmpl:
                continue
            rx, names = pattern(tmpl)
            m = rx.match(line)
            assert m, (tmpl, line)
            for name, reg in zip(names, m.groups()):
                assert re.fullmatch(r"s\d+|s\[\d+:\d+\]", reg), f"%[{name}] is {reg} in: {line}"
                checked += 1
    assert checked > 1000


def test_generator_path_check_follows_branches():
    # An exponential at a branch target reads an MFMA result two instructions after the MFMA
    # along the branch; in text order 20 instructions separate them, so only the check that
    # follows branches (check_paths) rejects the program.
    import importlib.util
    import pathlib
    csrc = pathlib.Path(sdv2.__file__).resolve().parent / "csrc"
    spec = importlib.util.spec_from_file_location("gen_attn_w64_paths", csrc / "gen_attn_w64.py")
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    prog = (["v_mfma_f32_32x32x16_bf16 v[0:15], v[128:131], a[0:3], v[0:15]", "s_cbranch_scc0 .Lx"]
            + ["v_mov_b32 v200, 0"] * 20 + ["s_branch .Ly", ".Lx:", "v_exp_f32 v190, v3", ".Ly:", "s_nop 0"])
    gen.check_hazards([l for l in prog if not l.startswith(".L")])          # text order: passes
    with pytest.raises(AssertionError):
        gen.check_paths(prog)
    # with 12 instructions between them on the branch path as well, both checks pass
    ok = (["v_mfma_f32_32x32x16_bf16 v[0:15], v[128:131], a[0:3], v[0:15]"] + ["v_mov_b32 v201, 0"] * 12
          + ["s_cbranch_scc0 .Lx"] + ["v_mov_b32 v200, 0"] * 20 + ["s_branch .Ly", ".Lx:", "v_exp_f32 v190, v3",
                                                                   ".Ly:", "s_nop 0"])
    gen.check_paths(ok)
    # the committed programs pass along every path
    for f8, scaled in ((False, False), (False, True), (True, True)):
        gen.set_mode(f8, scaled)
        gen.check_paths(gen.loop_program())


@pytest.mark.parametrize("c", configs.ALL, ids=lambda c: c.name)
def test_split_plans_cover_every_key_tile_once(c, monkeypatch):
    # For every state the stream reaches (elements in flight, cached frames present), the work
    # plan the attention launches is checked by enumerating its workgroups through the kernels'
    # own decoder: every key tile of every query tile exactly once, partials inside the workspace
    cfg = sdv2.config_of(c)
    for forced in (None, "3", "16"):
        if forced:
            monkeypatch.setenv("SDV2_NSPLIT", forced)
        for nb in range(1, c.stream_batch + 1):
            for shared in range(c.sink_frames + c.window_frames + 1):
                sdv2.sdv2_debug_check_plan(cfg, nb, shared)
    monkeypatch.delenv("SDV2_NSPLIT", raising=False)
    if c.name == "wan14b_512_40layer_b4":
        # 640 query tiles on 8 x 32 CUs: 512 run whole, 128 split in two (768 workgroups)
        assert sdv2.sdv2_debug_check_plan(cfg, 4, 9) == (2, 128, 768)


def test_split_plans_on_random_shapes():
    rng = np.random.default_rng(11)
    for _ in range(150):
        c = configs.WAN13B_1LAYER.with_(num_heads=int(rng.integers(1, 48)), grid_h=int(rng.integers(1, 40)),
                                        grid_w=int(rng.integers(1, 60)), sink_frames=int(rng.integers(0, 4)),
                                        window_frames=int(rng.integers(1, 12)), chunk_frames=int(rng.integers(1, 4)),
                                        stream_batch=1)
        c = c.with_(stream_batch=int(rng.integers(1, 8 // c.chunk_frames + 1)))
        cfg = sdv2.config_of(c)
        nb = int(rng.integers(1, c.stream_batch + 1))
        shared = int(rng.integers(0, c.sink_frames + c.window_frames + 1))
        sdv2.sdv2_debug_check_plan(cfg, nb, shared)


def test_key_scale_validation():
    # key_scale > 0 (keys cached times it) only for the bf16 cache at head_dim 128; it must be
    # finite and >= 0; the scaled cache keeps the layout (same sizes)
    from synth import configs
    base = configs.WAN13B_1LAYER
    assert base.key_scale == base.softmax_scale
    good = sdv2.config_of(base)
    plain = sdv2.config_of(base.with_(scaled_keys=False))
    assert good.key_scale > 0 and plain.key_scale == 0
    assert sdv2.sdv2_cache_size(good) == sdv2.sdv2_cache_size(plain)
    for field, value in (("key_scale", -1.0), ("key_scale", float("nan")), ("key_scale", float("inf"))):
        c = sdv2.config_of(base)
        setattr(c, field, value)
        with pytest.raises(sdv2.SDV2Error) as e:
            sdv2.sdv2_cache_size(c)
        assert e.value.code == sdv2.SDV2_EINVAL and "key_scale" in str(e.value)
    for other in (base.with_(dtype="fp32"), base.with_(head_dim=64, rope_dim_t=24, rope_dim_h=20, rope_dim_w=20)):
        assert other.key_scale == 0          # the workload leaves it off where it is not allowed
        c = sdv2.config_of(other)
        c.key_scale = 0.125
        with pytest.raises(sdv2.SDV2Error) as e:
            sdv2.sdv2_cache_size(c)
        assert e.value.code == sdv2.SDV2_EINVAL and "key_scale" in str(e.value)
    # the e4m3 cache requires it
    fp8 = sdv2.config_of(base.with_(kv_fp8=True))
    assert fp8.key_scale == base.softmax_scale
    sdv2.sdv2_cache_size(fp8)
    fp8.key_scale = 0.0
    with pytest.raises(sdv2.SDV2Error) as e:
        sdv2.sdv2_cache_size(fp8)
    assert e.value.code == sdv2.SDV2_EINVAL and "key_scale" in str(e.value)
