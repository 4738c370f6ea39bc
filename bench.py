"""Throughput of the sink + rolling-KV chunk-attention step on one MI355X.

A step is one pass of the whole hot path over one stream-batch of synthetic input: RoPE refresh
(when due), per layer the fused RoPE + append and the chunk attention, the commit of the
finished chunk, and - where the workload has them - the sink similarity decision + replacement
and the motion reduction of the newest latent frame.  Inputs are seeded device-resident random
tensors of the workload's shapes, generated before the timed region.

Prints one JSON line.  `value` is the attention work of the step (algorithmic FLOPs,
4 * nbatch * H * N * L * d per layer with L = (S + W + 1) * N keys) divided by the step time.
`roofline` scores the attention call (split-KV kernel + combine) against the bf16 MFMA peak;
its duration comes from HIP events on the library's stream around each attention call of steps
run after the timed ones, in the same order (workloads of 8 or more layers; a single-layer
workload, whose step the host cannot keep ahead of, times a batch of back-to-back calls
instead).  No event sits inside the timed steps.  `hbm_kernels` scores the HBM-bound kernels
(append, rebase, sink copy, split combine, motion reduction) against 8 TB/s.  `cpu_baseline`
times the float64 oracle on a bounded sample of the same workload on the host cores.
`reference_rates` (bf16 workloads, after the timed steps) times torch.matmul's square bf16 GEMM
(hipBLASLt) and PyTorch's SDPA on the workload's attention shape on the same GPU;
`roofline.frac_of_measured_gemm` divides `achieved` by the 16384^3 GEMM's rate, a measured
second denominator beside the published peak.

The default workload is the largest single-GPU one: the Wan-14B-shaped 40-layer stack with a
stream batch of 4 and the sink refresh.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the attention kernels, their shared definitions and the host code that sizes their launches
# (the split-KV work plan): a profile taken on other sources is not used
ATTN_SOURCES = ("k_attention.hip", "k_attention_w64.hip", "attn_w64_asm.h", "attn_tiles.h", "common.h", "sdv2.cpp")


def attn_source_hash() -> str:
    """First 16 hex digits of the sha256 of the attention kernels' sources (in this order)."""
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        h.update((ROOT / "rolling_kv_causal_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def visible_keys(c, t):
    """Keys a query of own-chunk frame t sees: sinks + window + own frames 0..t (block-causal)."""
    return (c.sink_frames + c.window_frames + t + 1) * c.tokens


def workload_numbers(c):
    N = c.tokens
    L = (c.sink_frames + c.window_frames + c.chunk_frames) * N
    B = c.stream_batch
    eb = 2 if c.dtype == "bf16" else 4                 # activations (Q, O)
    kb = 1 if c.kv_fp8 else eb                          # cache elements (K, V)
    flops_layer = 4 * B * c.num_heads * N * c.head_dim * sum(visible_keys(c, t) for t in range(c.chunk_frames))
    # algorithmic bytes of one attention call: Q + O, the shared sink+window K/V read once, and
    # each element's own chunk K/V
    qo = 2 * B * c.chunk_rows * c.num_heads * c.head_dim * eb
    shared = 2 * (c.sink_frames + c.window_frames) * N * c.num_heads * c.head_dim * kb
    own = 2 * B * c.chunk_rows * c.num_heads * c.head_dim * kb
    return {"keys": L, "flops_per_layer": flops_layer, "attn_bytes_per_layer": qo + shared + own}


def make_inputs(c, run, pool, seed=20261203):
    """Seeded device-resident q, k, v of the workload's shapes: pool sets per layer."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    shape = (c.stream_batch, c.chunk_rows, c.num_heads, c.head_dim)
    return [[tuple((torch.randn(shape, generator=g, device="cuda") *
                    (c.q_prescale if j == 0 else 1.0)).to(run.dtype) for j in range(3))
             for _ in range(c.num_layers)] for _ in range(pool)]


class Stepper:
    """One stream of the workload over device-resident inputs; steps of the whole hot path."""

    def __init__(self, c, pool=2):
        import torch

        from rolling_kv_causal_amd.stream import StreamRunner
        from synth import inputs
        self.c = c
        self.run = StreamRunner(self._cfg(c), 1 << 40, c.softmax_scale)   # unbounded: steady state
        self.sets = make_inputs(c, self.run, pool)
        self.embeds = None
        if c.embed_dim > 0:
            self.embeds = torch.stack([torch.from_numpy(inputs.chunk_embedding(c, i))
                                       for i in range(c.num_chunks)]).cuda()
        self.frames = None
        if c.motion is not None:
            self.frames = torch.from_numpy(inputs.motion_frames(c)).cuda()
        self.stats = torch.empty(4 + 2 * c.sink_frames, dtype=torch.float64, device="cuda")
        self.s = 0

    @staticmethod
    def _cfg(c):
        from rolling_kv_causal_amd import sdv2
        return sdv2.config_of(c)

    def step(self, ev=None, attn_repeat=1, calls=None):
        """One step.  ev: dict of event pairs to record around the append batch, the attention
        batch (all layers back to back, each call repeated attn_repeat times), the refresh and
        the end-of-step chunk statistics / sink refresh.  Without ev, append and attention
        alternate per layer as in a DiT forward; calls: then a dict whose "attention" list holds
        one event pair per layer, recorded around each attention call."""
        c, run = self.c, self.run
        first, nb, commit, newest = run.plan(self.s)
        st = self.sets[self.s % len(self.sets)]
        mark = (lambda k, i: ev[k][i].record()) if ev else (lambda k, i: None)
        mark("refresh", 0)
        run.cache.refresh(newest)
        mark("refresh", 1)
        if ev:
            mark("append", 0)
            for layer in range(c.num_layers):
                q, k, v = st[layer]
                run.cache.append(layer, first, nb, q[:nb], k[:nb], v[:nb])
            mark("append", 1)
            mark("attention", 0)
            for layer in range(c.num_layers):
                for _ in range(attn_repeat):
                    run.cache.attention(layer, nb, st[layer][0][:nb], run.out[layer, :nb], run.scale)
            mark("attention", 1)
        else:
            for layer in range(c.num_layers):
                q, k, v = st[layer]
                run.cache.append(layer, first, nb, q[:nb], k[:nb], v[:nb])
                if calls:
                    calls["attention"][layer][0].record()
                run.cache.attention(layer, nb, q[:nb], run.out[layer, :nb], run.scale)
                if calls:
                    calls["attention"][layer][1].record()
        if commit >= 0:
            run.cache.commit(commit)
            last = (commit + 1) * c.chunk_frames - 1            # the chunk's last frame
            e = self.embeds[commit % len(self.embeds)] if self.embeds is not None else None
            prev = cur = None
            if self.frames is not None:
                t = 1 + last % (len(self.frames) - 1)
                prev, cur = self.frames[t - 1], self.frames[t]
            if e is not None or cur is not None:
                mark("stats", 0)
                run.cache.sink_replace(last, e, prev, cur, self.stats, sync=False)
                mark("stats", 1)
        self.s += 1


def events(names):
    import torch
    return {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}


def run_gpu(c, steps, warmup):
    """Whole-step time over the timed steps (no event inside them: an event record between two
    calls delays the next kernel by several microseconds); then per-call attention times from
    HIP events around each attention call of further steps of the same kind (workloads of 8 or
    more layers, where the host enqueues far ahead of the GPU), else from a pass with events
    around batched calls."""
    import torch
    torch.cuda.set_device(0)
    st = Stepper(c)
    fill = c.sink_frames + c.window_frames + c.stream_batch + 1
    for _ in range(fill + warmup):
        st.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        st.step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    med = lambda v: sorted(v)[len(v) // 2] if v else None
    per_call = c.num_layers >= 8
    npass = max(3, min(10, steps // 2))
    if per_call:
        calls = [{"attention": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                                for _ in range(c.num_layers)]} for _ in range(npass)]
        for cl in calls:
            st.step(calls=cl)
        torch.cuda.synchronize()
        mean_ms = lambda pairs: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
        in_step_us = med([mean_ms(cl["attention"]) for cl in calls]) * 1e3
    # batched pass: events around the append batch and the attention batch of each step; a
    # single-layer workload repeats its attention call so that a batch holds several calls
    repeat = max(1, 8 // c.num_layers)
    names = ("refresh", "append", "attention", "stats")
    acc = {n: [] for n in names}
    for _ in range(npass):
        ev = events(names)
        st.step(ev, attn_repeat=repeat)
        torch.cuda.synchronize()
        for n in names:
            a, b = ev[n]
            try:
                acc[n].append(a.elapsed_time(b))
            except (RuntimeError, ValueError):    # the pair was not recorded this step
                pass
    attn_ms = med(acc["attention"])
    if per_call:
        timing = (f"HIP events on the library's stream around each of the {c.num_layers} attention calls of "
                  f"{npass} steps run after the timed ones (append and attention alternating per layer, as "
                  "in the timed steps); median over the steps of the mean per call")
    else:
        timing = (f"HIP events on the library's stream around {c.num_layers * repeat} back-to-back attention "
                  "calls per step (median of the batched steps)")
    return {"ms_per_step": ms_step, "wall_s": wall,
            "attention_us": in_step_us if per_call else attn_ms * 1e3 / (c.num_layers * repeat),
            "attention_timing": timing,
            "attention_batched_us": attn_ms * 1e3 / (c.num_layers * repeat),
            # the append (HBM-bound, 50 us or less) from the back-to-back batch: a per-call event
            # pair adds the few microseconds between the previous kernel's end and its start
            "append_us": med(acc["append"]) * 1e3 / c.num_layers,
            "stats_us": None if not acc["stats"] else med(acc["stats"]) * 1e3,
            "refreshes": st.run.cache.state()[2]}


def hbm_side_runs(c, append_us):
    """HBM-bound kernels at the workload's shape, each scored on 8 TB/s:
    rope_append from the batched pass; rebase and sink copy in a side stream of the same shape
    with a refresh every frame (every cached key rebased each step) and, where the workload has
    chunk embeddings, a threshold every cosine is below (every commit replaces a sink); the
    motion reduction over 1025 latent frames of 16x60x104."""
    import torch

    from rolling_kv_causal_amd import sdv2
    out = {}
    eb = 2 if c.dtype == "bf16" else 4
    kb = 1 if c.kv_fp8 else eb
    tensor = c.stream_batch * c.chunk_rows * c.num_heads * c.head_dim
    def entry(nbytes, us, note):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"bytes_per_call": int(nbytes), "us": round(us, 3), "gbs": round(gbs, 1),
                "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "how": note}
    # append: q, k, v read, q rotated back, k_rot and v^T written.  A workload of fewer than 8
    # layers is timed on a side stream of 8 layers of its shape, so that the events bracket
    # back-to-back launches rather than one launch's latency.
    how = "events around all layers' appends of a step, per layer"
    if c.num_layers < 8:
        st = Stepper(c.with_(num_layers=8, name=c.name + "_8l"), pool=1)
        for _ in range(c.sink_frames + c.window_frames + c.stream_batch + 1):
            st.step()
        app = []
        for _ in range(5):
            ev = events(("refresh", "append", "attention", "stats"))
            st.step(ev)
            torch.cuda.synchronize()
            app.append(ev["append"][0].elapsed_time(ev["append"][1]) * 1e3 / 8)
        del st
        torch.cuda.empty_cache()
        append_us = sorted(app)[2]
        how = "events around the appends of 8 layers of this shape (a side stream), per layer"
    side = c.with_(rope_refresh_period=1, name=c.name + "_side",
                   sink_threshold=(2.0 if c.embed_dim > 0 else None))
    st = Stepper(side, pool=1)
    fill = c.sink_frames + c.window_frames + c.stream_batch + 1
    for _ in range(fill):
        st.step()
    torch.cuda.synchronize()
    reb, stats = [], []
    for _ in range(5):
        ev = events(("refresh", "append", "attention", "stats"))
        st.step(ev)
        torch.cuda.synchronize()
        reb.append(ev["refresh"][0].elapsed_time(ev["refresh"][1]))
        if c.embed_dim > 0:
            stats.append(ev["stats"][0].elapsed_time(ev["stats"][1]))
    out["rope_append"] = entry(3 * tensor * eb + tensor * eb + 2 * tensor * kb, append_us, how)
    N = c.tokens
    nslots = c.window_frames + (0 if c.rope_pin_sinks else c.sink_frames)   # the slots a refresh turns
    pairs_bytes = c.num_layers * nslots * c.num_heads * N * c.rope_dim_t * kb
    out["rebase"] = entry(2 * pairs_bytes, sorted(reb)[2] * 1e3,
                          "refresh with T_reset = 1: every cached key's temporal pairs turned each step")
    if c.embed_dim > 0:
        L = sdv2.sdv2_cache_layout(Stepper._cfg(c))
        slot_bytes = L.slot_stride * L.elem_bytes
        out["sink_copy"] = entry(2 * 2 * c.num_layers * slot_bytes, sorted(stats)[2] * 1e3,
                                 "sdv2_sink_replace with every cosine below tau: statistics, decision and "
                                 "the copy of K and V of one frame into the sink, all layers")
    del st
    torch.cuda.empty_cache()
    # motion reduction over 1025 frames of the 480p latent shape
    n = 16 * 60 * 104
    F = 1025
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    frames = torch.randn((F, n), generator=g, device="cuda")
    dist = torch.empty(F - 1, dtype=torch.float64, device="cuda")
    ws = torch.empty(sdv2.sdv2_motion_workspace_size(F, n), dtype=torch.uint8, device="cuda")
    sdv2.sdv2_motion_l2(frames, F, n, dist, ws)
    ev = events(("m",))
    ev["m"][0].record()
    for _ in range(5):
        sdv2.sdv2_motion_l2(frames, F, n, dist, ws)
    ev["m"][1].record()
    torch.cuda.synchronize()
    out["motion_1025_frames"] = entry(F * n * 4, ev["m"][0].elapsed_time(ev["m"][1]) * 1e3 / 5,
                                      "sdv2_motion_l2 over 1025 frames of 16x60x104 fp32, mean of 5 calls")
    return out


def cpu_baseline(c, budget_s=12.0):
    """Oracle (float64 numpy) attention calls of the workload in steady state on host cores."""
    import numpy as np

    from oracle import stream as ost
    from synth import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    st = ost.OracleStream(c, layers=[0])
    steady = c.sink_frames + c.window_frames + c.stream_batch
    for s in range(steady):                        # fill the cache (bookkeeping + K/V decode)
        st.begin_step(s)
        _, k, v = inputs.qkv(c, s, 0, 0)
        st.end_step({0: (k, v)}, inputs.chunk_embedding(c, st.plan["commit"]) if (c.embed_dim and st.plan["commit"] is not None) else None)
    st.begin_step(steady)
    q, k, v = inputs.qkv(c, steady, 0, 0)
    calls, t_used = 0, 0.0
    rows = c.tokens                                # frame 0's query rows
    while t_used < budget_s and calls < 64:
        # one element's attention over the full key set, a slice of the rows at a time
        n = max(1, min(rows, 64 if c.num_heads > 12 else 128))
        r0 = (calls * n) % rows
        sel = np.arange(r0, min(rows, r0 + n))
        t0 = time.perf_counter()
        st.attend(0, 0, q, k, v, rows=sel)
        t_used += time.perf_counter() - t0
        calls += 1
        last_rows = len(sel)
    L = visible_keys(c, 0)                         # the sampled rows are frame 0's
    flops = calls * 4 * last_rows * c.num_heads * L * c.head_dim
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{calls} oracle attend calls of {last_rows} query rows x {c.num_heads} heads over "
                      f"{L} keys (layer 0, element 0, steady-state step {steady}), {t_used:.1f} s"}


def profile_fields(stem: str):
    """key: value lines of a committed rocprofv3 summary (profiles/<stem>.md), or None when it is
    missing or the attention sources changed since it was taken."""
    p = ROOT / "profiles" / f"{stem}.md"
    if not p.exists():
        return None
    fields = {}
    for ln in p.read_text().splitlines():
        if ":" in ln and not ln.startswith(("|", "#", " ", "`")) and ln.split(":", 1)[0].replace("_", "").isalnum():
            k, v = ln.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("attn_sources_sha256_16", "") != attn_source_hash():
        return None
    return fields


def load_traffic(workload: str):
    """HBM bytes per attention call (kernel + combine) from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source changed since it was taken."""
    f = profile_fields(f"attn_traffic_{workload}")
    return None if not f or "bytes_per_call" not in f else int(f["bytes_per_call"])


def calibration_copy(nbytes=1 << 30):
    """A plain elementwise copy of known size (read nbytes, write nbytes), larger than the
    256 MB Infinity Cache, used to scale the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"bench: calibration copy of {nbytes} bytes done")


def reference_rates(c, n=20, warmup=5):
    """Library rates on this GPU for context: torch.matmul bf16 (hipBLASLt) on square GEMMs and
    PyTorch's scaled_dot_product_attention (flash and memory-efficient backends) on the
    workload's attention shape (B x H heads, T'N queries, every visible key, one call per layer
    without the block-causal mask).  HIP events around n calls after warmup calls."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n * 1e-3

    out = {"gemm_bf16": {}, "sdpa_bf16": {}}
    for M in (8192, 16384):
        a = torch.randn(M, M, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(M, M, device="cuda", dtype=torch.bfloat16)
        t = timed(lambda: torch.matmul(a, b))
        out["gemm_bf16"][str(M)] = {"us": round(t * 1e6, 1), "tflops": round(2 * M ** 3 / t / 1e12, 1)}
        del a, b
    L = visible_keys(c, c.chunk_frames - 1)
    q = torch.randn(c.stream_batch, c.num_heads, c.chunk_rows, c.head_dim, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(c.stream_batch, c.num_heads, L, c.head_dim, device="cuda", dtype=torch.bfloat16)
    v = torch.randn_like(k)
    flops = 4.0 * c.stream_batch * c.num_heads * c.chunk_rows * L * c.head_dim
    for name, backend in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel(backend):
                t = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v))
            out["sdpa_bf16"][name] = {"us": round(t * 1e6, 1), "tflops": round(flops / t / 1e12, 1)}
        except RuntimeError as ex:                 # backend not built for this GPU
            out["sdpa_bf16"][name] = {"unavailable": str(ex)[:120]}
    out["sdpa_shape"] = {"batch": c.stream_batch, "heads": c.num_heads, "queries": c.chunk_rows, "keys": L,
                         "head_dim": c.head_dim}
    return out


SLO_GRID = [(1, 1), (2, 1), (4, 1), (8, 1), (1, 2), (2, 2), (4, 2), (1, 4), (2, 4), (1, 8)]


def slo_table(base, steps, warmup, target_fps, deadline_s):
    """Measured step latency L(B, T') of a workload over a (B, T') grid, the library's fit
    L = c0 + c1 B T' and its SLO-aware choice ([WT] SLO-aware batching scheduler)."""
    from rolling_kv_causal_amd import sdv2
    rows = []
    for B, T in SLO_GRID:
        c = base.with_(stream_batch=B, chunk_frames=T, num_chunks=max(64, 4 * B))
        g = run_gpu(c, steps, warmup)
        rows.append({"B": B, "T": T, "frames": B * T, "ms_per_step": round(g["ms_per_step"], 4),
                     "fps": round(B * T / (g["ms_per_step"] * 1e-3), 1)})
        log(f"bench: slo B={B} T'={T} {g['ms_per_step']:.3f} ms/step")
    c0, c1 = sdv2.sdv2_latency_fit([r["frames"] for r in rows], [r["ms_per_step"] * 1e-3 for r in rows])
    pick = sdv2.sdv2_slo_select(c0, c1, target_fps, deadline_s, 8, 8, 8)
    return {"workload": base.name, "grid": rows, "fit_c0_s": c0, "fit_c1_s_per_frame": c1,
            "target_fps": target_fps, "deadline_s": deadline_s, "choice": pick}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="wan14b_512_40layer_b4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm", action="store_true", help="skip the HBM-bound kernels' side runs")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run a 1 GiB plain copy first (scales HBM counters in rocprofv3 runs)")
    ap.add_argument("--slo-table", action="store_true",
                    help="measure L(B, T') over a grid on --workload, fit it and print the SLO-aware choice")
    ap.add_argument("--pin-sinks", action="store_true",
                    help="pinned-sink RoPE refresh: the refresh rebases only the window")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="OCP e4m3 KV cache (bf16 queries, scores and outputs)")
    ap.add_argument("--reference-rates", action="store_true",
                    help="print library rates on this GPU (bf16 GEMM, PyTorch SDPA on the workload's shape)")
    ap.add_argument("--no-reference-rates", action="store_true",
                    help="leave the library reference rates out of the line")
    ap.add_argument("--target-fps", type=float, default=30.0)
    ap.add_argument("--deadline-ms", type=float, default=100.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the head-sharded multi-GPU layout is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if os.environ.get("RANK", "0") != "0":
        sys.exit(0)

    from synth import configs
    c = configs.BY_NAME[args.workload]
    if args.pin_sinks:
        c = c.with_(rope_pin_sinks=True)
    if args.kv_fp8:
        c = c.with_(kv_fp8=True, name=c.name + "_kvfp8")
    if args.reference_rates:
        print(json.dumps({"workload": c.name, **reference_rates(c)}), flush=True)
        return
    if args.slo_table:
        print(json.dumps(slo_table(c, min(args.steps, 20), min(args.warmup, 5), args.target_fps,
                                   args.deadline_ms * 1e-3)), flush=True)
        return
    wn = workload_numbers(c)
    log(f"bench: workload {c.name}, {args.steps} timed steps after {args.warmup} warmup")
    if args.calibration_copy:
        calibration_copy()
    g = run_gpu(c, args.steps, args.warmup)
    log(f"bench: {g['ms_per_step']:.4f} ms/step, attention call {g['attention_us']:.2f} us")
    ms = g["ms_per_step"]
    step_flops = wn["flops_per_layer"] * c.num_layers
    value = step_flops / (ms * 1e-3) / 1e12
    attn_us = g["attention_us"]
    achieved = wn["flops_per_layer"] / (attn_us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if c.dtype == "bf16" else PEAK_FP32_TFLOPS
    prof = profile_fields(f"attn_trace_{c.name}")
    traffic = load_traffic(c.name)
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": "sdv2_chunk_attention (%s + combine_kernel)"
                      % ("attn_w64_kernel<e4m3 cache>" if c.kv_fp8 and c.head_dim == 128 else
                         "attn_w64_kernel" if c.dtype == "bf16" and c.head_dim == 128 else
                         "attn_bf16_kernel" if c.dtype == "bf16" else "attn_f32_kernel"),
            "flops_per_call": wn["flops_per_layer"], "avg_call_us": round(attn_us, 3),
            "timing": g["attention_timing"],
            "back_to_back_call_us": round(g["attention_batched_us"], 3)}
    if prof:
        roof["profile_call_us"] = prof.get("call_us")
        roof["profile_kernel_us"] = prof.get("kernel_us")
    out = {
        "metric": "sink+rolling-KV chunk attention TFLOP/s & HBM GB/s, % of roofline, 1 GPU",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": c.name, "layers": c.num_layers, "heads": c.num_heads,
                   "head_dim": c.head_dim, "tokens_per_frame": c.tokens, "sink_frames": c.sink_frames,
                   "window_frames": c.window_frames, "chunk_frames": c.chunk_frames,
                   "stream_batch": c.stream_batch, "keys_per_query": wn["keys"],
                   "rope_refresh_period": c.rope_refresh_period, "rope_pin_sinks": c.rope_pin_sinks,
                   "kv_cache": "e4m3" if c.kv_fp8 else c.dtype,
                   "sink_threshold": c.sink_threshold, "parallelism": "single GPU"},
        "roofline": roof,
        "chunk_attention_calls_per_s": round(c.num_layers / (ms * 1e-3), 1),
        "latent_frames_per_s": round(c.chunk_frames / (ms * 1e-3), 2),
        "attention_hbm_gbs": round(wn["attn_bytes_per_layer"] / (attn_us * 1e-6) / 1e9, 1),
        "append_us_per_layer": round(g["append_us"], 3),
        "stats_sink_us_per_step": None if g["stats_us"] is None else round(g["stats_us"], 3),
        "wall_s_timed": round(g["wall_s"], 4),
    }
    if not args.no_hbm:
        log("bench: HBM-bound kernels at the workload's shape")
        hbm = hbm_side_runs(c, g["append_us"])
        if prof and prof.get("combine_us") and float(prof.get("combine_bytes") or 0) > 0:
            us, nb = float(prof["combine_us"]), float(prof["combine_bytes"])
            hbm["combine"] = {"bytes_per_call": int(nb), "us": us, "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                              "frac_of_peak": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                              "how": f"rocprofv3 kernel trace, profiles/attn_trace_{c.name}.md "
                                     f"({prof.get('nsplit')} split partials read, output written)"}
        out["hbm_kernels"] = hbm
    if not args.no_reference_rates and c.dtype == "bf16":
        log("bench: library reference rates (bf16 GEMM, PyTorch SDPA) on this GPU")
        ref = reference_rates(c, n=10, warmup=3)
        gemm = ref["gemm_bf16"]["16384"]["tflops"]
        roof["measured_gemm_tflops"] = gemm
        roof["frac_of_measured_gemm"] = round(achieved / gemm, 4)
        out["reference_rates"] = ref
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on the host (bounded sample)")
        out["cpu_baseline"] = cpu_baseline(c)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
