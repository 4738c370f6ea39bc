"""Throughput of the sink + rolling-KV chunk-attention step on one MI355X.

A step is one pass of the whole hot path over one stream-batch of synthetic input: RoPE refresh
(when due), per layer the fused RoPE + append and the chunk attention, the commit of the
finished chunk, and - where the workload has them - the sink similarity decision + replacement
and the motion reduction of the newest latent frame.  Inputs are seeded device-resident random
tensors of the workload's shapes, generated before the timed region.

Prints one JSON line.  `value` is the attention work of the step (algorithmic FLOPs,
4 * nbatch * H * N * L * d per layer with L = (S + W + 1) * N keys) divided by the step time.
`roofline` scores the attention call (split-KV kernel + combine) against the bf16 MFMA peak
with its average duration measured by HIP events on the library's stream.  `cpu_baseline`
times the float64 oracle on a bounded sample of the same workload on the host cores.
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


ATTN_SOURCES = ("k_attention.hip", "k_attention_w64.hip", "attn_w64_asm.h", "attn_tiles.h")


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


def run_gpu(c, steps, warmup, pool=2):
    import torch

    from rolling_kv_causal_amd import sdv2
    from rolling_kv_causal_amd.stream import StreamRunner
    from synth import inputs

    torch.cuda.set_device(0)
    dev = "cuda"
    cfg = sdv2.config_of(c)
    big = 1 << 40                                  # an unbounded stream: steady state throughout
    run = StreamRunner(cfg, big, c.softmax_scale)
    dt = run.dtype
    B, N, H, D, Lyr = c.stream_batch, c.tokens, c.num_heads, c.head_dim, c.num_layers
    g = torch.Generator(device=dev)
    g.manual_seed(20261203)
    shape = (B, c.chunk_rows, H, D)
    sets = [[tuple((torch.randn(shape, generator=g, device=dev) *
                    (c.q_prescale if j == 0 else 1.0)).to(dt) for j in range(3))
             for _ in range(Lyr)] for _ in range(pool)]
    embeds = None
    if c.embed_dim > 0:
        embeds = torch.stack([torch.from_numpy(inputs.chunk_embedding(c, i)) for i in range(c.num_chunks)]).to(dev)
    motion = None
    if c.motion is not None:
        m = c.motion
        frames = torch.from_numpy(inputs.motion_frames(c)).to(dev)
        dist = torch.empty(m.frames, dtype=torch.float64, device=dev)
        mws = torch.empty(sdv2.sdv2_motion_workspace_size(2, m.elems), dtype=torch.uint8, device=dev)
        motion = (frames, dist, mws, m)

    events = {}

    def ev_pair(name):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        events.setdefault(name, []).append((a, b))
        return a, b

    def one_step(s, timed_parts=False):
        first, nb, commit, newest = run.plan(s)
        st = sets[s % pool]
        if timed_parts:
            a, b = ev_pair("refresh"); a.record()
        run.cache.refresh(newest)
        if timed_parts:
            b.record()
        for layer in range(Lyr):
            q, k, v = st[layer]
            if timed_parts:
                a, b = ev_pair("append"); a.record()
            run.cache.append(layer, first, nb, q[:nb], k[:nb], v[:nb])
            if timed_parts:
                b.record(); a, b = ev_pair("attention"); a.record()
            run.cache.attention(layer, nb, q[:nb], run.out[layer, :nb], run.scale)
            if timed_parts:
                b.record()
        if commit >= 0:
            if timed_parts:
                a, b = ev_pair("commit"); a.record()
            run.cache.commit(commit)
            if timed_parts:
                b.record()
            if embeds is not None:
                if timed_parts:
                    a, b = ev_pair("sink_replace"); a.record()
                last = (commit + 1) * c.chunk_frames - 1          # the chunk's last frame
                run.cache.sink_replace(last, embeds[commit % len(embeds)], sync=False)
                if timed_parts:
                    b.record()
            if motion is not None:
                frames, dist, mws, m = motion
                t = 1 + commit % (m.frames - 1)
                if timed_parts:
                    a, b = ev_pair("motion"); a.record()
                sdv2.sdv2_motion_l2(frames[t - 1:t + 1], 2, m.elems, dist, mws)
                if timed_parts:
                    b.record()

    fill = c.sink_frames + c.window_frames + B + 1
    s = 0
    for _ in range(fill + warmup):
        one_step(s)
        s += 1
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        one_step(s)
        s += 1
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    # second pass: per-call durations by HIP events on the same stream
    for _ in range(steps):
        one_step(s, timed_parts=True)
        s += 1
    torch.cuda.synchronize()
    parts = {k: sum(a.elapsed_time(b) for a, b in v) / len(v) * 1e3 for k, v in events.items()}
    counts = {k: len(v) for k, v in events.items()}
    return {"ms_per_step": ms_step, "wall_s": wall, "part_us": parts, "part_calls": counts,
            "refreshes": run.cache.state()[2]}


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


def load_traffic(workload: str):
    """HBM bytes per attention call (kernel + combine) from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source changed since it was taken."""
    p = ROOT / "profiles" / f"attn_traffic_{workload}.md"
    if not p.exists():
        return None
    fields = dict(ln.split(":", 1) for ln in p.read_text().splitlines()
                  if ln.startswith(("bytes_per_call:", "attn_sources_sha256_16:")))
    if fields.get("attn_sources_sha256_16", "").strip() != attn_source_hash():
        return None
    return int(fields["bytes_per_call"].strip())


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
    ap.add_argument("--workload", default="wan13b_512_1layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run a 1 GiB plain copy first (scales HBM counters in rocprofv3 runs)")
    ap.add_argument("--slo-table", action="store_true",
                    help="measure L(B, T') over a grid on --workload, fit it and print the SLO-aware choice")
    ap.add_argument("--pin-sinks", action="store_true",
                    help="pinned-sink RoPE refresh: the refresh rebases only the window")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="OCP e4m3 KV cache (bf16 queries, scores and outputs)")
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
    if args.slo_table:
        print(json.dumps(slo_table(c, min(args.steps, 20), min(args.warmup, 5), args.target_fps,
                                   args.deadline_ms * 1e-3)), flush=True)
        return
    wn = workload_numbers(c)
    log(f"bench: workload {c.name}, {args.steps} timed steps after {args.warmup} warmup")
    if args.calibration_copy:
        calibration_copy()
    g = run_gpu(c, args.steps, args.warmup)
    ms = g["ms_per_step"]
    step_flops = wn["flops_per_layer"] * c.num_layers
    value = step_flops / (ms * 1e-3) / 1e12
    attn_us = g["part_us"]["attention"]
    achieved = wn["flops_per_layer"] / (attn_us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if c.dtype == "bf16" else PEAK_FP32_TFLOPS
    traffic = load_traffic(c.name)
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
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": "sdv2_chunk_attention (%s + combine_kernel)"
                               % ("attn_w64_kernel<e4m3 cache>" if c.kv_fp8 and c.head_dim == 128 else
                                  "attn_w64_kernel" if c.dtype == "bf16" and c.head_dim == 128 else
                                  "attn_bf16_kernel"),
                     "flops_per_call": wn["flops_per_layer"], "avg_call_us": round(attn_us, 3)},
        "chunk_attention_calls_per_s": round(c.num_layers / (ms * 1e-3), 1),
        "latent_frames_per_s": round(c.chunk_frames / (ms * 1e-3), 2),
        "attention_hbm_gbs": round(wn["attn_bytes_per_layer"] / (attn_us * 1e-6) / 1e9, 1),
        "per_call_us": {k: round(v, 3) for k, v in g["part_us"].items()},
        "calls_per_step": {k: round(v / args.steps, 3) for k, v in g["part_calls"].items()},
        "wall_s_timed": round(g["wall_s"], 4),
    }
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on the host (bounded sample)")
        out["cpu_baseline"] = cpu_baseline(c)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
