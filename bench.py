#!/usr/bin/env python3
"""Benchmark: joint RoPE attention on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic input:
the RoPE angle table plus the joint attention kernel (RoPE fused into its Q/K
loads, online softmax, bf16 MFMA), through the C ABI.  The timed workload is the
1024^2 single-reference edit call: 512 text + 4,096 image + 4,096 reference
tokens (8,704), 24 heads, head_dim 128, bf16 Q/K/V ~ N(0, 0.25).  Inputs are
resident in HBM before timing starts.  The 4,608-token text-to-image call, the
66,048-token e4m3 call, the edit call in segment-local mode (each segment
attending to itself), one GPU's share of the edit call under 8-way head
sharding (3 heads, persistent split schedule), the edit call with cold
caches (a 512 MiB buffer written before each call, so Q, K, V come from HBM
rather than the 256 MB MALL), tile-sparse attention on edit-call tokens with
position-local attention (thresholds 0.1 and 0.01), the attention backward
(dq, dk, dv) of the edit call and, with --all, the 25,088-token call are
reported as extra fields of the same JSON line.  Kernel times are the mean of
the library's per-call HIP event pairs; the median and minimum are reported
beside it.

Rank 0 prints one JSON line.  Only one GPU is supported: the path shards over
heads with no communication inside the kernel; one GPU's share is among the
extra fields.
"""
import argparse
import hashlib
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "joint-attention TFLOP/s and % MFMA peak at 4,608 and 8,704 tokens, 1 GPU"
BF16_PEAK = 2516.6   # TFLOP/s, MI355X dense bf16 MFMA (published)
FP8_PEAK = 5033.2    # TFLOP/s, MI355X dense fp8 MFMA (published)
HBM_PEAK = 8000.0    # GB/s
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "attn_bf16": os.path.join(ROOT, "diffusion_transformer_joint_amd", "csrc", "attn_bf16.hip"),
    "attn_fp8": os.path.join(ROOT, "diffusion_transformer_joint_amd", "csrc", "attn_fp8.hip"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel):
    p = KERNEL_SOURCES[kernel]
    if not os.path.exists(p):
        return None
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "diffusion_transformer_joint_amd", "csrc")
    for f in (p, os.path.join(csrc, "attn_common.h"), os.path.join(csrc, "device_common.h")):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it matches the source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != source_sha(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measure(workload, steps, warmup, mode="joint"):
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    w = I.WORKLOADS[workload] if isinstance(workload, str) else workload
    inp = I.make_inputs(w)
    dev = torch.device("cuda:0")
    if inp.scales is None:
        cv = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        sc = None
    else:
        cv = lambda a: torch.from_numpy(a).to(dev)
        sc = torch.from_numpy(inp.scales).to(dev)
    q, k, v = cv(inp.q), cv(inp.k), cv(inp.v)
    pos = torch.from_numpy(inp.pos).to(dev)
    out = torch.empty((w.batch, w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens, dtype="fp8" if w.fp8 else "bf16")
    segs = w.segment_tokens
    for _ in range(warmup):
        plan.forward(q, k, v, segs, pos, out=out, scales=sc, mode=mode)
    torch.cuda.synchronize()
    plan.timing_enable(steps)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        plan.forward(q, k, v, segs, pos, out=out, scales=sc, mode=mode)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kernel_ms = plan.timing_read()
    plan.close()
    step_ms = e0.elapsed_time(e1) / steps
    if mode == "joint":
        flops = w.flops()
    else:  # each segment attends to itself
        flops = 4.0 * w.batch * w.heads * w.head_dim * sum(n * n for n in segs)
    kavg = sum(kernel_ms) / len(kernel_ms)
    return {
        "workload": w.name if mode == "joint" else f"{w.name} ({mode})", "mode": mode, "tokens": w.tokens, "heads": w.heads, "head_dim": w.head_dim, "batch": w.batch,
        "dtype": "fp8_e4m3" if w.fp8 else "bf16", "flops": flops,
        "ms_per_step": step_ms, "wall_ms_per_step": (t1 - t0) * 1e3 / steps,
        "kernel_ms_avg": kavg, "kernel_ms_min": min(kernel_ms), "kernel_ms_median": statistics.median(kernel_ms),
        "tflops": flops / (step_ms * 1e-3) / 1e12, "kernel_tflops": flops / (kavg * 1e-3) / 1e12,
    }


def measure_cold(workload, calls, flush_mib=512):
    """The joint call with cold caches: before each call a buffer of flush_mib
    MiB (twice the 256 MB MALL) is overwritten, so Q, K, V and the RoPE table
    come from HBM.  The library's event pair brackets the attention kernel
    only, so the flush is not timed."""
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    w = I.WORKLOADS[workload]
    inp = I.make_inputs(w)
    dev = torch.device("cuda:0")
    cv = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    q, k, v = cv(inp.q), cv(inp.k), cv(inp.v)
    pos = torch.from_numpy(inp.pos).to(dev)
    out = torch.empty((w.batch, w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    flush = torch.empty(flush_mib << 18, dtype=torch.float32, device=dev)
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens)
    plan.forward(q, k, v, w.segment_tokens, pos, out=out)
    torch.cuda.synchronize()
    plan.timing_enable(calls)
    for i in range(calls):
        flush.fill_(float(i))
        plan.forward(q, k, v, w.segment_tokens, pos, out=out)
    torch.cuda.synchronize()
    kernel_ms = plan.timing_read()
    plan.close()
    med = statistics.median(kernel_ms)
    return {"workload": f"{w.name} (cold caches: {flush_mib} MiB written before each call)", "tokens": w.tokens,
            "heads": w.heads, "head_dim": w.head_dim, "batch": w.batch, "dtype": "bf16", "flops": w.flops(),
            "calls": calls, "kernel_ms_median": med, "kernel_ms_min": min(kernel_ms),
            "kernel_tflops_median": w.flops() / (med * 1e-3) / 1e12, "frac_bf16_peak": w.flops() / (med * 1e-3) / 1e12 / BF16_PEAK}


def measure_sparse(workload, tau, steps, warmup):
    """Tile-sparse attention: the tile mask of threshold tau (built and timed
    once), then forward_sparse timed like forward."""
    import numpy as np
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    w = I.WORKLOADS[workload]
    inp = I.make_inputs(w)
    dev = torch.device("cuda:0")
    cv = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    q, k, v = cv(inp.q), cv(inp.k), cv(inp.v)
    pos = torch.from_numpy(inp.pos).to(dev)
    out = torch.empty((w.batch, w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens)
    segs = w.segment_tokens
    mask = plan.block_mask(q, k, segs, pos, tau)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        plan.block_mask(q, k, segs, pos, tau, mask=mask)
    e1.record()
    torch.cuda.synchronize()
    mask_ms = e0.elapsed_time(e1) / steps
    for _ in range(warmup):
        plan.forward_sparse(q, k, v, segs, pos, mask, out=out)
    torch.cuda.synchronize()
    plan.timing_enable(steps)
    e0.record()
    for _ in range(steps):
        plan.forward_sparse(q, k, v, segs, pos, mask, out=out)
    e1.record()
    torch.cuda.synchronize()
    kernel_ms = plan.timing_read()
    plan.close()
    step_ms = e0.elapsed_time(e1) / steps
    m = mask.cpu().numpy().astype(bool)
    n = w.tokens
    rows_per_qt = np.minimum(256, n - 256 * np.arange(m.shape[2]))
    keys_per_kt = np.minimum(64, n - 64 * np.arange(m.shape[3]))
    kept_pairs = float(np.einsum("bhqk,q,k->", m.astype(np.float64), rows_per_qt, keys_per_kt))
    kavg = sum(kernel_ms) / len(kernel_ms)
    dense_flops = w.flops()
    kept_flops = 4.0 * w.head_dim * kept_pairs
    return {
        "workload": f"{w.name} (tile-sparse, tau {tau})", "tokens": n, "heads": w.heads, "head_dim": w.head_dim,
        "batch": w.batch, "dtype": "bf16", "tau": tau, "kept_tile_fraction": float(m.mean()),
        "kept_pair_fraction": kept_pairs / (w.batch * w.heads * n * n),
        "mask_ms": mask_ms, "ms_per_step": step_ms, "kernel_ms_avg": kavg,
        "flops": kept_flops, "kernel_tflops": kept_flops / (kavg * 1e-3) / 1e12,
        "dense_equivalent_tflops": dense_flops / (kavg * 1e-3) / 1e12,
    }


def measure_backward(workload, steps, warmup):
    """Training forward (with the row log-sum-exp) and the backward, timed apart.
    Backward flops follow the usual count of five N x N x D products
    (recomputed S, dP, dV, dQ, dK): 2.5 x the forward's."""
    import numpy as np
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    w = I.WORKLOADS[workload]
    inp = I.make_inputs(w)
    dev = torch.device("cuda:0")
    cv = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
    q, k, v = cv(inp.q), cv(inp.k), cv(inp.v)
    pos = torch.from_numpy(inp.pos).to(dev)
    rng = np.random.default_rng(99)
    do = cv(I.f32_to_bf16_bits(rng.standard_normal(inp.q.shape, dtype=np.float32) * np.float32(0.5)))
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens)
    segs = w.segment_tokens
    out, lse = plan.forward_lse(q, k, v, segs, pos)
    for _ in range(warmup):
        plan.backward(q, k, v, out, do, lse, segs, pos)
    torch.cuda.synchronize()
    plan.timing_enable(steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        plan.backward(q, k, v, out, do, lse, segs, pos)
    e1.record()
    torch.cuda.synchronize()
    kernel_ms = plan.timing_read()
    plan.close()
    flops = 2.5 * w.flops()
    kavg = sum(kernel_ms) / len(kernel_ms)
    return {"workload": f"{w.name} (backward: dq, dk, dv)", "tokens": w.tokens, "heads": w.heads,
            "head_dim": w.head_dim, "batch": w.batch, "dtype": "bf16", "flops": flops,
            "ms_per_step": e0.elapsed_time(e1) / steps, "kernel_ms_avg": kavg,
            "kernel_tflops": flops / (kavg * 1e-3) / 1e12, "frac_bf16_peak": flops / (kavg * 1e-3) / 1e12 / BF16_PEAK}


def cpu_baseline(workload, rows_count):
    """The fp64 oracle, as it stands, on a bounded sample of query rows."""
    import numpy as np
    import oracle
    from diffusion_transformer_joint_amd import inputs as I

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    w = I.WORKLOADS[workload]
    inp = I.make_inputs(w)
    q, k, v = oracle.inputs_to_fp64(inp)
    rows = np.linspace(0, w.tokens - 1, rows_count).astype(np.int64)
    t0 = time.perf_counter()
    oracle.joint_rope_attention_rows(q, k, v, inp.pos, w.axes_dim, rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.batch * w.heads * len(rows) * w.tokens * w.head_dim
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 2), "gflops": round(flops / dt / 1e9, 1), "cpu": cpu,
            "sample": f"{len(rows)} of {w.tokens} query rows, all {w.heads} heads, full K/V "
                      f"(RoPE of all keys included), {workload}; {dt:.1f} s"}


def calibrate_copy(mb):
    """Plain device copy of a known size, for scaling HBM counters."""
    import torch
    n = mb * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 2,000 warm-up calls (~1.7 s) bring the GPU to its steady clock under this
    # load; 50 calls after 10 read 2-3% slower, still on the way up from idle.
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="edit1024")
    ap.add_argument("--all", action="store_true", help="also time the 25,088-token and FP8 workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8704)
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="only run a plain copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: joint attention shards over heads with no communication "
              "inside the kernel, so one GPU's share (3 of 24 heads) is timed among the extra fields; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy_mb:
        calibrate_copy(args.calibrate_copy_mb)
        return

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    main_run = measure(args.workload, args.steps, args.warmup)
    log(f"{args.workload}: {main_run['kernel_tflops']:.1f} TFLOP/s kernel, {main_run['ms_per_step']:.3f} ms/step")
    extra = []
    import dataclasses
    from diffusion_transformer_joint_amd import inputs as I
    share = dataclasses.replace(I.WORKLOADS["edit1024"], heads=3, name="edit1024_3heads",
                                description="one GPU's share (3 of 24 heads) of the 8,704-token edit call")
    others = [("t2i1024", "joint"), ("gen4k_fp8", "joint"), ("edit1024", "segment_local"), (share, "joint")] + \
        ([("gen2048r2", "joint")] if args.all else [])
    xs, xw = min(args.steps, 50), min(args.warmup, 10)  # extra fields: short runs
    for name, mode in others:
        if name == args.workload and mode == "joint":
            continue
        r = measure(name, max(5, xs // 5) if name == "gen4k_fp8" else max(5, xs // 2),
                    max(2, xw // 2), mode=mode)
        r["frac_bf16_peak"] = r["kernel_tflops"] / BF16_PEAK
        if r["dtype"] != "bf16":
            # QK^T runs at the fp8 rate, PV at the bf16 rate (P is kept in bf16)
            r["frac_fp8_peak"] = r["kernel_tflops"] / FP8_PEAK
            r["frac_mixed_ceiling"] = r["kernel_tflops"] / (2.0 / (1.0 / FP8_PEAK + 1.0 / BF16_PEAK))
        extra.append(r)
        log(f"{r['workload']}: {r['kernel_tflops']:.1f} TFLOP/s kernel")
    r = measure_cold(args.workload, max(5, xs // 5))
    extra.append(r)
    log(f"{r['workload']}: {r['kernel_tflops_median']:.1f} TFLOP/s kernel (median)")
    r = measure_backward("edit1024", max(5, xs // 5), max(2, xw // 2))
    extra.append(r)
    log(f"{r['workload']}: {r['kernel_ms_avg']:.3f} ms, {r['kernel_tflops']:.1f} TFLOP/s (2.5 x forward flops)")
    for tau in (0.1, 0.01):
        r = measure_sparse("edit1024_local", tau, max(5, xs // 2), max(2, xw // 2))
        r["speedup_vs_dense_edit1024"] = main_run["kernel_ms_avg"] / r["kernel_ms_avg"]
        extra.append(r)
        log(f"{r['workload']}: kept {r['kept_pair_fraction']:.2f} of pairs, {r['kernel_ms_avg']:.3f} ms, "
            f"{r['kernel_tflops']:.1f} TFLOP/s on kept pairs, x{r['speedup_vs_dense_edit1024']:.2f} vs dense")

    kernel = "attn_bf16"
    traffic = recorded_traffic(kernel, args.workload)
    achieved = main_run["kernel_tflops"]
    line = {
        "metric": METRIC,
        "value": round(main_run["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_run["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: 1024^2 single-reference edit call, 512 text + 4096 image + "
                               f"4096 reference tokens", "batch": main_run["batch"], "seq_len": main_run["tokens"],
                   "heads": main_run["heads"], "head_dim": main_run["head_dim"], "parallelism": "none (1 GPU)"},
        "frac_bf16_peak": round(main_run["tflops"] / BF16_PEAK, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK, 4), "traffic": traffic,
                     "kernel": "attn_fwd_bf16_kernel<128, false>", "kernel_ms_avg": round(main_run["kernel_ms_avg"], 4),
                     "kernel_ms_median": round(main_run["kernel_ms_median"], 4),
                     "flops_per_launch": main_run["flops"]},
        "extra": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in extra],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
