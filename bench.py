#!/usr/bin/env python3
"""Benchmark: joint RoPE attention on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over one batch of synthetic input:
the RoPE angle table plus the joint attention kernel (RoPE fused into its Q/K
loads, online softmax, bf16 MFMA) and the exact merge of its split pieces,
through the C ABI.  The timed workload is the 1024^2 single-reference edit
call: 512 text + 4,096 image + 4,096 reference tokens (8,704), 24 heads,
head_dim 128, bf16 Q/K/V ~ N(0, 0.25).  Inputs are resident in HBM before
timing starts.  W untimed calls precede exactly K timed ones, bracketed by
device synchronisations.

Extra fields of the same JSON line (each with its own timing):
  * the other four workloads: 4,608-token text-to-image call (same K and W as
    the headline), the 80-token tiny call, the 25,088-token 2048^2 call with
    two references, the 66,048-token e4m3 call;
  * one GPU's share of the edit call when its heads are split over 8, 4 or 2
    GPUs (3, 6 and 12 heads);
  * the 3-head share and the edit call captured once into a HIP graph and
    replayed (one graph launch per call instead of three kernel launches);
  * the edit call in segment-local mode, with cold caches, its backward, and
    tile-sparse attention on edit-call tokens with position-local attention.
Per workload: seed, SHA-256 of the input bytes, attention-kernel time (mean of
the library's per-call HIP event pairs on the launch stream; median and
minimum beside it), kernel plus merge time, and the average shader clock the
kernel's workgroups ran at (s_memtime / s_memrealtime, measured inside the
kernel).  The cpu_baseline leg times the fp64 oracle on the whole edit call
and, from the same oracle, reports max-abs and relative L2 error of each
workload's GPU output (whole tensor at 80, 4,608 and 8,704 tokens, sampled
rows beyond).

Rank 0 prints one JSON line.  Only one GPU is supported: the path shards over
heads with no communication inside the kernel; one GPU's share is among the
extra fields.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "joint-attention TFLOP/s and % MFMA peak at 4,608 and 8,704 tokens, 1 GPU"
BF16_PEAK = 2516.6   # TFLOP/s, MI355X dense bf16 MFMA (published)
FP8_PEAK = 5033.2    # TFLOP/s, MI355X dense fp8 MFMA (published)
MIXED_CEIL = 2.0 / (1.0 / FP8_PEAK + 1.0 / BF16_PEAK)  # QK^T at the fp8 rate, PV at the bf16 rate
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "diffusion_transformer_joint_amd", "csrc")
KERNEL_SOURCES = {
    "attn_bf16": os.path.join(CSRC, "attn_bf16.hip"),
    "attn_fp8": os.path.join(CSRC, "attn_fp8.hip"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kernel):
    p = KERNEL_SOURCES[kernel]
    if not os.path.exists(p):
        return None
    h = hashlib.sha256()
    for f in (p, os.path.join(CSRC, "attn_common.h"), os.path.join(CSRC, "device_common.h")):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it matches the source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != source_sha(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _device_inputs(inp):
    import torch
    dev = torch.device("cuda:0")
    if inp.scales is None:
        cv = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
        sc = None
    else:
        cv = lambda a: torch.from_numpy(a).to(dev)
        sc = torch.from_numpy(inp.scales).to(dev)
    return cv(inp.q), cv(inp.k), cv(inp.v), torch.from_numpy(inp.pos).to(dev), sc


def measure(w, steps, warmup, mode="joint", keep_output=False):
    """Time `steps` forward calls of workload w after `warmup` untimed ones."""
    import numpy as np
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    inp = I.make_inputs(w)
    q, k, v, pos, sc = _device_inputs(inp)
    out = torch.empty((w.batch, w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda:0")
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
    tm = plan.timing_read(with_merge=True)
    plan.close()
    step_ms = e0.elapsed_time(e1) / steps
    if mode == "joint":
        flops = w.flops()
    else:  # each segment attends to itself
        flops = 4.0 * w.batch * w.heads * w.head_dim * sum(n * n for n in segs)
    ka, kt = tm["attn_ms"], tm["total_ms"]
    kavg, tavg = sum(ka) / len(ka), sum(kt) / len(kt)
    r = {
        "workload": w.name if mode == "joint" else f"{w.name} ({mode})", "mode": mode, "tokens": w.tokens,
        "heads": w.heads, "head_dim": w.head_dim, "batch": w.batch, "dtype": "fp8_e4m3" if w.fp8 else "bf16",
        "seed": w.seed, "input_sha256": inp.sha256(), "steps": steps, "warmup": warmup, "flops": flops,
        "ms_per_step": step_ms, "wall_ms_per_step": (t1 - t0) * 1e3 / steps,
        "kernel_ms_avg": kavg, "kernel_ms_min": min(ka), "kernel_ms_median": statistics.median(ka),
        "kernel_plus_merge_ms_avg": tavg, "clock_mhz": tm["clock_mhz"],
        "tflops": flops / (step_ms * 1e-3) / 1e12, "kernel_tflops": flops / (kavg * 1e-3) / 1e12,
        "kernel_plus_merge_tflops": flops / (tavg * 1e-3) / 1e12,
    }
    r["frac_bf16_peak"] = r["kernel_tflops"] / BF16_PEAK
    if w.fp8:
        r["frac_fp8_peak"] = r["kernel_tflops"] / FP8_PEAK
        r["frac_mixed_ceiling"] = r["kernel_tflops"] / MIXED_CEIL
    output = out.view(torch.int16).cpu().numpy().view(np.uint16) if keep_output else None
    return r, inp, output


def measure_graph(w, steps, warmup):
    """The joint call captured once into a HIP graph (RoPE table, attention,
    merge) and replayed: `warmup` untimed replays, then `steps` timed ones
    (events on the replay stream).  Launch work per call is one graph launch."""
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    inp = I.make_inputs(w)
    q, k, v, pos, sc = _device_inputs(inp)
    out = torch.empty((w.batch, w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda:0")
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens, dtype="fp8" if w.fp8 else "bf16")
    plan.forward(q, k, v, w.segment_tokens, pos, out=out, scales=sc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.forward(q, k, v, w.segment_tokens, pos, out=out, scales=sc)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    del g
    plan.close()
    return {"workload": f"{w.name} (one call captured in a HIP graph, replayed)", "tokens": w.tokens,
            "heads": w.heads, "head_dim": w.head_dim, "batch": w.batch, "dtype": "fp8_e4m3" if w.fp8 else "bf16",
            "flops": w.flops(), "steps": steps, "warmup": warmup, "ms_per_step": step_ms,
            "tflops": w.flops() / (step_ms * 1e-3) / 1e12}


def measure_cold(w, calls, flush_mib=512):
    """The joint call with cold caches: before each call a buffer of flush_mib
    MiB (twice the 256 MB MALL) is overwritten, so Q, K, V and the RoPE table
    come from HBM.  The library's event pair brackets the attention kernel
    only, so the flush is not timed."""
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    inp = I.make_inputs(w)
    q, k, v, pos, _ = _device_inputs(inp)
    out = torch.empty((w.batch, w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda:0")
    flush = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda:0")
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens)
    plan.forward(q, k, v, w.segment_tokens, pos, out=out)
    torch.cuda.synchronize()
    plan.timing_enable(calls)
    for i in range(calls):
        flush.fill_(float(i))
        plan.forward(q, k, v, w.segment_tokens, pos, out=out)
    torch.cuda.synchronize()
    tm = plan.timing_read(with_merge=True)
    plan.close()
    med = statistics.median(tm["attn_ms"])
    return {"workload": f"{w.name} (cold caches: {flush_mib} MiB written before each call)", "tokens": w.tokens,
            "heads": w.heads, "head_dim": w.head_dim, "batch": w.batch, "dtype": "bf16", "flops": w.flops(),
            "calls": calls, "kernel_ms_median": med, "kernel_ms_min": min(tm["attn_ms"]),
            "clock_mhz": tm["clock_mhz"], "kernel_tflops_median": w.flops() / (med * 1e-3) / 1e12,
            "frac_bf16_peak": w.flops() / (med * 1e-3) / 1e12 / BF16_PEAK}


def measure_sparse(w, tau, steps, warmup, rule="bound"):
    """Tile-sparse attention: the tile mask of threshold tau by `rule` (timed
    over `steps` builds), then forward_sparse timed like forward; the
    deviation of its output from the dense forward on the same inputs."""
    import numpy as np
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    inp = I.make_inputs(w)
    q, k, v, pos, _ = _device_inputs(inp)
    out = torch.empty((w.batch, w.tokens, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda:0")
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens)
    segs = w.segment_tokens
    mask = plan.block_mask(q, k, segs, pos, tau, rule=rule)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        plan.block_mask(q, k, segs, pos, tau, mask=mask, rule=rule)
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
    dense = plan.forward(q, k, v, segs, pos)
    torch.cuda.synchronize()
    plan.close()
    diff = (out.float() - dense.float())
    dev_rel = float(torch.linalg.vector_norm(diff) / torch.linalg.vector_norm(dense.float()))
    dev_max = float(diff.abs().max())
    step_ms = e0.elapsed_time(e1) / steps
    m = mask.cpu().numpy().astype(bool)
    n = w.tokens
    rows_per_qt = np.minimum(256, n - 256 * np.arange(m.shape[2]))
    keys_per_kt = np.minimum(64, n - 64 * np.arange(m.shape[3]))
    kept_pairs = float(np.einsum("bhqk,q,k->", m.astype(np.float64), rows_per_qt, keys_per_kt))
    kavg = sum(kernel_ms) / len(kernel_ms)
    kept_flops = 4.0 * w.head_dim * kept_pairs
    return {
        "workload": f"{w.name} (tile-sparse, {rule} rule, tau {tau})", "tokens": n, "heads": w.heads,
        "head_dim": w.head_dim, "batch": w.batch, "dtype": "bf16", "rule": rule, "tau": tau,
        "kept_tile_fraction": float(m.mean()), "kept_pair_fraction": kept_pairs / (w.batch * w.heads * n * n),
        "mask_ms": mask_ms, "ms_per_step": step_ms, "kernel_ms_avg": kavg,
        "flops": kept_flops, "kernel_tflops": kept_flops / (kavg * 1e-3) / 1e12,
        "dense_equivalent_tflops": w.flops() / (kavg * 1e-3) / 1e12,
        "deviation_from_dense_rel_l2": dev_rel, "deviation_from_dense_max_abs": dev_max,
    }, inp, m


def measure_backward(w, steps, warmup):
    """Training forward (with the row log-sum-exp) and the backward, timed apart.
    Backward flops follow the usual count of five N x N x D products
    (recomputed S, dP, dV, dQ, dK): 2.5 x the forward's."""
    import numpy as np
    import torch
    from diffusion_transformer_joint_amd import inputs as I
    from diffusion_transformer_joint_amd.flux_attn import Plan

    inp = I.make_inputs(w)
    q, k, v, pos, _ = _device_inputs(inp)
    rng = np.random.default_rng(99)
    do = torch.from_numpy(I.f32_to_bf16_bits(rng.standard_normal(inp.q.shape, dtype=np.float32) *
                                             np.float32(0.5)).view("int16")).view(torch.bfloat16).to("cuda:0")
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


def _bf16_out_fp64(bits):
    import numpy as np
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def cpu_baseline(main_inp, main_out, checks, sparse_checks):
    """The cpu_baseline leg: the fp64 oracle, as it stands, timed on the whole
    headline call (its output also gives the headline's error), then the same
    oracle on the other workloads' outputs (whole tensors up to 4,608 tokens,
    sampled rows beyond) for their error fields."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1

    def errors(got, ref):
        d = got - ref
        return {"max_abs": float(np.abs(d).max()), "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref))}

    w = main_inp.workload
    q, k, v = oracle.inputs_to_fp64(main_inp)
    t0 = time.perf_counter()
    ref = oracle.joint_rope_attention(q, k, v, main_inp.pos, w.axes_dim)
    dt = time.perf_counter() - t0
    main_err = dict(errors(_bf16_out_fp64(main_out), ref), rows="all")
    del q, k, v, ref
    flops = w.flops()
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 2), "gflops": round(flops / dt / 1e9, 1), "cpu": cpu,
            "sample": f"the whole {w.name} call: all {w.tokens} query rows, all {w.heads} heads, full K/V "
                      f"(RoPE of all keys included); {dt:.1f} s"}
    log(f"cpu_baseline: oracle {dt:.1f} s on {cores} threads; {w.name} max-abs {main_err['max_abs']:.3e} "
        f"rel-L2 {main_err['rel_l2']:.3e}")
    out_err = {}
    for name, (inp, got_bits) in checks.items():
        wl = inp.workload
        qq, kk, vv = oracle.inputs_to_fp64(inp)
        got = _bf16_out_fp64(got_bits)
        if wl.tokens <= 4608:
            e = dict(errors(got, oracle.joint_rope_attention(qq, kk, vv, inp.pos, wl.axes_dim)), rows="all")
        else:
            n = wl.tokens
            rows = np.unique(np.concatenate([np.linspace(0, n - 1, 192).astype(np.int64),
                                             np.random.default_rng(wl.seed).integers(0, n, 64)]))
            refr = oracle.joint_rope_attention_rows(qq, kk, vv, inp.pos, wl.axes_dim, rows)
            e = dict(errors(got[:, rows], refr), rows=f"{len(rows)} sampled of {n}")
        out_err[name] = e
        log(f"  oracle check {name}: max-abs {e['max_abs']:.3e} rel-L2 {e['rel_l2']:.3e} ({e['rows']})")
    # score-bound sparse runs: the proven distance from dense attention,
    # delta_i (max V - min V) per element, with delta_i the dense softmax mass
    # of row i's skipped keys, against the oracle's sparse-vs-dense distance
    for name, (inp, mask) in sparse_checks.items():
        wl = inp.workload
        qq, kk, vv = oracle.inputs_to_fp64(inp)
        n = wl.tokens
        rows = np.unique(np.linspace(0, n - 1, 48).astype(np.int64))
        delta = oracle.skipped_mass(qq, kk, inp.pos, wl.axes_dim, mask)
        bound = oracle.dense_error_bound(delta, vv)[:, rows]
        dense = oracle.joint_rope_attention_rows(qq, kk, vv, inp.pos, wl.axes_dim, rows)
        sparse = oracle.block_sparse_attention(qq, kk, vv, inp.pos, wl.axes_dim, mask, rows=rows)
        dev = np.abs(sparse - dense)
        out_err[name] = {"rows": f"{len(rows)} sampled of {n}", "max_skipped_mass": float(delta.max()),
                         "mean_skipped_mass": float(delta.mean()),
                         "oracle_deviation_rel_l2": float(np.linalg.norm(dev) / np.linalg.norm(dense)),
                         "bound_rel_l2": float(np.linalg.norm(bound) / np.linalg.norm(dense)),
                         "deviation_within_bound": bool((dev <= bound + 1e-12).all())}
        log(f"  oracle check {name}: skipped mass max {delta.max():.3e}, deviation rel-L2 "
            f"{out_err[name]['oracle_deviation_rel_l2']:.3e} <= bound rel-L2 {out_err[name]['bound_rel_l2']:.3e}: "
            f"{out_err[name]['deviation_within_bound']}")
    return base, main_err, out_err


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


def rnd(r):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 2,000 warm-up calls (~1.7 s) bring the GPU to its steady clock under this
    # load; short runs read slower, still on the way up from idle.
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--only-headline", action="store_true", help="time the edit call only (profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="only run a plain copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: joint attention shards over heads with no communication "
              "inside the kernel, so one GPU's share (3, 6 or 12 of 24 heads) is timed among the extra "
              "fields; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy_mb:
        calibrate_copy(args.calibrate_copy_mb)
        return

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from diffusion_transformer_joint_amd import inputs as I

    K, W = args.steps, args.warmup
    WL = I.WORKLOADS
    main_run, main_inp, main_out = measure(WL["edit1024"], K, W, keep_output=True)
    log(f"edit1024: {main_run['kernel_tflops']:.1f} TFLOP/s kernel, {main_run['ms_per_step']:.3f} ms/step, "
        f"clock {main_run['clock_mhz']:.0f} MHz")
    extra, checks, sparse_checks = [], {}, {}
    if not args.only_headline:
        share = lambda h: dataclasses.replace(WL["edit1024"], heads=h, name=f"edit1024_{h}heads",
                                              description=f"one GPU's share ({h} of 24 heads) of the edit call")
        runs = [
            (WL["t2i1024"], K, W, "joint"),                       # named in the metric: same counts
            (WL["tiny"], K, W, "joint"),
            (WL["gen2048r2"], min(K, 100), min(W, 200), "joint"),
            (WL["gen4k_fp8"], min(K, 20), min(W, 5), "joint"),
            (share(3), min(K, 200), min(W, 400), "joint"),
            (share(6), min(K, 200), min(W, 400), "joint"),
            (share(12), min(K, 200), min(W, 400), "joint"),
            (WL["edit1024"], min(K, 100), min(W, 200), "segment_local"),
        ]
        for w, k_, w_, mode in runs:
            r, inp, out = measure(w, k_, w_, mode=mode, keep_output=(mode == "joint"))
            if mode == "joint":
                checks[r["workload"]] = (inp, out)
            extra.append(r)
            log(f"{r['workload']}: {r['kernel_tflops']:.1f} TFLOP/s kernel ({r['frac_bf16_peak']:.3f} of bf16 peak), "
                f"clock {r['clock_mhz']:.0f} MHz")
        for w, k_, w_ in ((share(3), min(K, 200), min(W, 400)), (WL["edit1024"], min(K, 100), min(W, 200))):
            r = measure_graph(w, k_, w_)
            extra.append(r)
            log(f"{r['workload']}: {r['ms_per_step'] * 1e3:.1f} us/step, {r['tflops']:.1f} TFLOP/s per step")
        r = measure_cold(WL["edit1024"], max(5, min(K, 20)))
        extra.append(r)
        log(f"{r['workload']}: {r['kernel_tflops_median']:.1f} TFLOP/s kernel (median)")
        r = measure_backward(WL["edit1024"], max(5, min(K, 20)), max(2, min(W, 5)))
        extra.append(r)
        log(f"{r['workload']}: {r['kernel_ms_avg']:.3f} ms, {r['kernel_tflops']:.1f} TFLOP/s (2.5 x forward flops)")
        for rule, tau in (("bound", 0.1), ("bound", 0.01), ("pooled", 0.1), ("pooled", 0.01)):
            r, sinp, smask = measure_sparse(WL["edit1024_local"], tau, max(5, min(K, 25)), max(2, min(W, 5)), rule)
            r["speedup_vs_dense_edit1024"] = main_run["kernel_ms_avg"] / r["kernel_ms_avg"]
            r["speedup_with_mask_vs_dense_edit1024"] = main_run["kernel_ms_avg"] / (r["kernel_ms_avg"] + r["mask_ms"])
            extra.append(r)
            if rule == "bound":
                sparse_checks[r["workload"]] = (sinp, smask)
            log(f"{r['workload']}: kept {r['kept_pair_fraction']:.2f} of pairs, mask {r['mask_ms']:.3f} ms, "
                f"attention {r['kernel_ms_avg']:.3f} ms (x{r['speedup_vs_dense_edit1024']:.2f} vs dense), "
                f"deviation from dense rel-L2 {r['deviation_from_dense_rel_l2']:.2e}")

    traffic = recorded_traffic("attn_bf16", "edit1024")
    achieved = main_run["kernel_tflops"]
    line = {
        "metric": METRIC,
        "value": round(main_run["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(main_run["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "edit1024: 1024^2 single-reference edit call, 512 text + 4096 image + "
                               "4096 reference tokens", "batch": main_run["batch"], "seq_len": main_run["tokens"],
                   "heads": main_run["heads"], "head_dim": main_run["head_dim"], "parallelism": "none (1 GPU)",
                   "seed": main_run["seed"], "input_sha256": main_run["input_sha256"]},
        "frac_bf16_peak": round(main_run["tflops"] / BF16_PEAK, 4),
        "clock_mhz": round(main_run["clock_mhz"], 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK, 4), "traffic": traffic,
                     "kernel": "attn_fwd_bf16_kernel<128, false>", "kernel_ms_avg": round(main_run["kernel_ms_avg"], 4),
                     "kernel_ms_median": round(main_run["kernel_ms_median"], 4),
                     "flops_per_launch": main_run["flops"],
                     "kernel_plus_merge_ms_avg": round(main_run["kernel_plus_merge_ms_avg"], 4),
                     "frac_with_merge": round(main_run["kernel_plus_merge_tflops"] / BF16_PEAK, 4)},
        "extra": [rnd(r) for r in extra],
    }
    if not args.no_cpu_baseline:
        base, main_err, out_err = cpu_baseline(main_inp, main_out, checks, sparse_checks)
        line["cpu_baseline"] = base
        line["error_vs_oracle"] = main_err
        for r in line["extra"]:
            if r["workload"] in out_err:
                r["error_vs_oracle"] = out_err[r["workload"]]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
