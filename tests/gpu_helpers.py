"""Helpers shared by the GPU parity tests: device upload, HIP call, oracle, metrics."""
import sys

import numpy as np

import oracle
from diffusion_transformer_joint_amd import inputs as I

BF16_TOL = (2e-2, 5e-3)   # (max-abs, relative L2) against the fp64 oracle
FP8_TOL = (6e-2, 2e-2)
# e4m3 kernel against oracle.fp8_requant_attention (the same requantization in
# fp64): what is left is bf16 P, the fp16 rotation (an e4m3 rounding decision
# within 2^-11 of a midpoint may go the other way) and fp32 sums
FP8_REQUANT_TOL = (6e-2, 1e-2)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inp):
    import torch
    dev = torch.device("cuda:0")
    if inp.scales is None:
        cv = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        sc = None
    else:
        cv = lambda a: torch.from_numpy(a).to(dev)
        sc = torch.from_numpy(inp.scales).to(dev)
    return cv(inp.q), cv(inp.k), cv(inp.v), torch.from_numpy(inp.pos).to(dev), sc


def run_hip(inp, plan=None, mode="joint", out=None, pos=None):
    from diffusion_transformer_joint_amd.flux_attn import Plan
    import torch
    w = inp.workload
    q, k, v, p, sc = to_device(inp)
    if pos is not None:
        p = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).to("cuda:0")
    own = plan is None
    if own:
        plan = Plan(w.batch, w.heads, w.head_dim, w.tokens, dtype="fp8" if inp.scales is not None else "bf16")
    say(f"  HIP forward: {w.name} B={w.batch} N={w.tokens} H={w.heads} D={w.head_dim} mode={mode}")
    o = plan.forward(q, k, v, inp.segment_tokens, p, out=out, scales=sc, mode=mode)
    torch.cuda.synchronize()
    if own:
        plan.close()
    return o


def out_fp64(o):
    import torch
    return o.float().cpu().numpy().astype(np.float64)


def ref_full(inp, pos=None, mode="joint"):
    w = inp.workload
    q, k, v = oracle.inputs_to_fp64(inp)
    pos = inp.pos if pos is None else pos
    if mode == "joint":
        return oracle.joint_rope_attention(q, k, v, pos, w.axes_dim)
    return oracle.segment_local_rope_attention(q, k, v, pos, inp.segment_tokens, w.axes_dim)


def ref_rows(inp, rows):
    w = inp.workload
    q, k, v = oracle.inputs_to_fp64(inp)
    return oracle.joint_rope_attention_rows(q, k, v, inp.pos, w.axes_dim, rows)


def errors(got, ref):
    d = got - ref
    max_abs = float(np.max(np.abs(d)))
    rel_l2 = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel_l2


def assert_close(got, ref, tol, label=""):
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    ma, rl = errors(got, ref)
    say(f"  {label}: max-abs {ma:.3e} (tol {tol[0]:.0e})  rel-L2 {rl:.3e} (tol {tol[1]:.0e})")
    assert ma <= tol[0] and rl <= tol[1], f"{label}: max-abs {ma:.3e}, rel-L2 {rl:.3e}"
    return ma, rl


def sample_rows(n, seed=0, count=96):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 255, 256, 511, 512, 513, n // 2, n - 257, n - 256, n - 65, n - 64, n - 2, n - 1]
    rows = set(r for r in fixed if 0 <= r < n)
    rows.update(rng.integers(0, n, size=count).tolist())
    return np.array(sorted(rows))


def custom(name, heads, head_dim, segs, batch=1, sigma=0.5, fp8=False, seed=11):
    return I.custom_workload(name, batch, heads, head_dim, segs, sigma=sigma, fp8=fp8, seed=seed)
