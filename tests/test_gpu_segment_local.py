"""GPU parity of segment-local mode (each token attends only inside its segment).

Segment-local attention is the separate-stream stage before the joint blocks
("FLUX.3 Image Klein Brings 2-Second AI Image Generation to Diffusers",
Summary).  The oracle is the joint formula applied to each segment on its own
(oracle.segment_local_rope_attention), with the tokens' own position ids.
"""
import numpy as np
import pytest

import oracle
from diffusion_transformer_joint_amd import inputs as I

from gpu_helpers import (BF16_TOL, FP8_TOL, assert_close, custom, out_fp64, ref_full, run_hip, sample_rows,
                         say)

pytestmark = pytest.mark.gpu

S = I.Segment

CASES = [
    ("seg_small", 1, 2, 128, [S("text", 40), S("image", 8, 8), S("ref", 6, 6, 1)]),
    ("seg_ragged_empty", 1, 3, 128, [S("text", 100), S("text", 0), S("image", 17, 13), S("ref", 5, 7, 1)]),
    ("seg_b2", 2, 2, 128, [S("text", 77), S("image", 12, 20)]),
    ("seg_d64", 1, 3, 64, [S("text", 16), S("image", 8, 8), S("ref", 8, 8, 1), S("ref", 8, 8, 2)]),
    ("seg_one_token", 1, 2, 128, [S("text", 1), S("image", 9, 9)]),
]


@pytest.mark.parametrize("name,batch,heads,d,segs", CASES, ids=[c[0] for c in CASES])
def test_segment_local_full(name, batch, heads, d, segs):
    inp = I.make_inputs(custom(name, heads, d, segs, batch=batch, sigma=1.0))
    got = out_fp64(run_hip(inp, mode="segment_local"))
    assert_close(got, ref_full(inp, mode="segment_local"), BF16_TOL, name)


def test_segment_local_differs_from_joint_and_single_segment_equals_joint():
    segs = [S("text", 64), S("image", 12, 12)]
    inp = I.make_inputs(custom("seg_vs_joint", 2, 128, segs, sigma=1.0))
    loc = out_fp64(run_hip(inp, mode="segment_local"))
    joint = out_fp64(run_hip(inp, mode="joint"))
    assert np.linalg.norm(loc - joint) / np.linalg.norm(joint) > 0.1
    one = I.make_inputs(custom("seg_single", 2, 128, [S("text", 300)], sigma=1.0))
    a = run_hip(one, mode="segment_local")
    b = run_hip(one, mode="joint")
    assert (a == b).all(), "one segment, segment-local vs joint"


def _segment_rows_ref(inp, rows):
    """Oracle rows of segment-local attention, one segment at a time."""
    w = inp.workload
    q, k, v = oracle.inputs_to_fp64(inp)
    bounds = np.cumsum([0] + list(inp.segment_tokens))
    out = np.zeros((w.batch, len(rows), w.heads, w.head_dim))
    for s in range(len(inp.segment_tokens)):
        lo, hi = bounds[s], bounds[s + 1]
        sel = [i for i, r in enumerate(rows) if lo <= r < hi]
        if not sel:
            continue
        local = np.asarray([rows[i] - lo for i in sel], dtype=np.int64)
        o = oracle.joint_rope_attention_rows(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], inp.pos[lo:hi], w.axes_dim, local)
        out[:, sel] = o
    return out


def test_edit1024_segment_local_sampled_rows():
    # 24 heads x (512 text + 4,096 image + 4,096 reference) tokens, each segment
    # attending to itself: three launches with split K/V schedules of their own.
    inp = I.make_inputs(I.WORKLOADS["edit1024"])
    got = out_fp64(run_hip(inp, mode="segment_local"))
    assert np.all(np.isfinite(got))
    rows = np.unique(np.concatenate([sample_rows(inp.workload.tokens, seed=5, count=36), [0, 511, 512, 4607, 4608, 8703]]))
    assert_close(got[:, rows], _segment_rows_ref(inp, rows), BF16_TOL, f"edit1024 segment-local ({len(rows)} rows)")


def test_fp8_segment_local():
    inp = I.make_inputs(custom("seg_fp8", 3, 128, [S("text", 60), S("image", 16, 16)], fp8=True))
    got = out_fp64(run_hip(inp, mode="segment_local"))
    assert_close(got, ref_full(inp, mode="segment_local"), FP8_TOL, "fp8 segment-local")


def test_segment_local_many_segments():
    # 18 non-empty segments (two launches of at most 16 token ranges each),
    # ragged lengths from 1 to 300 tokens and two empty segments.
    from diffusion_transformer_joint_amd.flux_attn import Plan
    lens = [300, 5, 0, 17, 64, 1, 129, 33, 0, 256, 7, 90, 2, 45, 3, 12, 70, 200, 9, 31]
    segs = [S("text", n) for n in lens]
    inp = I.make_inputs(custom("seg_many", 2, 128, segs, sigma=1.0))
    w = inp.workload
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens, max_segments=len(lens))
    try:
        got = out_fp64(run_hip(inp, plan=plan, mode="segment_local"))
    finally:
        plan.close()
    assert_close(got, ref_full(inp, mode="segment_local"), BF16_TOL, "seg_many")


def test_segment_local_last_launch_persistent_at_offset(monkeypatch):
    # 17 non-empty segments: the first launch takes the 16 longest, the second
    # holds only the shortest (100 tokens), which starts at token 600, not 0.
    # A single-range launch may take the persistent split; forcing it makes
    # the merge of the cut tile write that segment's rows at their offset.
    from diffusion_transformer_joint_amd.flux_attn import Plan
    monkeypatch.setenv("FLUX_ATTN_SCHEDULE", "persistent")
    lens = [300, 300, 100] + [130 + 10 * i for i in range(14)]
    segs = [S("text", n) for n in lens]
    inp = I.make_inputs(custom("seg_tail", 2, 128, segs, sigma=1.0))
    w = inp.workload
    plan = Plan(w.batch, w.heads, w.head_dim, w.tokens, max_segments=len(lens))
    try:
        got = out_fp64(run_hip(inp, plan=plan, mode="segment_local"))
    finally:
        plan.close()
    assert_close(got, ref_full(inp, mode="segment_local"), BF16_TOL, "seg_tail (persistent, offset 600)")


def test_host_tensors_rejected_before_launch():
    # out, lse and mask on the host: the binding raises before any kernel runs
    import torch
    from diffusion_transformer_joint_amd.flux_attn import FluxAttnError, Plan
    from gpu_helpers import to_device
    inp = I.make_inputs(custom("hostout", 2, 128, [S("text", 70)]))
    w = inp.workload
    q, k, v, pos, _ = to_device(inp)
    shape = (w.batch, w.tokens, w.heads, w.head_dim)
    with Plan(w.batch, w.heads, w.head_dim, w.tokens) as plan:
        for mode in ("joint", "segment_local"):
            with pytest.raises(FluxAttnError):
                plan.forward(q, k, v, inp.segment_tokens, pos, out=torch.empty(shape, dtype=torch.bfloat16),
                             mode=mode)
        with pytest.raises(FluxAttnError):
            plan.forward_lse(q, k, v, inp.segment_tokens, pos,
                             lse=torch.empty((w.batch, w.heads, w.tokens), dtype=torch.float32))
        with pytest.raises(FluxAttnError):
            plan.block_mask(q, k, inp.segment_tokens, pos, 0.1,
                            mask=torch.empty(plan.mask_shape(w.tokens), dtype=torch.uint8))
        with pytest.raises(FluxAttnError):
            plan.forward_sparse(q, k, v, inp.segment_tokens, pos,
                                torch.ones(plan.mask_shape(w.tokens), dtype=torch.uint8))
        with pytest.raises(FluxAttnError):
            plan.forward(q.cpu(), k, v, inp.segment_tokens, pos)
        torch.cuda.synchronize()
