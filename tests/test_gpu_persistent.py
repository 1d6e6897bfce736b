"""GPU parity of the persistent split schedule of the bf16 kernel.

With the persistent split, one workgroup per compute unit runs an equal slice
of all (query tile, 64-key tile) positions, storing partial softmax states for
the tiles its slice cuts, and a merge kernel combines them.  The library picks
it by cost where a launch has fewer query tiles than compute units (one GPU's
3-head share of the 8,704-token call: 102 tiles); the 4,608- and 8,704-token
calls over all 24 heads run the whole-tile schedule (unsplit and split,
respectively).  FLUX_ATTN_SCHEDULE=persistent forces it at plan creation,
which these tests use to cover small, ragged, batched and D = 64 launches
(including slices of a single position and empty slices) against the oracle.
"""
import numpy as np
import pytest

import oracle
from diffusion_transformer_joint_amd import inputs as I

from gpu_helpers import BF16_TOL, assert_close, custom, out_fp64, ref_full, ref_rows, run_hip, sample_rows

pytestmark = pytest.mark.gpu

S = I.Segment

CASES = [
    # 12 tiles x 16 positions = 192 < 256 slices: single-position slices and empty ones
    ("pk_n1000", 1, 3, 128, [S("text", 40), S("image", 24, 40)]),
    ("pk_b2_n2000", 2, 4, 128, [S("text", 80), S("image", 40, 48)]),
    ("pk_d64_n1500", 1, 4, 64, [S("text", 60), S("image", 30, 48)]),
    ("pk_n65", 1, 2, 128, [S("text", 1), S("image", 8, 8)]),
]


@pytest.mark.parametrize("name,batch,heads,d,segs", CASES, ids=[c[0] for c in CASES])
def test_persistent_against_oracle(monkeypatch, name, batch, heads, d, segs):
    monkeypatch.setenv("FLUX_ATTN_SCHEDULE", "persistent")
    inp = I.make_inputs(custom(name, heads, d, segs, batch=batch, sigma=1.0))
    assert_close(out_fp64(run_hip(inp)), ref_full(inp), BF16_TOL, name)


def test_persistent_three_heads_full_length(monkeypatch):
    # one GPU's 3-head share at 8,704 tokens: 102 tiles x 136 positions, ~54 per slice
    monkeypatch.setenv("FLUX_ATTN_SCHEDULE", "persistent")
    inp = I.make_inputs(custom("pk_h3_n8704", 3, 128, [S("text", 512), S("image", 64, 64), S("ref", 64, 64, 1)]))
    got = out_fp64(run_hip(inp))
    rows = sample_rows(8704, seed=9, count=64)
    assert_close(got[:, rows], ref_rows(inp, rows), BF16_TOL, "persistent 3 heads x 8704")


def test_persistent_lse(monkeypatch):
    # the merge of a persistent launch also writes the row log-sum-exp
    import torch
    from diffusion_transformer_joint_amd.flux_attn import Plan
    from gpu_helpers import to_device
    monkeypatch.setenv("FLUX_ATTN_SCHEDULE", "persistent")
    inp = I.make_inputs(custom("pk_lse", 3, 128, [S("text", 40), S("image", 24, 40)], sigma=1.0))
    w = inp.workload
    q, k, v, pos, _ = to_device(inp)
    with Plan(w.batch, w.heads, w.head_dim, w.tokens) as plan:
        out, lse = plan.forward_lse(q, k, v, inp.segment_tokens, pos)
        torch.cuda.synchronize()
    qq, kk, _ = oracle.inputs_to_fp64(inp)
    rl = oracle.attention_lse(qq, kk, inp.pos, w.axes_dim)
    err = float(np.abs(lse.cpu().numpy().astype(np.float64) - rl).max())
    assert err < 2e-2, err
    assert_close(out_fp64(out), ref_full(inp), BF16_TOL, "persistent forward_lse")
