"""GPU parity of tile-sparse attention and of its tile-mask rule.

forward_sparse is compared with the oracle's exact attention over the same
kept tiles (oracle/block_sparse.py); the masks are drawn by seeded random
generators here or computed by the oracle's rule, never taken from the GPU.
The GPU mask rule is compared with the oracle's rule wherever the decision is
clear (|margin| > 1e-3 in the exp2 domain); closer decisions may go either way
in fp32 and are only checked to be 0/1.
"""
import numpy as np
import pytest

import oracle
from diffusion_transformer_joint_amd import inputs as I

from gpu_helpers import BF16_TOL, assert_close, custom, out_fp64, sample_rows, say, to_device

pytestmark = pytest.mark.gpu

S = I.Segment


def _plan(w):
    from diffusion_transformer_joint_amd.flux_attn import Plan
    return Plan(w.batch, w.heads, w.head_dim, w.tokens)


def _mask_shape(w):
    return (w.batch, w.heads, (w.tokens + 255) // 256, (w.tokens + 63) // 64)


def _run_sparse(inp, mask):
    import torch
    w = inp.workload
    q, k, v, pos, _ = to_device(inp)
    m = torch.from_numpy(np.ascontiguousarray(mask.astype(np.uint8))).to("cuda:0")
    with _plan(w) as plan:
        say(f"  HIP forward_sparse: {w.name} N={w.tokens} H={w.heads} D={w.head_dim} kept {mask.mean():.2f}")
        o = plan.forward_sparse(q, k, v, inp.segment_tokens, pos, m)
        torch.cuda.synchronize()
    return o


def _oracle(inp, mask, rows=None):
    w = inp.workload
    q, k, v = oracle.inputs_to_fp64(inp)
    return oracle.block_sparse_attention(q, k, v, inp.pos, w.axes_dim, mask, rows=rows)


CASES = [
    ("sp_n1000", 1, 3, 128, [S("text", 40), S("image", 24, 40)]),
    ("sp_n4097", 1, 2, 128, [S("text", 1), S("image", 64, 64)]),
    ("sp_b2_n333", 2, 2, 128, [S("text", 45), S("image", 12, 24)]),
    ("sp_d64_n300", 1, 3, 64, [S("text", 12), S("image", 12, 12), S("ref", 12, 12, 1)]),
]


@pytest.mark.parametrize("name,batch,heads,d,segs", CASES, ids=[c[0] for c in CASES])
def test_forward_sparse_random_mask(name, batch, heads, d, segs):
    inp = I.make_inputs(custom(name, heads, d, segs, batch=batch, sigma=1.0))
    rng = np.random.default_rng(abs(hash(name)) % (2 ** 32))
    mask = rng.random(_mask_shape(inp.workload)) < 0.4
    mask[..., -1] = True                      # the ragged last key tile
    mask[0, 0, -1, :] = False                 # a query tile that keeps nothing -> 0
    got = out_fp64(_run_sparse(inp, mask))
    ref = _oracle(inp, mask)
    assert np.all(got[0, 256 * (mask.shape[2] - 1):, 0] == 0.0)
    assert_close(got, ref, BF16_TOL, name)


def test_all_kept_equals_dense_bitwise(monkeypatch):
    # The sparse launch always uses the split schedule; the dense call is held
    # to it too (this size, 60 tiles, would otherwise get the persistent one).
    import torch
    from gpu_helpers import run_hip
    monkeypatch.setenv("FLUX_ATTN_SCHEDULE", "split")
    inp = I.make_inputs(custom("sp_dense", 6, 128, [S("text", 512), S("image", 48, 48)]))
    dense = run_hip(inp)
    sparse = _run_sparse(inp, np.ones(_mask_shape(inp.workload), bool))
    assert torch.equal(dense.view(torch.int16), sparse.view(torch.int16))


def test_edit1024_local_oracle_mask_sampled_rows():
    # sigma 1.5 with a shared Q/K direction: scores span tens of units, rows are
    # peaked, and the bf16 error of the dense kernel itself is near the 5e-3
    # bound (like the sigma = 2 stress case).  The sparse path must be as
    # accurate as the dense kernel on the same inputs and rows.
    from gpu_helpers import errors, ref_rows, run_hip
    w = I.WORKLOADS["edit1024_local"]
    inp = I.make_inputs(w)
    q, k, v = oracle.inputs_to_fp64(inp)
    mask, _ = oracle.block_mask(oracle.block_scores(q, k, inp.pos, w.axes_dim), 0.01)
    got = out_fp64(_run_sparse(inp, mask))
    assert np.all(np.isfinite(got))
    rows = sample_rows(w.tokens, seed=9, count=40)
    ma, rl = errors(got[:, rows], _oracle(inp, mask, rows=rows))
    dma, drl = errors(out_fp64(run_hip(inp))[:, rows], ref_rows(inp, rows))
    say(f"  edit1024_local tau 0.01, kept {mask.mean():.2f}: sparse max-abs {ma:.3e} rel-L2 {rl:.3e}; "
        f"dense max-abs {dma:.3e} rel-L2 {drl:.3e}")
    assert rl <= 1.2 * drl + 1e-4 and ma <= 2.0 * dma + 1e-3
    assert rl <= 1e-2


@pytest.mark.parametrize("name,tau", [("edit1024_local", 0.01), ("edit1024_local", 0.1), ("sp_small", 0.3)])
def test_block_mask_matches_oracle_rule(name, tau):
    import torch
    if name == "sp_small":
        w = custom("sp_small", 3, 128, [S("text", 200), S("image", 30, 30)], sigma=1.5)
        w = I.Workload(w.name, w.batch, w.heads, w.head_dim, w.segments, w.sigma, w.fp8, w.seed, w.description, 0.9)
    else:
        w = I.WORKLOADS[name]
    inp = I.make_inputs(w)
    q, k, v = oracle.inputs_to_fp64(inp)
    want, margin = oracle.block_mask(oracle.block_scores(q, k, inp.pos, w.axes_dim), tau)
    qd, kd, _, pos, _ = to_device(inp)
    with _plan(w) as plan:
        got = plan.block_mask(qd, kd, inp.segment_tokens, pos, tau)
        torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert set(np.unique(got)) <= {0, 1}
    clear = np.abs(margin) > 1e-3
    say(f"  {name} tau {tau}: kept {want.mean():.3f}, unclear decisions {int((~clear).sum())} of {clear.size}")
    assert np.array_equal(got.astype(bool)[clear], want[clear])
    assert got.sum(axis=-1).min() >= 1
