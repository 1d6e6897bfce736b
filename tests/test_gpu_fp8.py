"""GPU parity of the e4m3 (FP8) path with the fp64 oracle on dequantized inputs.

The oracle computes attention of codes x per-(batch, head) scale in fp64; the
tolerances are those stated for FP8 (max-abs 6e-2, relative L2 2e-2).
"""
import dataclasses

import numpy as np
import pytest

import oracle
from diffusion_transformer_joint_amd import inputs as I

from gpu_helpers import FP8_TOL, assert_close, custom, out_fp64, ref_full, ref_rows, run_hip, sample_rows, say

pytestmark = pytest.mark.gpu

S = I.Segment


def test_gen4k_fp8_sampled_rows():
    inp = I.make_inputs(I.WORKLOADS["gen4k_fp8"])
    got = out_fp64(run_hip(inp))
    assert np.all(np.isfinite(got))
    rows = sample_rows(inp.workload.tokens, seed=7, count=48)
    assert_close(got[:, rows], ref_rows(inp, rows), FP8_TOL, f"gen4k_fp8 ({len(rows)} rows)")


FP8_CASES = [
    ("fp8_n1000", 1, 3, 128, [S("text", 40), S("image", 24, 40)]),
    ("fp8_n4608", 1, 2, 128, [S("text", 512), S("image", 64, 64)]),
    ("fp8_b2_n333", 2, 3, 128, [S("text", 45), S("image", 12, 24)]),
    ("fp8_d64_n300", 1, 3, 64, [S("text", 12), S("image", 12, 12), S("ref", 12, 12, 1)]),
    ("fp8_n1", 1, 2, 128, [S("text", 1)]),
]


@pytest.mark.parametrize("name,batch,heads,d,segs", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_fp8_full(name, batch, heads, d, segs):
    inp = I.make_inputs(custom(name, heads, d, segs, batch=batch, fp8=True))
    assert_close(out_fp64(run_hip(inp)), ref_full(inp), FP8_TOL, name)


def test_fp8_decodes_every_code_exactly():
    # One token: the output is V times its scale.  With scale 1 and the 254
    # finite codes spread over two heads, every output element must equal the
    # code's value exactly (each e4m3 value is a bf16 value).
    w = custom("codes", 2, 128, [S("text", 1)], fp8=True)
    inp = I.make_inputs(w)
    codes = np.arange(256, dtype=np.uint8)
    codes[codes == 0x7F] = 0x00
    codes[codes == 0xFF] = 0x80
    v = codes.reshape(1, 1, 2, 128)
    inp = dataclasses.replace(inp, v=np.ascontiguousarray(v), scales=np.ones((3, 1, 2), np.float32))
    got = out_fp64(run_hip(inp))
    want = oracle.e4m3_table()[v.astype(np.int64)]
    np.testing.assert_array_equal(got, want)


def test_fp8_scales_apply_per_head():
    w = custom("scales", 3, 128, [S("text", 70), S("image", 9, 9)], fp8=True)
    inp = I.make_inputs(w)
    sc = inp.scales.copy()
    sc[0] *= np.array([[0.5, 1.0, 3.0]], np.float32)
    sc[2] *= np.array([[2.0, 0.25, 1.0]], np.float32)
    inp = dataclasses.replace(inp, scales=sc)
    assert_close(out_fp64(run_hip(inp)), ref_full(inp), FP8_TOL, "per-head scales")
