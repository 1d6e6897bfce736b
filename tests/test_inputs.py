"""Host-side checks of the seeded workload generator (no GPU)."""
import numpy as np
import pytest

from diffusion_transformer_joint_amd import inputs as I


def test_workload_token_counts():
    n = {k: w.tokens for k, w in I.WORKLOADS.items()}
    assert n == {"tiny": 80, "t2i1024": 4608, "edit1024": 8704, "gen2048r2": 25088, "gen4k_fp8": 66048,
                 "edit1024_local": 8704}
    assert I.WORKLOADS["edit1024"].segment_tokens == [512, 4096, 4096]
    assert I.WORKLOADS["gen2048r2"].segment_tokens == [512, 16384, 4096, 4096]


def test_coherence_zero_keeps_draws_and_positive_shares_a_direction():
    w = I.custom_workload("c", 1, 2, 64, [I.Segment("text", 300)], sigma=1.0)
    a = I.make_inputs(w)
    b = I.make_inputs(I.Workload(w.name, w.batch, w.heads, w.head_dim, w.segments, w.sigma, w.fp8, w.seed,
                                 w.description, 0.0))
    assert a.sha256() == b.sha256()
    c = I.make_inputs(I.Workload(w.name, w.batch, w.heads, w.head_dim, w.segments, w.sigma, w.fp8, w.seed,
                                 w.description, 0.9))
    np.testing.assert_array_equal(c.v, a.v)          # V is not shared
    q, k = I.bf16_bits_to_f32(c.q), I.bf16_bits_to_f32(c.k)
    cos = (q * k).sum(-1) / np.linalg.norm(q, axis=-1) / np.linalg.norm(k, axis=-1)
    assert 0.7 < cos.mean() < 0.9                    # a^2 = 0.81 of the energy is common


def test_axes_split():
    assert I.default_axes_dim(64) == (16, 24, 24)
    assert I.default_axes_dim(128) == (32, 48, 48)


def test_position_ids_structure():
    segs = I.WORKLOADS["gen2048r2"].segments
    pos = I.position_ids(segs)
    assert pos.shape == (25088, 3) and pos.dtype == np.int32
    np.testing.assert_array_equal(pos[:512, 0], np.arange(512))
    assert np.all(pos[:512, 1:] == 0)
    img = pos[512:512 + 16384]
    assert np.all(img[:, 0] == 0)
    np.testing.assert_array_equal(img[:, 1], np.repeat(np.arange(128), 128))
    np.testing.assert_array_equal(img[:, 2], np.tile(np.arange(128), 128))
    r1, r2 = pos[512 + 16384:512 + 16384 + 4096], pos[-4096:]
    assert np.all(r1[:, 0] == 1) and np.all(r2[:, 0] == 2)
    np.testing.assert_array_equal(r2[:, 1:], r1[:, 1:])


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]   # exact ties
    bits = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_make_inputs_deterministic_and_distribution():
    w = I.WORKLOADS["tiny"]
    a, b = I.make_inputs(w), I.make_inputs(w)
    assert a.sha256() == b.sha256()
    assert a.q.shape == (1, 80, 2, 64) and a.q.dtype == np.uint16
    c = I.make_inputs(w, seed=99)
    assert c.sha256() != a.sha256()
    q = I.bf16_bits_to_f32(a.q)
    assert 0.8 < q.std() < 1.2


def test_fp8_quantization_scales():
    w = I.custom_workload("f8", 1, 3, 128, [I.Segment("text", 40), I.Segment("image", 4, 6)], fp8=True, seed=7)
    inp = I.make_inputs(w)
    assert inp.q.dtype == np.uint8 and inp.scales.shape == (3, 1, 3)
    import torch
    for t, codes in enumerate((inp.q, inp.k, inp.v)):
        vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
        # per-head absmax maps to the largest code value
        np.testing.assert_array_equal(np.abs(vals).max(axis=(1, 3)), 448.0)
        assert np.all(inp.scales[t] > 0)
