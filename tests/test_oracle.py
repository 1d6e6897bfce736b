"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Closed forms worked by hand, an independent complex-number form of the rotary
embedding, a textbook attention routine (torch's scaled_dot_product_attention
in fp64), brute-force loops on tiny inputs, invariants of softmax attention,
and the e4m3 format's reference values.  A mutation test at the end plants
plausible mistakes into copies of the oracle functions and checks that these
pins catch them.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import softmax_attention as oatt
from oracle import rope as orope
from diffusion_transformer_joint_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------------
# independent helpers (written differently from the oracle on purpose)

def rope_complex(x, pos, axes_dim, theta):
    """Rotary embedding as complex multiplication, built axis by axis with loops."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    n_tok = x.shape[1]
    off = 0
    for a, d in enumerate(axes_dim):
        for j in range(d // 2):
            w = theta ** (-(2.0 * j) / d)
            e = np.array([cmath.exp(1j * pos[n][a] * w) for n in range(n_tok)])
            z = x[..., off + 2 * j] + 1j * x[..., off + 2 * j + 1]
            z = z * e[None, :, None]
            out[..., off + 2 * j] = z.real
            out[..., off + 2 * j + 1] = z.imag
        off += d
    return out


def sdpa_fp64(qr, kr, v, scale=None):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(qr.transpose(0, 2, 1, 3)))
    k = torch.from_numpy(np.ascontiguousarray(kr.transpose(0, 2, 1, 3)))
    vv = torch.from_numpy(np.ascontiguousarray(np.asarray(v, np.float64).transpose(0, 2, 1, 3)))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, vv, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


def brute_attention(qr, kr, v, scale):
    B, N, H, D = qr.shape
    out = np.zeros_like(qr)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                s = [scale * sum(qr[b, i, h, d] * kr[b, j, h, d] for d in range(D)) for j in range(N)]
                mx = max(s)
                w = [math.exp(t - mx) for t in s]
                z = sum(w)
                for d in range(v.shape[-1]):
                    out[b, i, h, d] = sum(w[j] * v[b, j, h, d] for j in range(N)) / z
    return out


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def rand_pos(n, seed, hi=64):
    return np.random.default_rng(seed).integers(0, hi, size=(n, 3)).astype(np.int64)


# ----------------------------------------------------------------------------------
# rotary embedding

def test_rope_hand_cases():
    # (axes, theta, pos, x, expected) worked by hand from the rotation definition
    cases = [
        # one pair per axis, frequency theta^0 = 1: rotate (1,0) by 1 rad and (0,1) by 2 rad
        ((2, 2, 0), 10000.0, (1, 2, 0), (1.0, 0.0, 0.0, 1.0),
         (math.cos(1), math.sin(1), -math.sin(2), math.cos(2))),
        # axis 0 of width 4: frequencies 1 and 10000^(-1/2) = 0.01; pos 100 -> angles 100, 1
        ((4, 0, 0), 10000.0, (100, 7, 9), (1.0, 0.0, 1.0, 0.0),
         (math.cos(100), math.sin(100), math.cos(1), math.sin(1))),
        # axis 2 of width 4, theta 100: frequencies 1 and 0.1; pos 5 -> angles 5, 0.5
        ((0, 0, 4), 100.0, (3, 4, 5), (2.0, 0.0, 0.0, 3.0),
         (2 * math.cos(5), 2 * math.sin(5), -3 * math.sin(0.5), 3 * math.cos(0.5))),
    ]
    for axes, theta, pos, x, exp in cases:
        got = orope.apply_rope(np.array(x, np.float64).reshape(1, 1, 1, 4), np.array([pos]), axes, theta)
        np.testing.assert_allclose(got.ravel(), exp, rtol=0, atol=1e-14)


def test_rope_frequencies_closed_form():
    f = orope.rope_frequencies((32, 48, 48), 10000.0)
    assert f.shape == (64,)
    assert f[0] == 1.0 and f[16] == 1.0 and f[40] == 1.0
    np.testing.assert_allclose(f[1], 10000.0 ** (-1 / 16), rtol=1e-15)
    np.testing.assert_allclose(f[15], 10000.0 ** (-30 / 32), rtol=1e-15)
    np.testing.assert_allclose(f[16 + 23], 10000.0 ** (-46 / 48), rtol=1e-15)


@pytest.mark.parametrize("axes", [(16, 24, 24), (32, 48, 48), (8, 8, 48)])
def test_rope_matches_complex_form(axes):
    D = sum(axes)
    x = rnd((2, 7, 3, D), 1)
    pos = rand_pos(7, 2, hi=600)
    np.testing.assert_allclose(orope.apply_rope(x, pos, axes, 10000.0),
                               rope_complex(x, pos, axes, 10000.0), rtol=0, atol=1e-12)


def test_rope_identity_norm_and_composition():
    axes = (32, 48, 48)
    x = rnd((1, 9, 2, 128), 3)
    zero = np.zeros((9, 3), np.int64)
    np.testing.assert_array_equal(orope.apply_rope(x, zero, axes), x)
    p1, p2 = rand_pos(9, 4), rand_pos(9, 5)
    y = orope.apply_rope(x, p1, axes)
    # each pair keeps its length
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # R(p2) R(p1) = R(p1 + p2)
    np.testing.assert_allclose(orope.apply_rope(y, p2, axes), orope.apply_rope(x, p1 + p2, axes),
                               rtol=0, atol=1e-11)


def test_rope_relative_offset_property():
    # <R(p) q, R(p') k> = <q, R(p' - p) k>
    axes = (32, 48, 48)
    q = rnd((1, 1, 1, 128), 6)
    k = rnd((1, 1, 1, 128), 7)
    for seed in range(5):
        p, pp = rand_pos(1, 10 + seed, hi=300), rand_pos(1, 20 + seed, hi=300)
        lhs = np.sum(orope.apply_rope(q, p, axes) * orope.apply_rope(k, pp, axes))
        rhs = np.sum(q * orope.apply_rope(k, pp - p, axes))
        assert abs(lhs - rhs) < 1e-11


# ----------------------------------------------------------------------------------
# attention

def test_softmax_rows_sum_to_one_and_shift_invariance():
    s = rnd((5, 17), 8, 3.0)
    p = oatt.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    v = rnd((17, 4), 9)
    base = oatt.attention_from_scores(s, v)
    np.testing.assert_allclose(oatt.attention_from_scores(s + 123.25, v), base, atol=1e-13)
    row_shift = rnd((5, 1), 10, 50.0)
    np.testing.assert_allclose(oatt.attention_from_scores(s + row_shift, v), base, atol=1e-12)
    # V = ones -> every output is exactly a convex combination summing to 1
    np.testing.assert_allclose(oatt.attention_from_scores(s, np.ones((17, 3))), 1.0, rtol=1e-14)


@pytest.mark.parametrize("N,D", [(1, 8), (5, 8), (12, 8)])
def test_attention_brute_force(N, D):
    axes = (2, 2, D - 4)
    q, k, v = rnd((1, N, 2, D), 11), rnd((1, N, 2, D), 12), rnd((1, N, 2, D), 13)
    pos = rand_pos(N, 14, hi=40)
    got = oracle.joint_rope_attention(q, k, v, pos, axes)
    qr, kr = rope_complex(q, pos, axes, 10000.0), rope_complex(k, pos, axes, 10000.0)
    np.testing.assert_allclose(got, brute_attention(qr, kr, v, 1 / math.sqrt(D)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("wl", ["tiny"])
def test_attention_vs_sdpa_on_workload(wl):
    w = I.WORKLOADS[wl]
    inp = I.make_inputs(w)
    q, k, v = oracle.inputs_to_fp64(inp)
    got = oracle.joint_rope_attention(q, k, v, inp.pos, w.axes_dim, row_block=32)
    qr, kr = rope_complex(q, inp.pos, w.axes_dim, 10000.0), rope_complex(k, inp.pos, w.axes_dim, 10000.0)
    np.testing.assert_allclose(got, sdpa_fp64(qr, kr, v), rtol=0, atol=1e-12)


def test_attention_vs_sdpa_mid_size_custom_scale():
    axes = (32, 48, 48)
    q, k, v = rnd((2, 300, 3, 128), 15, 0.5), rnd((2, 300, 3, 128), 16, 0.5), rnd((2, 300, 3, 128), 17)
    pos = rand_pos(300, 18, hi=200)
    got = oracle.joint_rope_attention(q, k, v, pos, axes, scale=0.2, row_block=64)
    qr, kr = rope_complex(q, pos, axes, 10000.0), rope_complex(k, pos, axes, 10000.0)
    np.testing.assert_allclose(got, sdpa_fp64(qr, kr, v, scale=0.2), rtol=0, atol=1e-12)


def test_rows_variant_matches_full():
    axes = (16, 24, 24)
    q, k, v = rnd((1, 90, 2, 64), 19), rnd((1, 90, 2, 64), 20), rnd((1, 90, 2, 64), 21)
    pos = rand_pos(90, 22)
    full = oracle.joint_rope_attention(q, k, v, pos, axes)
    rows = np.array([0, 5, 63, 64, 89])
    np.testing.assert_allclose(oracle.joint_rope_attention_rows(q, k, v, pos, axes, rows), full[:, rows],
                               rtol=0, atol=1e-14)


def test_translation_invariance():
    axes = (32, 48, 48)
    q, k, v = rnd((1, 40, 2, 128), 23), rnd((1, 40, 2, 128), 24), rnd((1, 40, 2, 128), 25)
    pos = rand_pos(40, 26)
    a = oracle.joint_rope_attention(q, k, v, pos, axes)
    b = oracle.joint_rope_attention(q, k, v, pos + np.array([[37, 5, 1000]]), axes)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_permutation_equivariance():
    axes = (32, 48, 48)
    q, k, v = rnd((1, 33, 2, 128), 27), rnd((1, 33, 2, 128), 28), rnd((1, 33, 2, 128), 29)
    perm = np.random.default_rng(30).permutation(33)
    zero = np.zeros((33, 3), np.int64)
    a = oracle.joint_rope_attention(q, k, v, zero, axes)
    b = oracle.joint_rope_attention(q[:, perm], k[:, perm], v[:, perm], zero, axes)
    np.testing.assert_allclose(b, a[:, perm], rtol=0, atol=1e-13)
    pos = rand_pos(33, 31)
    a = oracle.joint_rope_attention(q, k, v, pos, axes)
    b = oracle.joint_rope_attention(q[:, perm], k[:, perm], v[:, perm], pos[perm], axes)
    np.testing.assert_allclose(b, a[:, perm], rtol=0, atol=1e-13)


def test_closed_forms():
    axes = (16, 24, 24)
    pos = rand_pos(20, 32)
    v = rnd((1, 20, 2, 64), 33)
    k = rnd((1, 20, 2, 64), 34)
    # Q = 0 -> uniform weights -> mean of V
    o = oracle.joint_rope_attention(np.zeros((1, 20, 2, 64)), k, v, pos, axes)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-14)
    # N = 1 -> O = V
    o = oracle.joint_rope_attention(rnd((1, 1, 2, 64), 35), k[:, :1], v[:, :1], pos[:1], axes)
    np.testing.assert_allclose(o, v[:, :1], atol=1e-15)
    # RoPE off and every key equal -> equal scores -> mean of V
    zero = np.zeros((20, 3), np.int64)
    keq = np.broadcast_to(k[:, :1], k.shape).copy()
    o = oracle.joint_rope_attention(rnd((1, 20, 2, 64), 36), keq, v, zero, axes)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-13)
    # orthogonal one-hot Q = K with a large gain -> each token picks its own V
    n = 16
    qk = np.zeros((1, n, 1, 64))
    qk[0, np.arange(n), 0, np.arange(n)] = 40.0
    vv = rnd((1, n, 1, 64), 37)
    o = oracle.joint_rope_attention(qk, qk, vv, np.zeros((n, 3), np.int64), axes)
    np.testing.assert_allclose(o, vv, atol=1e-12)


def test_segment_local_matches_masked_brute_force():
    axes = (2, 2, 4)
    segs = [3, 0, 4, 2]
    N = sum(segs)
    q, k, v = rnd((1, N, 2, 8), 38), rnd((1, N, 2, 8), 39), rnd((1, N, 2, 8), 40)
    pos = rand_pos(N, 41)
    got = oracle.segment_local_rope_attention(q, k, v, pos, segs, axes)
    qr, kr = rope_complex(q, pos, axes, 10000.0), rope_complex(k, pos, axes, 10000.0)
    seg_id = np.repeat(np.arange(len(segs)), segs)
    exp = np.zeros_like(q)
    for b in range(1):
        for h in range(2):
            s = (qr[b, :, h] @ kr[b, :, h].T) / math.sqrt(8)
            s = np.where(seg_id[:, None] == seg_id[None, :], s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            exp[b, :, h] = (p / p.sum(axis=1, keepdims=True)) @ v[b, :, h]
    np.testing.assert_allclose(got, exp, atol=1e-13)
    one = oracle.segment_local_rope_attention(q, k, v, pos, [N], axes)
    np.testing.assert_allclose(one, oracle.joint_rope_attention(q, k, v, pos, axes), atol=1e-14)


# ----------------------------------------------------------------------------------
# e4m3

def test_e4m3_spec_points():
    with open(os.path.join(GOLDEN, "e4m3_spec_points.json")) as f:
        pts = json.load(f)["points"]
    tab = oracle.e4m3_table()
    for p in pts:
        c = int(p["code"], 16)
        if p["value"] == "nan":
            assert np.isnan(tab[c])
        else:
            assert tab[c] == p["value"] and math.copysign(1, tab[c]) == math.copysign(1, p["value"])
    assert np.isnan(tab).sum() == 2


def test_e4m3_all_codes_vs_torch():
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(ref), np.isnan(oracle.e4m3_table()))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ref[ok], oracle.e4m3_table()[ok])


def _bf16_from_format(bits):
    """bfloat16 decoded from its format definition (1 sign bit, 8 exponent bits
    with bias 127, 7 fraction bits; exponent 0 holds subnormals f/128 * 2^-126,
    exponent 255 holds infinities and NaNs): an independent route from the
    oracle's bit shift."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(np.float64)
    val = np.where(e == 0, (f / 128.0) * 2.0 ** -126, (1.0 + f / 128.0) * np.exp2(e.astype(np.float64) - 127.0))
    val = np.where(e == 0xFF, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def test_bf16_widening_all_patterns():
    # every one of the 65,536 bfloat16 bit patterns: the oracle's widening must
    # give the format's value exactly (torch's bfloat16 -> float64 cast and the
    # format definition decoded by hand), NaN exactly where the format has NaN
    import torch
    from oracle.inputs_fp64 import bf16_to_fp64
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = bf16_to_fp64(bits)
    assert got.dtype == np.float64 and got.shape == (65536,)
    via_torch = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    by_hand = _bf16_from_format(bits)
    for ref in (via_torch, by_hand):
        np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
        ok = ~np.isnan(ref)
        np.testing.assert_array_equal(got[ok], ref[ok])
        np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))   # -0.0 stays -0.0
    assert np.isnan(got).sum() == 2 * 127            # exponent 255 with a nonzero fraction
    # shapes are kept (the oracle widens [B, N, H, D] tensors)
    x = bits[:24].reshape(1, 2, 3, 4)
    np.testing.assert_array_equal(bf16_to_fp64(x), got[:24].reshape(1, 2, 3, 4))


def test_e4m3_positive_codes_monotone():
    tab = oracle.e4m3_table()[:127]
    assert np.all(np.diff(tab) > 0)


def test_dequantize_per_head_scale():
    codes = np.full((1, 3, 2, 4), 0x38, np.uint8)   # value 1.0
    got = oracle.dequantize(codes, np.array([[0.5, 3.0]], np.float32))
    np.testing.assert_array_equal(got[0, :, 0], 0.5)
    np.testing.assert_array_equal(got[0, :, 1], 3.0)


# ----------------------------------------------------------------------------------
# mutation test: plausible mistakes planted in copies of the oracle must be caught

def _rope_sign_flip(x, pos, axes_dim, theta=10000.0):
    x = np.asarray(x, np.float64)
    ang = orope.rope_angles(pos, axes_dim, theta)
    c, s = np.cos(ang)[None, :, None, :], np.sin(ang)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s       # wrong sign
    out[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _rope_wrong_freq(x, pos, axes_dim, theta=10000.0):
    # frequency exponent over the whole head instead of per axis
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    j = np.arange(D // 2)
    axis = np.concatenate([np.full(d // 2, a) for a, d in enumerate(axes_dim)])
    ang = np.asarray(pos, np.float64)[:, axis] * theta ** (-2.0 * j / D)
    c, s = np.cos(ang)[None, :, None, :], np.sin(ang)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


_ORIG_ATTENTION = oatt.attention


def _attention_no_scale(q, k, v, scale=None, row_block=1024, rows=None):
    return _ORIG_ATTENTION(q, k, v, scale=1.0)


def _attention_transposed_k(q, k, v, scale=None, row_block=1024, rows=None):
    k = np.asarray(k)
    return _ORIG_ATTENTION(q, np.ascontiguousarray(k[..., ::-1]), v, scale)


@pytest.mark.parametrize("mut", ["rope_sign", "rope_freq", "att_scale", "att_k"])
def test_mutations_are_caught(mut, monkeypatch):
    axes = (32, 48, 48)
    q, k, v = rnd((1, 24, 2, 128), 50), rnd((1, 24, 2, 128), 51), rnd((1, 24, 2, 128), 52)
    pos = rand_pos(24, 53, hi=300)
    if mut == "rope_sign":
        monkeypatch.setattr(oatt, "apply_rope", _rope_sign_flip)
    elif mut == "rope_freq":
        monkeypatch.setattr(oatt, "apply_rope", _rope_wrong_freq)
    elif mut == "att_scale":
        monkeypatch.setattr(oatt, "attention", _attention_no_scale)
    else:
        monkeypatch.setattr(oatt, "attention", _attention_transposed_k)
    got = oatt.joint_rope_attention(q, k, v, pos, axes)
    qr, kr = rope_complex(q, pos, axes, 10000.0), rope_complex(k, pos, axes, 10000.0)
    ref = sdpa_fp64(qr, kr, v)
    assert np.max(np.abs(got - ref)) > 1e-3
