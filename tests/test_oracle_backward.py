"""Pins of the attention-backward oracle (oracle/backward.py) against facts that
do not come from it: torch autograd in fp64 on an independently written forward,
central finite differences, the adjointness of the rotary embedding, closed
forms, and planted mistakes.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import backward as ob

AXES = (8, 12, 12)


def _rand(shape, seed, s=1.0):
    return s * np.random.default_rng(seed).standard_normal(shape)


def _pos(n, seed=0):
    return np.random.default_rng(seed).integers(0, 30, size=(n, 3)).astype(np.int32)


def _torch_forward(q, k, v, pos, axes, theta=10000.0):
    """Forward written with torch ops (complex rotation), for autograd."""
    import torch
    B, N, H, D = q.shape
    ang = []
    for a, d in enumerate(axes):
        j = torch.arange(d // 2, dtype=torch.float64)
        w = theta ** (-2.0 * j / d)
        ang.append(torch.as_tensor(pos[:, a], dtype=torch.float64)[:, None] * w[None, :])
    ang = torch.cat(ang, dim=1)                       # [N, D/2]
    rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]

    def rope(x):
        z = torch.view_as_complex(x.reshape(B, N, H, D // 2, 2).contiguous())
        return torch.view_as_real(z * rot).reshape(B, N, H, D)

    qr, kr = rope(q), rope(k)
    s = torch.einsum("bihd,bjhd->bhij", qr, kr) / math.sqrt(D)
    p = torch.softmax(s, dim=-1)
    return torch.einsum("bhij,bjhd->bihd", p, v), torch.logsumexp(s, dim=-1)


def test_against_torch_autograd():
    torch = pytest.importorskip("torch")
    B, N, H, D = 2, 23, 2, 32
    q, k, v, do = (_rand((B, N, H, D), s, 0.8) for s in (1, 2, 3, 4))
    pos = _pos(N)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o, lse = _torch_forward(tq, tk, tv, pos, AXES)
    o.backward(torch.from_numpy(do))
    dq, dk, dv = ob.attention_backward(q, k, v, pos, AXES, do)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ob.attention_lse(q, k, pos, AXES), lse.detach().numpy(), rtol=1e-12)
    np.testing.assert_allclose(oracle.joint_rope_attention(q, k, v, pos, AXES), o.detach().numpy(), rtol=1e-10,
                               atol=1e-12)


def test_finite_differences():
    B, N, H, D = 1, 7, 1, 32
    q, k, v, do = (_rand((B, N, H, D), s) for s in (5, 6, 7, 8))
    pos = _pos(N, 1)
    dq, dk, dv = ob.attention_backward(q, k, v, pos, AXES, do)
    f = lambda q_, k_, v_: float((oracle.joint_rope_attention(q_, k_, v_, pos, AXES) * do).sum())
    h = 1e-6
    rng = np.random.default_rng(9)
    for which, g in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = tuple(rng.integers(0, n) for n in (B, N, H, D))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[which][idx] += h
            fp = f(args["q"], args["k"], args["v"])
            args[which][idx] -= 2 * h
            fm = f(args["q"], args["k"], args["v"])
            assert abs((fp - fm) / (2 * h) - g[idx]) < 1e-6 * max(1.0, abs(g[idx])), (which, idx)


def test_rope_transpose_is_the_adjoint():
    x, y = _rand((1, 9, 2, 32), 10), _rand((1, 9, 2, 32), 11)
    pos = _pos(9, 2)
    lhs = (oracle.apply_rope(x, pos, AXES) * y).sum()
    rhs = (x * ob.rope_transpose(y, pos, AXES)).sum()
    assert abs(lhs - rhs) < 1e-12 * abs(lhs)
    np.testing.assert_allclose(ob.rope_transpose(oracle.apply_rope(x, pos, AXES), pos, AXES), x, atol=1e-13)


def test_closed_forms():
    # Q = 0: P is uniform (1/N), so dV_j = mean_i dO_i for every j, and dK = 0
    # (all scores equal, dS = P * (dP - rowsum(P dP)) has zero sum along keys,
    # and Q = 0 gives dK~ = scale dS^T Q~ = 0).
    B, N, H, D = 1, 12, 2, 32
    k, v, do = (_rand((B, N, H, D), s) for s in (12, 13, 14))
    q = np.zeros_like(k)
    pos = _pos(N, 3)
    dq, dk, dv = ob.attention_backward(q, k, v, pos, AXES, do)
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=1, keepdims=True), dv.shape), atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    # N = 1: O = V, so dV = dO and dq = dk = 0
    q1, k1, v1, do1 = (_rand((1, 1, 2, 32), s) for s in (15, 16, 17, 18))
    dq1, dk1, dv1 = ob.attention_backward(q1, k1, v1, _pos(1), AXES, do1)
    np.testing.assert_allclose(dv1, do1, atol=1e-15)
    np.testing.assert_allclose(dq1, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk1, 0.0, atol=1e-15)


def test_mutations_are_caught():
    torch = pytest.importorskip("torch")
    B, N, H, D = 1, 9, 2, 32
    q, k, v, do = (_rand((B, N, H, D), s) for s in (20, 21, 22, 23))
    pos = _pos(N, 4)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o, _ = _torch_forward(tq, tk, tv, pos, AXES)
    o.backward(torch.from_numpy(do))
    ref = (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())
    orig_rt = ob.rope_transpose
    try:
        ob.rope_transpose = lambda x, p, a, theta=10000.0: np.asarray(x, dtype=np.float64)   # forgot R^T
        bad = ob.attention_backward(q, k, v, pos, AXES, do)
        assert not np.allclose(bad[0], ref[0], atol=1e-6)
        ob.rope_transpose = lambda x, p, a, theta=10000.0: oracle.apply_rope(x, p, a, theta)  # R instead of R^T
        bad = ob.attention_backward(q, k, v, pos, AXES, do)
        assert not np.allclose(bad[1], ref[1], atol=1e-6)
    finally:
        ob.rope_transpose = orig_rt
    # mistakes planted in copies of the gradient function's source
    import inspect
    src = inspect.getsource(ob.attention_backward)
    plants = [
        ("ds = p * (dp - dr)", "ds = p * dp", (0, 1)),                    # dropped Dr term
        ("dqr[b, :, h] = scale * (ds @ kr[b, :, h])", "dqr[b, :, h] = ds @ kr[b, :, h]", (0,)),  # lost scale
        ("dv[b, :, h] = p.T @ do", "dv[b, :, h] = p @ do", (2,)),          # transposed P
        ("dp = do @ v[b, :, h].T", "dp = do @ v[b, :, h].T * scale", (0, 1)),  # spurious factor
    ]
    for old, new, hit in plants:
        assert old in src
        ns = dict(vars(ob))
        exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
        bad = ns["attention_backward"](q, k, v, pos, AXES, do)
        for i in hit:
            assert not np.allclose(bad[i], ref[i], atol=1e-6), (old, new, i)
    good = ob.attention_backward(q, k, v, pos, AXES, do)
    for g, r in zip(good, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)
