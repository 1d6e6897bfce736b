"""Backward of joint RoPE attention, fp64 (oracle; test infrastructure).

Source: the attention backward is the adjacent training workload of the path
(LoRA fine-tuning of the base model: "FLUX.3 Image Klein Brings 2-Second AI
Image Generation to Diffusers", Summary, and the Diffusers post's training
section).  The pages give no formula; these are the gradients of the forward
definition in ``softmax_attention`` (softmax attention, Vaswani et al. 2017;
the row-sum form of the softmax gradient as in FlashAttention, Dao et al. 2022),
written out step by step:

    Q~ = R q,  K~ = R k                    (rotary embedding per token)
    S  = scale Q~ K~^T,  P = softmax_rows(S),  O = P V
    dV = P^T dO
    dP = dO V^T
    Dr = rowsum(dO * O)                    (= rowsum(P * dP))
    dS = P * (dP - Dr)
    dQ~ = scale dS K~,   dK~ = scale dS^T Q~
    dq = R^T dQ~,  dk = R^T dK~            (R^T: rotation by the negative angle)

plus the per-row log-sum-exp  lse = log sum_j exp(S_ij)  that a training
forward stores.  Layout [B, N, H, D] as everywhere.
"""
import numpy as np

from .rope import apply_rope, rope_angles


def rope_transpose(x, pos, axes_dim, theta=10000.0):
    """R^T x: every pair rotated by the negative of its angle."""
    x = np.asarray(x, dtype=np.float64)
    ang = rope_angles(pos, axes_dim, theta)
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c + x1 * s
    out[..., 1::2] = -x0 * s + x1 * c
    return out


def attention_lse(q, k, pos, axes_dim, theta=10000.0, scale=None):
    """Natural-log log-sum-exp of each row of S: [B, H, N]."""
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    qr, kr = apply_rope(q, pos, axes_dim, theta), apply_rope(k, pos, axes_dim, theta)
    B, N, H, _ = q.shape
    out = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            s = scale * (qr[b, :, h] @ kr[b, :, h].T)
            m = s.max(axis=1)
            out[b, h] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def attention_backward(q, k, v, pos, axes_dim, dout, theta=10000.0, scale=None):
    """(dq, dk, dv) of joint RoPE attention for upstream gradient dout."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    qr, kr = apply_rope(q, pos, axes_dim, theta), apply_rope(k, pos, axes_dim, theta)
    dqr = np.empty_like(qr)
    dkr = np.empty_like(kr)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            s = scale * (qr[b, :, h] @ kr[b, :, h].T)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, :, h]
            do = dout[b, :, h]
            dv[b, :, h] = p.T @ do
            dp = do @ v[b, :, h].T
            dr = (do * o).sum(axis=1, keepdims=True)
            ds = p * (dp - dr)
            dqr[b, :, h] = scale * (ds @ kr[b, :, h])
            dkr[b, :, h] = scale * (ds.T @ qr[b, :, h])
    return rope_transpose(dqr, pos, axes_dim, theta), rope_transpose(dkr, pos, axes_dim, theta), dv
