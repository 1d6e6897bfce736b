"""Attention of the FP8 path with its requantization step, fp64 (oracle; test infrastructure).

Source: "Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell GPUs",
How it works: quantized attention with query, key and value in FP8.  The pages
do not say where the rotary embedding sits relative to the quantization.  The
reading used by the path: the inputs are e4m3 codes of the *unrotated* Q, K, V
with one scale per (tensor, batch, head); the rotary embedding is applied
inside the attention (fused into its Q/K loads), so the rotated Q and K are
quantized a second time before the e4m3 score products: each rotated code
vector is halved and rounded to e4m3 (a rotated component is at most sqrt(2)
times its pair's largest code, so halving keeps it within +-448).  Rotation is
linear, so the scales multiply the scores afterwards: 2 s_q * 2 s_k.

``fp8_requant_attention`` is that definition written out:
    Q~ = e4m3_round(R(codes_q) / 2) * 2 s_q,  K~ likewise,  V = codes_v * s_v,
    O  = softmax(scale Q~ K~^T) V,
with R the exact multi-axis rotation (``rope.apply_rope``), ``e4m3_round`` the
format's nearest-even rounding (``e4m3.e4m3_round``) and the softmax exact.

The plain oracle (``softmax_attention`` on dequantized codes) has no second
quantization; the difference between the two is the error the requantization
adds, which grows with the size of the scores (input scale sigma).  This
module lets a test compare the FP8 kernel with the arithmetic it is meant to
perform at any input scale, not only where that error is small.
"""
import numpy as np

from .e4m3 import e4m3_round, e4m3_table
from .rope import apply_rope
from .softmax_attention import attention


def requantized_operands(q_codes, k_codes, v_codes, scales, pos, axes_dim, theta=10000.0):
    """(Q~, K~, V) in fp64 [B,N,H,D] as defined in the module docstring.

    scales: [3, B, H] (q, k, v) per (batch, head).
    """
    tab = e4m3_table()
    sc = np.asarray(scales, dtype=np.float64)
    q = tab[np.asarray(q_codes, dtype=np.uint8)]
    k = tab[np.asarray(k_codes, dtype=np.uint8)]
    v = tab[np.asarray(v_codes, dtype=np.uint8)]
    qr = e4m3_round(apply_rope(q, pos, axes_dim, theta) / 2.0) * 2.0 * sc[0][:, None, :, None]
    kr = e4m3_round(apply_rope(k, pos, axes_dim, theta) / 2.0) * 2.0 * sc[1][:, None, :, None]
    return qr, kr, v * sc[2][:, None, :, None]


def fp8_requant_attention(q_codes, k_codes, v_codes, scales, pos, axes_dim, segment_tokens=None,
                          theta=10000.0, scale=None):
    """Joint (segment_tokens None) or segment-local attention over the requantized operands."""
    qr, kr, v = requantized_operands(q_codes, k_codes, v_codes, scales, pos, axes_dim, theta)
    if segment_tokens is None:
        return attention(qr, kr, v, scale)
    out = np.empty(v.shape, dtype=np.float64)
    t0 = 0
    for n in segment_tokens:
        sl = slice(t0, t0 + n)
        if n:
            out[:, sl] = attention(qr[:, sl], kr[:, sl], v[:, sl], scale)
        t0 += n
    return out
