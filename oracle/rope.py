"""Multi-axis rotary position embedding, fp64 (oracle; test infrastructure).

Source: "Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell GPUs",
section "How it works", names rotary position embeddings as part of the
transformer's projection path; the pages give no formula.  The definition used
is the rotary embedding of RoFormer (Su et al., 2021): a vector is split into
pairs and pair j is rotated by the angle  pos * theta^(-2j/d).

Multi-axis reading (the pages are silent): each token carries three integer
position ids (text (i,0,0), image (0,row,col), reference k (k,row,col)).  The
head dimension is cut into three contiguous slices of widths axes_dim =
(d0, d1, d2); slice a is rotated with its own axis' position and its own
frequencies theta^(-2j/d_a), j = 0 .. d_a/2 - 1.  Pairs are adjacent elements
(2j, 2j+1) of a slice.
"""
import numpy as np


def rope_frequencies(axes_dim, theta=10000.0):
    """Per-pair angular frequencies, length sum(axes_dim)/2, fp64.

    Pair j of axis a (within the slice) has frequency theta ** (-2j / d_a).
    """
    freqs = []
    for d in axes_dim:
        if d % 2:
            raise ValueError("each axis width must be even")
        j = np.arange(d // 2, dtype=np.float64)
        freqs.append(np.power(np.float64(theta), -2.0 * j / d) if d else np.zeros(0))
    return np.concatenate(freqs)


def rope_angles(pos, axes_dim, theta=10000.0):
    """Angles [N, D/2] fp64: angle of pair p of token n = pos[n, axis(p)] * freq[p]."""
    pos = np.asarray(pos, dtype=np.float64)
    freqs = rope_frequencies(axes_dim, theta)
    axis_of_pair = np.concatenate([np.full(d // 2, a, dtype=np.int64)
                                   for a, d in enumerate(axes_dim)])
    return pos[:, axis_of_pair] * freqs[None, :]


def apply_rope(x, pos, axes_dim, theta=10000.0):
    """Rotate x [B, N, H, D] (fp64) by its tokens' angles; returns a new array.

    (x0, x1) -> (x0 cos a - x1 sin a,  x0 sin a + x1 cos a) for every pair.
    """
    x = np.asarray(x, dtype=np.float64)
    B, N, H, D = x.shape
    if sum(axes_dim) != D:
        raise ValueError("axes_dim must sum to head_dim")
    ang = rope_angles(pos, axes_dim, theta)          # [N, D/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
