"""Non-causal joint softmax attention with RoPE, fp64 (oracle; test infrastructure).

Sources:
  * "Welcome FLUX.3 Image Klein in Diffusers", Architecture section, "Two-Stage
    Processing": in the joint blocks the text, noisy-image and reference streams
    are concatenated and attend together.  Reading: joint *self*-attention, every
    token attends to every token of the one concatenated sequence, no mask.
  * "FLUX.3 Image Klein Brings 2-Second AI Image Generation to Diffusers",
    Summary: five separate-stream blocks precede the 28 joint blocks; the
    separate-stream stage is the segment-local variant below (each segment
    attends only within itself).
  * "Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell GPUs", "How it
    works": attention dominates GPU kernel time at high resolution.

Definition (softmax attention, Vaswani et al. 2017): for each batch b and head h
    S = scale * Q~ K~^T,  P = softmax over keys of S,  O = P V,
with Q~, K~ the rotary-embedded Q and K (``rope.apply_rope``), V unrotated and
scale = 1/sqrt(D) unless given.  Layout of every tensor: [B, N, H, D].

The only blocking is over query rows (``row_block`` rows of S live at a time);
each row is computed exactly as the definition states, with dense matrix
products as library steps.
"""
import numpy as np

from .rope import apply_rope


def softmax_rows(s):
    """Row softmax of a 2-D fp64 array: exp(s - rowmax) / sum(exp(s - rowmax))."""
    s = np.asarray(s, dtype=np.float64)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_from_scores(s, v):
    """O = softmax(s) v for one (batch, head): s [M, N], v [N, Dv]."""
    return softmax_rows(s) @ np.asarray(v, dtype=np.float64)


def _default_scale(d):
    return 1.0 / np.sqrt(d)


def attention(q, k, v, scale=None, row_block=1024, rows=None):
    """Softmax attention over already-rotated q, k (fp64 [B,N,H,D]).

    rows: optional sorted array of query indices; only those output rows are
    computed (returns [B, len(rows), H, D]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, D = k.shape
    scale = _default_scale(D) if scale is None else float(scale)
    if rows is not None:
        q = q[:, np.asarray(rows)]
    M = q.shape[1]
    out = np.empty((B, M, H, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kh = np.ascontiguousarray(k[b, :, h, :])
            vh = np.ascontiguousarray(v[b, :, h, :])
            for r0 in range(0, M, row_block):
                qh = q[b, r0:r0 + row_block, h, :]
                s = scale * (qh @ kh.T)
                out[b, r0:r0 + row_block, h, :] = attention_from_scores(s, vh)
    return out


def joint_rope_attention(q, k, v, pos, axes_dim, theta=10000.0, scale=None, row_block=1024):
    """Joint self-attention with RoPE on Q and K over the whole sequence."""
    qr = apply_rope(q, pos, axes_dim, theta)
    kr = apply_rope(k, pos, axes_dim, theta)
    return attention(qr, kr, v, scale, row_block)


def joint_rope_attention_rows(q, k, v, pos, axes_dim, rows, theta=10000.0, scale=None):
    """Output rows ``rows`` of ``joint_rope_attention`` (each row is exact)."""
    rows = np.asarray(rows)
    pos = np.asarray(pos)
    qr = apply_rope(np.asarray(q, dtype=np.float64)[:, rows], pos[rows], axes_dim, theta)
    kr = apply_rope(k, pos, axes_dim, theta)
    return attention(qr, kr, v, scale)


def segment_local_rope_attention(q, k, v, pos, segment_tokens, axes_dim, theta=10000.0,
                                 scale=None):
    """Separate-stream attention: tokens attend only within their own segment.

    Segments are consecutive ranges of lengths ``segment_tokens``; the result for
    a segment is ``joint_rope_attention`` restricted to that segment's tokens.
    """
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[-1]
    scale = _default_scale(D) if scale is None else scale
    out = np.empty(q.shape, dtype=np.float64)
    t0 = 0
    pos = np.asarray(pos)
    for n in segment_tokens:
        sl = slice(t0, t0 + n)
        if n:
            out[:, sl] = joint_rope_attention(q[:, sl], np.asarray(k)[:, sl], np.asarray(v)[:, sl],
                                              pos[sl], axes_dim, theta, scale)
        t0 += n
    return out
