"""Tile-sparse joint RoPE attention, fp64 (oracle; test infrastructure).

Source: "Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell GPUs",
How it works: sparse attention skips the work for less important token pairs
according to a sparsity threshold (tau, What you can do), after some dense
denoising steps.  The pages give neither the importance measure nor the
granularity; the reading used here, by both sides:

  * granularity: query tiles of 256 tokens x key tiles of 64 tokens of the
    joint sequence (the attention kernel's tiles; the last tile of each kind
    may be partial);
  * importance of a tile pair: the pooled score  c * <mean_i R(p_i) q_i,
    mean_j R(p_j) k_j>,  means over the tiles' tokens of the rotated vectors,
    c = scale * log2(e) (exp2 domain);
  * rule: a key tile is kept for a query tile when its pooled score is at
    least the query tile's largest pooled score plus log2(tau), tau in (0, 1];
    the largest one is always kept;
  * attention: exact softmax attention of each query over the keys of the
    kept key tiles of its query tile; the other keys are left out, not
    approximated.

The rule is computed here in fp64; a decision within rounding of the
threshold may legitimately come out the other way in lower precision, so
``block_scores`` also returns the margin of each decision.
"""
import numpy as np

from .rope import apply_rope
from .softmax_attention import attention_from_scores

LOG2E = 1.4426950408889634


def tile_means(x_rot, tile):
    """Mean over the tokens of each tile: x_rot [B, N, H, D] -> [B, T, H, D]."""
    x_rot = np.asarray(x_rot, dtype=np.float64)
    B, N, H, D = x_rot.shape
    T = (N + tile - 1) // tile
    out = np.empty((B, T, H, D))
    for t in range(T):
        out[:, t] = x_rot[:, t * tile:(t + 1) * tile].mean(axis=1)
    return out


def block_scores(q, k, pos, axes_dim, q_tile=256, k_tile=64, theta=10000.0, scale=None):
    """Pooled scores [B, H, QT, KT] in the exp2 domain (see module docstring)."""
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[-1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    qm = tile_means(apply_rope(q, pos, axes_dim, theta), q_tile)   # [B, QT, H, D]
    km = tile_means(apply_rope(k, pos, axes_dim, theta), k_tile)   # [B, KT, H, D]
    return scale * LOG2E * np.einsum("bqhd,bkhd->bhqk", qm, km)


def block_mask(scores, tau):
    """Kept tiles: score >= row max + log2(tau).  Returns (mask, margin)."""
    if not 0.0 < tau <= 1.0:
        raise ValueError("tau must be in (0, 1]")
    scores = np.asarray(scores, dtype=np.float64)
    margin = scores - (scores.max(axis=-1, keepdims=True) + np.log2(tau))
    return margin >= 0.0, margin


def block_sparse_attention(q, k, v, pos, axes_dim, mask, q_tile=256, k_tile=64, theta=10000.0,
                           scale=None, rows=None):
    """Attention of each query over the keys of its query tile's kept key tiles.

    mask: bool [B, H, QT, KT].  A query tile without kept key tiles gets output 0.
    rows: optional query indices; returns [B, len(rows), H, Dv] then.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    qr = apply_rope(q, pos, axes_dim, theta)
    kr = apply_rope(k, pos, axes_dim, theta)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.zeros((B, len(rows), H, v.shape[-1]))
    KT = (N + k_tile - 1) // k_tile
    for b in range(B):
        for h in range(H):
            for qt in np.unique(rows // q_tile):
                sel = np.nonzero(rows // q_tile == qt)[0]
                kept = [t for t in range(KT) if mask[b, h, qt, t]]
                if not kept:
                    continue
                keys = np.concatenate([np.arange(t * k_tile, min((t + 1) * k_tile, N)) for t in kept])
                s = scale * (qr[b, rows[sel], h, :] @ kr[b, keys, h, :].T)
                out[b, sel, h, :] = attention_from_scores(s, v[b, keys, h, :])
    return out
