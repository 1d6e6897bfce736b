"""Tile-sparse joint RoPE attention, fp64 (oracle; test infrastructure).

Source: "Optimizing FLUX 3 Image Klein inference on NVIDIA Blackwell GPUs",
How it works: sparse attention skips the work for less important token pairs
according to a sparsity threshold (tau, What you can do), after some dense
denoising steps.  The pages give neither the importance measure nor the
granularity; the reading used here, by both sides:

  * granularity: query tiles of 256 tokens x key tiles of 64 tokens of the
    joint sequence (the attention kernel's tiles; the last tile of each kind
    may be partial);
  * attention: exact softmax attention of each query over the keys of the
    kept key tiles of its query tile; the other keys are left out, not
    approximated.

Two rules decide the kept tiles (c = scale * log2(e), scores in the exp2
domain, s_ij = c <R(p_i) q_i, R(p_j) k_j>):

  * score-bound rule (``tile_score_maxima``, ``bound_mask``): a key tile t is
    skipped for query tile Q when, for every query i of Q, the largest score
    of i over t is below L_i + log2(tau), where L_i is i's largest score over
    the key tiles aligned with Q (its own 256 positions), a lower bound of
    i's row maximum m_i.  Then every skipped pair has weight
    2^(s_ij - m_i) < tau relative to its row's largest, and the distance from
    dense attention is bounded (``skip_mass_bound``, ``dense_error_bound``):
    with delta_i the dense softmax mass of row i's skipped keys,
        O_sparse - O_dense = delta_i (O_kept - O_skipped),
        |O_sparse - O_dense|[i, d] <= delta_i (max_j V[j, d] - min_j V[j, d]),
        delta_i <= sum over skipped tiles t of n_t 2^(smax_it - m_i)
                <  tau * (number of skipped keys of row i);
  * pooled-score rule (``block_scores``, ``block_mask``), an alternative
    without that guarantee: a key tile is kept when its pooled score
    c <mean_i R(p_i) q_i, mean_j R(p_j) k_j> is at least the query tile's
    largest pooled score plus log2(tau).

Rules are computed here in fp64; a decision within rounding of the threshold
may legitimately come out the other way in lower precision, so both rules
also return the margin of each decision.
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


def _tile_ranges(n, tile):
    return [(t * tile, min((t + 1) * tile, n)) for t in range((n + tile - 1) // tile)]


def tile_score_maxima(q, k, pos, axes_dim, k_tile=64, theta=10000.0, scale=None, row_block=1024):
    """Largest score of every query over every key tile, and every row's maximum.

    Returns (smax [B, H, N, KT], m [B, H, N]) in the exp2 domain:
    smax[b, h, i, t] = max over keys j of tile t of c * <R(p_i) q_i, R(p_j) k_j>.
    """
    q = np.asarray(q, dtype=np.float64)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    c = scale * LOG2E
    qr = apply_rope(q, pos, axes_dim, theta)
    kr = apply_rope(k, pos, axes_dim, theta)
    kts = _tile_ranges(N, k_tile)
    smax = np.empty((B, H, N, len(kts)))
    for b in range(B):
        for h in range(H):
            kh = kr[b, :, h, :]
            for r0 in range(0, N, row_block):
                s = c * (qr[b, r0:r0 + row_block, h, :] @ kh.T)
                for t, (j0, j1) in enumerate(kts):
                    smax[b, h, r0:r0 + row_block, t] = s[:, j0:j1].max(axis=1)
    return smax, smax.max(axis=-1)


def bound_mask(smax, tau, q_tile=256, k_tile=64):
    """The score-bound skip rule (see the module docstring).

    smax: [B, H, N, KT] from ``tile_score_maxima``.  Returns (mask, margin),
    bool and fp64 [B, H, QT, KT]: margin[Q, t] = max over queries i of Q of
    (smax[i, t] - L_i), L_i = max of smax[i, t'] over the key tiles t' aligned
    with Q; a tile is kept when margin >= log2(tau).  For every query, the
    aligned tile that attains its L_i has margin >= 0 and is kept, so no
    query is left without keys.
    """
    if not 0.0 < tau <= 1.0:
        raise ValueError("tau must be in (0, 1]")
    smax = np.asarray(smax, dtype=np.float64)
    B, H, N, KT = smax.shape
    per = q_tile // k_tile
    qts = _tile_ranges(N, q_tile)
    margin = np.empty((B, H, len(qts), KT))
    for qt, (i0, i1) in enumerate(qts):
        own = smax[:, :, i0:i1, qt * per:min((qt + 1) * per, KT)]
        low = own.max(axis=-1, keepdims=True)                    # L_i <= m_i
        margin[:, :, qt, :] = (smax[:, :, i0:i1, :] - low).max(axis=2)
    return margin >= np.log2(tau), margin


def _expand_mask(mask, n, q_tile=256, k_tile=64):
    """Tile mask [B, H, QT, KT] -> pair mask [B, H, N, N]."""
    m = np.repeat(np.repeat(np.asarray(mask, dtype=bool), q_tile, axis=2)[:, :, :n], k_tile, axis=3)
    return m[:, :, :, :n]


def skipped_mass(q, k, pos, axes_dim, mask, q_tile=256, k_tile=64, theta=10000.0, scale=None):
    """delta [B, H, N]: the dense softmax probability mass of each row's skipped keys."""
    q = np.asarray(q, dtype=np.float64)
    B, N, H, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    qr = apply_rope(q, pos, axes_dim, theta)
    kr = apply_rope(k, pos, axes_dim, theta)
    delta = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            keep = _expand_mask(np.asarray(mask)[b:b + 1, h:h + 1], N, q_tile, k_tile)[0, 0]
            s = scale * (qr[b, :, h, :] @ kr[b, :, h, :].T)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            delta[b, h] = (p * ~keep).sum(axis=1) / p.sum(axis=1)
    return delta


def skip_mass_bound(smax, m, mask, n_keys_per_tile, q_tile=256):
    """B_i = sum over the key tiles t skipped for row i of n_t 2^(smax_it - m_i),
    an upper bound of delta_i (the row's softmax normaliser is at least 1)."""
    smax = np.asarray(smax, dtype=np.float64)
    B, H, N, KT = smax.shape
    skip = ~np.repeat(np.asarray(mask, dtype=bool), q_tile, axis=2)[:, :, :N]     # [B, H, N, KT]
    w = np.exp2(smax - np.asarray(m)[..., None]) * np.asarray(n_keys_per_tile, dtype=np.float64)
    return (w * skip).sum(axis=-1)


def dense_error_bound(delta, v):
    """Per-element bound of |O_sparse - O_dense|: delta_i (max_j V[j,d] - min_j V[j,d]),
    [B, N, H, D] for delta [B, H, N] and v [B, N, H, D]."""
    v = np.asarray(v, dtype=np.float64)
    rng = v.max(axis=1) - v.min(axis=1)                       # [B, H, D]
    return np.transpose(np.asarray(delta), (0, 2, 1))[..., None] * rng[:, None, :, :]
