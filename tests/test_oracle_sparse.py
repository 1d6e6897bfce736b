"""Pins of the tile-sparse oracle (oracle/block_sparse.py) against facts that do
not come from it: a hand-worked mask, the extremes of tau, bilinearity of the
pooled score (the mean of the per-pair scores of the full score matrix), an
all-kept mask reducing to the dense oracle, brute-force loops on tiny inputs
and torch's scaled_dot_product_attention with the equivalent boolean mask.
A mutation check plants plausible mistakes in copies of the functions.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import block_sparse as obs

AXES = (8, 12, 12)  # D = 32


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _pos(n, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 40, size=(n, 3)).astype(np.int32)


def test_hand_worked_mask():
    # D = 2, RoPE off (positions 0), scale 1: q tiles of 2 tokens, k tiles of 1.
    # q tile 0 = rows (1, 0), (3, 0): mean (2, 0); q tile 1 = (0, 1), (0, 3): mean (0, 2).
    # keys (1, 0), (0, 1), (1, 1): pooled dots: tile 0 -> 2, 0, 2; tile 1 -> 0, 2, 2.
    q = np.array([[1, 0], [3, 0], [0, 1], [0, 3]], float).reshape(1, 4, 1, 2)
    k = np.array([[1, 0], [0, 1], [1, 1]], float).reshape(1, 3, 1, 2)
    pos = np.zeros((4, 3), np.int32)
    s = obs.block_scores(q, np.concatenate([k, np.zeros((1, 1, 1, 2))], axis=1), pos, (0, 0, 2),
                         q_tile=2, k_tile=1, scale=1.0)
    l2e = 1.0 / math.log(2.0)
    np.testing.assert_allclose(s[0, 0], l2e * np.array([[2, 0, 2, 0], [0, 2, 2, 0]]), rtol=1e-15)
    mask, margin = obs.block_mask(s, tau=0.25)   # keep score >= max - 2 (exp2 domain)
    # max = 2 * l2e = 2.885; threshold 0.885: keys with pooled dot 2 kept, 0 dropped
    assert mask[0, 0].tolist() == [[True, False, True, False], [False, True, True, False]]
    np.testing.assert_allclose(margin[0, 0, 0, 0], 2.0, rtol=1e-14)


def test_tau_extremes():
    q, k = _rand((2, 50, 3, 32), 1), _rand((2, 50, 3, 32), 2)
    pos = _pos(50)
    s = obs.block_scores(q, k, pos, AXES, q_tile=16, k_tile=8)
    m1, _ = obs.block_mask(s, 1.0)
    assert (m1 == (s == s.max(axis=-1, keepdims=True))).all()
    assert m1.sum(axis=-1).min() >= 1
    m0, _ = obs.block_mask(s, 1e-300)
    assert m0.all()
    with pytest.raises(ValueError):
        obs.block_mask(s, 0.0)


def test_pooled_score_is_mean_of_pair_scores():
    # Bilinearity: <mean q, mean k> is the mean over the tile pair of <q_i, k_j>.
    B, N, H, D = 1, 37, 2, 32
    q, k = _rand((B, N, H, D), 3), _rand((B, N, H, D), 4)
    pos = _pos(N, 1)
    qr, kr = oracle.apply_rope(q, pos, AXES), oracle.apply_rope(k, pos, AXES)
    full = np.einsum("bihd,bjhd->bhij", qr, kr) / math.sqrt(D) / math.log(2.0)
    s = obs.block_scores(q, k, pos, AXES, q_tile=10, k_tile=6)
    for qt in range(4):
        for kt in range(7):
            blk = full[:, :, qt * 10:(qt + 1) * 10, kt * 6:(kt + 1) * 6]
            np.testing.assert_allclose(s[:, :, qt, kt], blk.mean(axis=(-1, -2)), rtol=1e-12, atol=1e-12)


def test_all_kept_equals_dense_oracle():
    B, N, H, D = 1, 45, 2, 32
    q, k, v = _rand((B, N, H, D), 5), _rand((B, N, H, D), 6), _rand((B, N, H, D), 7)
    pos = _pos(N, 2)
    mask = np.ones((B, H, 3, 6), bool)
    got = obs.block_sparse_attention(q, k, v, pos, AXES, mask, q_tile=16, k_tile=8)
    np.testing.assert_allclose(got, oracle.joint_rope_attention(q, k, v, pos, AXES), rtol=1e-12, atol=1e-13)


def _brute(q, k, v, pos, mask, qt_sz, kt_sz):
    """Triple loops: masked scores set aside, softmax written out."""
    qr, kr = oracle.apply_rope(q, pos, AXES), oracle.apply_rope(k, pos, AXES)
    B, N, H, D = q.shape
    out = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                w = []
                for j in range(N):
                    if mask[b, h, i // qt_sz, j // kt_sz]:
                        w.append((sum(qr[b, i, h, d] * kr[b, j, h, d] for d in range(D)) / math.sqrt(D), j))
                if not w:
                    continue
                mx = max(x for x, _ in w)
                z = sum(math.exp(x - mx) for x, _ in w)
                for x, j in w:
                    out[b, i, h] += math.exp(x - mx) / z * v[b, j, h]
    return out


def test_brute_force_tiny():
    B, N, H, D = 1, 11, 2, 32
    q, k, v = _rand((B, N, H, D), 8), _rand((B, N, H, D), 9), _rand((B, N, H, D), 10)
    pos = _pos(N, 3)
    rng = np.random.default_rng(11)
    mask = rng.random((B, H, 3, 4)) < 0.5
    mask[0, 0, 2] = False          # a query tile with nothing kept -> zeros
    mask[0, 1, :, 0] = True
    got = obs.block_sparse_attention(q, k, v, pos, AXES, mask, q_tile=4, k_tile=3)
    np.testing.assert_allclose(got, _brute(q, k, v, pos, mask, 4, 3), rtol=1e-11, atol=1e-12)
    assert np.all(got[0, 8:, 0] == 0.0)


def test_torch_sdpa_with_boolean_mask():
    torch = pytest.importorskip("torch")
    B, N, H, D = 1, 70, 2, 32
    q, k, v = _rand((B, N, H, D), 12), _rand((B, N, H, D), 13), _rand((B, N, H, D), 14)
    pos = _pos(N, 4)
    rng = np.random.default_rng(15)
    mask = rng.random((B, H, 3, 9)) < 0.4
    mask[..., 0] = True
    got = obs.block_sparse_attention(q, k, v, pos, AXES, mask, q_tile=32, k_tile=8)
    qr, kr = oracle.apply_rope(q, pos, AXES), oracle.apply_rope(k, pos, AXES)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3)))
    tok_mask = np.repeat(np.repeat(mask, 32, axis=2)[:, :, :N], 8, axis=3)[:, :, :, :N]
    ref = torch.nn.functional.scaled_dot_product_attention(t(qr), t(kr), t(v), attn_mask=torch.from_numpy(tok_mask))
    np.testing.assert_allclose(got, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-12)


def test_mutations_are_caught():
    B, N, H, D = 1, 11, 2, 32
    q, k, v = _rand((B, N, H, D), 16), _rand((B, N, H, D), 17), _rand((B, N, H, D), 18)
    pos = _pos(N, 5)
    mask = np.random.default_rng(19).random((B, H, 3, 4)) < 0.6
    mask[..., 0] = True
    ref = _brute(q, k, v, pos, mask, 4, 3)
    orig = obs.block_sparse_attention

    def off_by_one_tile(q, k, v, pos, axes, m, q_tile, k_tile, **kw):
        return orig(q, k, v, pos, axes, np.roll(m, 1, axis=-1), q_tile, k_tile, **kw)

    def transposed_mask(q, k, v, pos, axes, m, q_tile, k_tile, **kw):
        m2 = np.zeros_like(m)
        n = min(m.shape[-1], m.shape[-2])
        m2[..., :n, :n] = np.swapaxes(m[..., :n, :n], -1, -2)
        return orig(q, k, v, pos, axes, m2 | (np.arange(m.shape[-1]) == 0), q_tile, k_tile, **kw)

    for bad in (off_by_one_tile, transposed_mask):
        got = bad(q, k, v, pos, AXES, mask, 4, 3)
        assert not np.allclose(got, ref, rtol=1e-6, atol=1e-8), bad.__name__
    s = obs.block_scores(q, k, pos, AXES, q_tile=4, k_tile=3)
    m_good, _ = obs.block_mask(s, 0.3)
    m_wrong_sign = s <= s.max(axis=-1, keepdims=True) + math.log2(0.3)
    assert (m_good != m_wrong_sign).any()


# ----------------------------------------------------------------------------------
# score-bound rule: guarantee and error bound against dense attention

def _peaked(n=72, h=2, seed=30, sigma=3.0, a=0.95):
    """Q and K sharing a per-head direction, positions along one axis: with
    RoPE the scores peak near equal positions, so far tiles can be skipped."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((1, 1, h, 32))
    b = math.sqrt(1 - a * a)
    q = sigma * (a * u + b * rng.standard_normal((1, n, h, 32)))
    k = sigma * (a * u + b * rng.standard_normal((1, n, h, 32)))
    v = rng.standard_normal((1, n, h, 32))
    pos = np.zeros((n, 3), np.int32)
    pos[:, 2] = np.arange(n)
    return q, k, v, pos


def _scores_loop(q, k, pos, b, h):
    """exp2-domain scores by explicit loops over a rotation written as 2x2 matrices."""
    n, D = q.shape[1], q.shape[3]
    freqs = []
    for d in AXES:
        freqs += [10000.0 ** (-2.0 * j / d) for j in range(d // 2)]
    axis = [a for a, d in enumerate(AXES) for _ in range(d // 2)]
    def rot(x, p):
        out = np.empty(D)
        for j in range(D // 2):
            ang = p[axis[j]] * freqs[j]
            cs, sn = math.cos(ang), math.sin(ang)
            out[2 * j] = cs * x[2 * j] - sn * x[2 * j + 1]
            out[2 * j + 1] = sn * x[2 * j] + cs * x[2 * j + 1]
        return out
    qr = [rot(q[b, i, h], pos[i]) for i in range(n)]
    kr = [rot(k[b, j, h], pos[j]) for j in range(n)]
    c = 1.0 / math.sqrt(D) / math.log(2.0)
    return np.array([[c * float(np.dot(qr[i], kr[j])) for j in range(n)] for i in range(n)])


def test_bound_rule_brute_force():
    q, k, v, pos = _peaked()
    n, qs, ks = q.shape[1], 16, 4
    smax, m = obs.tile_score_maxima(q, k, pos, AXES, k_tile=ks)
    mask, margin = obs.bound_mask(smax, 0.1, q_tile=qs, k_tile=ks)
    for h in range(2):
        s = _scores_loop(q, k, pos, 0, h)
        for qt in range((n + qs - 1) // qs):
            rows = range(qt * qs, min(n, (qt + 1) * qs))
            own = range(qt * qs // ks, min((n + ks - 1) // ks, (qt + 1) * qs // ks))
            low = {i: max(s[i, j] for t in own for j in range(t * ks, min(n, (t + 1) * ks))) for i in rows}
            for t in range((n + ks - 1) // ks):
                keys = range(t * ks, min(n, (t + 1) * ks))
                want = max(s[i, j] - low[i] for i in rows for j in keys)
                assert abs(margin[0, h, qt, t] - want) < 1e-9
                assert mask[0, h, qt, t] == (want >= math.log2(0.1))
        np.testing.assert_allclose(m[0, h], s.max(axis=1), rtol=0, atol=1e-10)


@pytest.mark.parametrize("tau", [0.3, 0.1, 0.01])
def test_bound_rule_guarantee_and_dense_error_bound(tau):
    q, k, v, pos = _peaked()
    n, qs, ks = q.shape[1], 16, 4
    smax, m = obs.tile_score_maxima(q, k, pos, AXES, k_tile=ks)
    mask, _ = obs.bound_mask(smax, tau, q_tile=qs, k_tile=ks)
    per = qs // ks
    for qt in range(mask.shape[2]):                      # every query keeps its best aligned tile
        best = qt * per + smax[:, :, qt * qs:(qt + 1) * qs, qt * per:(qt + 1) * per].argmax(axis=-1)
        for h in range(2):
            assert mask[0, h, qt, best[0, h]].all()
    keep = obs._expand_mask(mask, n, qs, ks)
    if tau <= 0.1:
        assert (~mask).mean() > 0.2                      # the rule does skip tiles here
    deltas = obs.skipped_mass(q, k, pos, AXES, mask, q_tile=qs, k_tile=ks)
    for h in range(2):
        s = _scores_loop(q, k, pos, 0, h)
        rel = np.exp2(s - s.max(axis=1, keepdims=True))  # weight relative to the row's largest
        assert (rel[~keep[0, h]] < tau).all()            # the guarantee, pair by pair
        p = rel / rel.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(deltas[0, h], (p * ~keep[0, h]).sum(axis=1), rtol=1e-12, atol=1e-15)
    nk = np.array([min(ks, n - t * ks) for t in range(mask.shape[3])])
    bound = obs.skip_mass_bound(smax, m, mask, nk, q_tile=qs)
    skipped_keys = (~keep).sum(axis=-1)
    assert (deltas <= bound * (1 + 1e-12)).all()
    assert (bound <= tau * skipped_keys + 1e-15).all()
    dense = oracle.joint_rope_attention(q, k, v, pos, AXES)
    sparse = obs.block_sparse_attention(q, k, v, pos, AXES, mask, q_tile=qs, k_tile=ks)
    eb = obs.dense_error_bound(deltas, v)
    assert (np.abs(sparse - dense) <= eb + 1e-13).all()
    # the bound is attained up to the spread of V: not vacuous
    if tau <= 0.1:
        assert np.abs(sparse - dense).max() > 0.05 * eb.max()


def test_bound_rule_tau_extremes():
    q, k, v, pos = _peaked()
    smax, _ = obs.tile_score_maxima(q, k, pos, AXES, k_tile=4)
    m1, mg = obs.bound_mask(smax, 1.0, q_tile=16, k_tile=4)
    assert (m1 == (mg >= 0.0)).all()
    m0, _ = obs.bound_mask(smax, 1e-300, q_tile=16, k_tile=4)
    assert m0.all()
    with pytest.raises(ValueError):
        obs.bound_mask(smax, 0.0)


def test_bound_rule_mutations_break_the_guarantee():
    # plausible mistakes in the rule: the smallest row instead of the largest
    # deciding a tile, or the lower bound taken from the whole row's minimum
    # tile; each must skip some pair whose weight reaches tau
    q, k, v, pos = _peaked()
    n, qs, ks, tau = q.shape[1], 16, 4, 0.1
    smax, m = obs.tile_score_maxima(q, k, pos, AXES, k_tile=ks)
    s = [_scores_loop(q, k, pos, 0, h) for h in range(2)]

    def violates(mask):
        keep = obs._expand_mask(mask, n, qs, ks)
        return any((np.exp2(s[h] - s[h].max(axis=1, keepdims=True))[~keep[0, h]] >= tau).any() for h in range(2))

    good, _ = obs.bound_mask(smax, tau, q_tile=qs, k_tile=ks)
    assert not violates(good)
    per = qs // ks
    bad_rows = np.empty_like(good)
    bad_low = np.empty_like(good)
    for qt in range(good.shape[2]):
        blk = smax[:, :, qt * qs:(qt + 1) * qs]
        low = blk[..., qt * per:(qt + 1) * per].max(axis=-1, keepdims=True)
        bad_rows[:, :, qt] = (blk - low).min(axis=2) >= math.log2(tau)
        bad_low[:, :, qt] = (blk - blk.max(axis=-1, keepdims=True)).max(axis=2) + 0.0 >= \
            math.log2(tau) + (blk.max(axis=-1) - blk.min(axis=-1)).mean(axis=2)[..., None]
    assert violates(bad_rows)
    assert violates(bad_low)
