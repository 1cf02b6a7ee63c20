"""Pins for the oracle's intra-block clustering scorer (CPU only): the one-group
case against the plain scorer, exact two-cluster blocks against a direct
softmax mixture, tie and empty-group handling worked by hand, Lloyd iterations
against scikit-learn's KMeans, the monotone k-means cost, and the invariants of
the full score matrix."""

import numpy as np
import pytest
from scipy.special import softmax

from oracle import score, valid_counts
from oracle.ibcs import cluster_block, group_mixture, score_ibcs


def _tiny(seed=0, B=1, H=2, N=300, N_pad=384, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N_pad, d)) * 0.7
    k = rng.standard_normal((B, H, N_pad, d)) * 0.7
    q[..., N:, :] = 0
    k[..., N:, :] = 0
    return q, k


@pytest.mark.parametrize("iters", [1, 3])
def test_one_group_is_the_plain_scorer(iters):
    q, k = _tiny()
    perm = np.random.default_rng(5).permutation(384).astype(np.int32)
    perm[300:] = np.arange(300, 384)
    perm[:300] = np.random.default_rng(6).permutation(300)
    for p in (None, perm):
        S, cent, sizes, _, _ = score_ibcs(q, k, 300, 64, 32, 0.9, 1, iters, p)
        S0, qb, _ = score(q, k, 300, 64, 32, 0.9, p)
        assert np.allclose(S, S0, rtol=1e-6, atol=1e-9)
        assert np.allclose(cent[:, :, :, 0, :], qb, rtol=1e-12, atol=1e-12)
        assert np.array_equal(sizes[..., 0], np.broadcast_to(valid_counts(300, 384, 64), sizes[..., 0].shape))


def _lattice(rng, d):
    """A vector of multiples of 1/8 in [-2, 2]: sums of up to 128 copies are exact in fp64."""
    return rng.integers(-16, 17, d) / 8.0


def test_two_exact_clusters_mixture():
    rng = np.random.default_rng(1)
    d, nku = 8, 6
    a, b = _lattice(rng, d), _lattice(rng, d)
    rows = np.array([a] * 60 + [b] * 68)
    cent, sizes, margin = cluster_block(rows, 2, 1)   # initial rows 0 (a) and 64 (b)
    assert np.array_equal(cent, np.array([a, b])) and list(sizes) == [60, 68]
    assert margin > 0.01
    kb = rng.standard_normal((nku, d))
    n_j = np.array([32, 32, 32, 32, 17, 0], dtype=np.float64)
    got = group_mixture(cent, sizes / 128, kb, n_j, 0.8)
    logn = np.where(n_j > 0, np.log(np.maximum(n_j, 1)), -np.inf)
    want = 60 / 128 * softmax(0.8 * kb @ a + logn) + 68 / 128 * softmax(0.8 * kb @ b + logn)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)
    assert got[-1] == 0.0


def test_duplicate_initial_centroids_and_an_empty_group():
    # rows 0..69 = a and 70..127 = b: both initial rows (0 and 64) are a, so the
    # first assignment is a tie everywhere and goes to group 0; group 1 is empty
    # and keeps a. The second assignment splits a from b.
    rng = np.random.default_rng(2)
    d = 8
    a, b = _lattice(rng, d), _lattice(rng, d)
    while np.array_equal(a, b):
        b = _lattice(rng, d)
    rows = np.array([a] * 70 + [b] * 58)
    c1, s1, m1 = cluster_block(rows, 2, 1)
    assert list(s1) == [128, 0]
    assert np.array_equal(c1[1], a)
    assert np.allclose(c1[0], (70 * a + 58 * b) / 128, rtol=0, atol=1e-15)
    assert m1 == np.inf  # every first assignment compared two identical centroids
    c2, s2, _ = cluster_block(rows, 2, 2)
    assert list(s2) == [58, 70]
    assert np.array_equal(c2, np.array([b, a]))


def test_fewer_rows_than_groups():
    rows = np.array([[0.0, 1.0], [2.0, 0.0], [5.0, 5.0]])
    # initial rows floor(g * 3 / 4) = 0, 0, 1, 2: group 1 duplicates group 0 and stays empty
    cent, sizes, _ = cluster_block(rows, 4, 3)
    assert list(sizes) == [1, 0, 1, 1]
    assert np.array_equal(cent, rows[[0, 0, 1, 2]])


def test_lloyd_iterations_match_scikit_learn():
    KMeans = pytest.importorskip("sklearn.cluster").KMeans
    rng = np.random.default_rng(3)
    centres = rng.standard_normal((3, 16)) * 3
    rows = centres[rng.integers(0, 3, 128)] + rng.standard_normal((128, 16))
    for groups, iters in ((4, 1), (4, 2), (4, 5), (2, 3), (8, 4)):
        cent, sizes, _ = cluster_block(rows, groups, iters)
        assert sizes.min() > 0  # scikit-learn relocates empty clusters; keep them out of the comparison
        init = rows[[(g * 128) // groups for g in range(groups)]]
        km = KMeans(n_clusters=groups, init=init, n_init=1, max_iter=iters, tol=0.0,
                    algorithm="lloyd").fit(rows)
        assert np.allclose(cent, km.cluster_centers_, rtol=1e-9, atol=1e-9), (groups, iters)


def test_kmeans_cost_never_increases():
    rng = np.random.default_rng(4)
    rows = rng.standard_normal((128, 32)) + np.repeat(rng.standard_normal((4, 32)) * 2, 32, axis=0)
    rng.shuffle(rows)
    cost = []
    for iters in range(1, 8):
        cent, _, _ = cluster_block(rows, 4, iters)
        cost.append(((rows[:, None, :] - cent[None]) ** 2).sum(-1).min(axis=1).sum())
    assert all(c2 <= c1 * (1 + 1e-12) for c1, c2 in zip(cost, cost[1:])), cost


def test_score_matrix_invariants():
    q, k = _tiny(seed=7, N=300, N_pad=512)   # query blocks 5..7 of 64 rows hold no valid row
    S, cent, sizes, margins, _ = score_ibcs(q, k, 300, 64, 32, 1.3, 4, 3)
    n_q = valid_counts(300, 512, 64)
    n_j = valid_counts(300, 512, 32)
    assert np.allclose(S.astype(np.float64).sum(-1), 1.0, atol=1e-6)
    assert np.all(S[..., n_j == 0] == 0)
    assert np.array_equal(sizes.sum(-1), np.broadcast_to(n_q, sizes.shape[:-1]))
    # an empty query block scores like the plain scorer's empty block (zero mean: mass in proportion to n_j)
    S0, _, _ = score(q, k, 300, 64, 32, 1.3)
    assert np.allclose(S[:, :, 5:], S0[:, :, 5:], rtol=1e-6)
    # more groups than one actually split these blocks
    assert np.all((sizes[:, :, :4] > 0).sum(-1) >= 2)
    # the subset form returns the same rows
    rows, c_sub, s_sub, m_sub = score_ibcs(q, k, 300, 64, 32, 1.3, 4, 3, blocks=[(0, 1, 2), (0, 0, 6)])
    assert np.array_equal(rows[0], S[0, 1, 2]) and np.array_equal(rows[1], S[0, 0, 6])
    assert np.array_equal(s_sub[0], sizes[0, 1, 2]) and m_sub[0] == margins[0, 1, 2]


def test_full_scorer_weights_groups_by_size():
    # query block 0 (64 rows) holds exactly two vectors: a in rows 0..29, b in rows 30..63;
    # the initial rows 0 and 32 split them at once, so S_0j = 30/64 m_a(j) + 34/64 m_b(j)
    rng = np.random.default_rng(8)
    d, N, Np = 8, 200, 256
    a, b = _lattice(rng, d), _lattice(rng, d)
    q = rng.standard_normal((1, 1, Np, d))
    q[0, 0, :30], q[0, 0, 30:64] = a, b
    k = rng.standard_normal((1, 1, Np, d))
    k[..., N:, :] = 0
    q[..., N:, :] = 0
    S, cent, sizes, _, _ = score_ibcs(q, k, N, 64, 32, 0.6, 2, 2)
    assert list(sizes[0, 0, 0]) == [30, 34]
    n_j = np.array([min(32, max(0, N - 32 * j)) for j in range(Np // 32)], dtype=np.float64)
    kb = np.array([k[0, 0, 32 * j: 32 * j + int(n)].mean(axis=0) if n else np.zeros(d)
                   for j, n in enumerate(n_j)])
    logn = np.where(n_j > 0, np.log(np.maximum(n_j, 1)), -np.inf)
    want = 30 / 64 * softmax(0.6 * kb @ a + logn) + 34 / 64 * softmax(0.6 * kb @ b + logn)
    assert np.allclose(S[0, 0, 0], want, rtol=1e-6, atol=1e-9)
