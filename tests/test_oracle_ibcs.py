"""Pins for the oracle's intra-block clustering scorer (CPU only): the one-group
case against the plain scorer, exact two-cluster blocks against a direct
softmax mixture, tie and empty-group handling worked by hand, the fixed-point
rounding rule, plain fp64 Lloyd on raw rows against scikit-learn's KMeans, the
fixed-point reading against both wherever every assignment clears the derived
rounding margin, the k-means cost bound of rounded centroids, and the
invariants of the full score matrix."""

import numpy as np
import pytest
from scipy.special import softmax

from oracle import score, valid_counts
from oracle.ibcs import certified_agreement, cluster_block, fixed_point, group_mixture, lloyd_block, score_ibcs


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
    perm = np.arange(384, dtype=np.int32)
    perm[:300] = np.random.default_rng(6).permutation(300)
    for p in (None, perm):
        S, reps, sizes, _ = score_ibcs(q, k, 300, 64, 32, 0.9, 1, iters, p)
        S0, qb, _ = score(q, k, 300, 64, 32, 0.9, p)
        assert np.allclose(S, S0, rtol=1e-6, atol=1e-9)
        assert np.allclose(reps[:, :, :, 0, :], qb, rtol=1e-12, atol=1e-12)
        assert np.array_equal(sizes[..., 0], np.broadcast_to(valid_counts(300, 384, 64), sizes[..., 0].shape))


def test_fixed_point_rule():
    rows = np.array([[0.75, -0.1], [0.3, 0.2]])        # max |q| = 0.75 = 0.75 * 2^0 -> s = 11
    qi, s = fixed_point(rows)
    assert s == 11 and qi.tolist() == [[1536, -205], [614, 410]]
    qi, s = fixed_point(np.array([[3.0, 2.5, -1.0 / 4096]]))  # 3 = 0.75 * 2^2 -> s = 9
    assert s == 9 and qi.tolist() == [[1536, 1280, 0]]
    qi, s = fixed_point(np.array([[1.5 / 2048, 0.5 / 2048, 2.5 / 2048]]))  # 2.5/2048 -> e = -9, s = 20
    assert s == 20 and qi.tolist() == [[768, 256, 1280]]
    qi, s = fixed_point(np.array([[1.0, 0.5 ** 13, 3 * 0.5 ** 13]]))  # 1 = 0.5 * 2^1 -> s = 10: 0.125 -> 0, 0.375 -> 0
    assert s == 10 and qi.tolist() == [[1024, 0, 0]]
    qi, s = fixed_point(np.array([[1.0, 0.5 ** 11, 3 * 0.5 ** 11]]))  # halves round to even: 0.5 -> 0, 1.5 -> 2
    assert qi.tolist() == [[1024, 0, 2]]
    qi, s = fixed_point(np.zeros((2, 3)))
    assert s == 0 and not qi.any()
    assert np.abs(fixed_point(np.random.default_rng(0).standard_normal((128, 128)))[0]).max() <= 2048


def _lattice(rng, d):
    """A vector of multiples of 1/8 in [-2, 2]: sums of up to 128 copies are exact in fp64."""
    return rng.integers(-16, 17, d) / 8.0


def test_two_exact_clusters_mixture():
    rng = np.random.default_rng(1)
    d, nku = 8, 6
    a, b = _lattice(rng, d), _lattice(rng, d)
    rows = np.array([a] * 60 + [b] * 68)
    reps, sizes = cluster_block(rows, 2, 1)   # initial rows 0 (a) and 64 (b)
    assert np.array_equal(reps, np.array([a, b])) and list(sizes) == [60, 68]
    kb = rng.standard_normal((nku, d))
    n_j = np.array([32, 32, 32, 32, 17, 0], dtype=np.float64)
    got = group_mixture(reps, sizes / 128, kb, n_j, 0.8)
    logn = np.where(n_j > 0, np.log(np.maximum(n_j, 1)), -np.inf)
    want = 60 / 128 * softmax(0.8 * kb @ a + logn) + 68 / 128 * softmax(0.8 * kb @ b + logn)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)
    assert got[-1] == 0.0


def test_duplicate_initial_centroids_and_an_empty_group():
    # rows 0..69 = a and 70..127 = b: both initial rows (0 and 64) are a, so the
    # first assignment is a tie everywhere and goes to group 0; group 1 is empty
    # (zero representative) but keeps its centroid a, so the second assignment
    # splits a from b.
    rng = np.random.default_rng(2)
    d = 8
    a, b = _lattice(rng, d), _lattice(rng, d)
    while np.array_equal(a, b):
        b = _lattice(rng, d)
    rows = np.array([a] * 70 + [b] * 58)
    r1, s1, hist, qi = cluster_block(rows, 2, 1, history=True)
    assert list(s1) == [128, 0]
    assert not r1[1].any()
    assert np.allclose(r1[0], (70 * a + 58 * b) / 128, rtol=0, atol=1e-15)
    assert np.array_equal(hist[0][1], qi[0])          # the empty group kept its centroid
    expect = (2 * (70 * qi[0] + 58 * qi[70]) + 128) // 256
    assert np.array_equal(hist[0][0], expect)          # rounded mean, half up
    r2, s2 = cluster_block(rows, 2, 2)
    assert list(s2) == [58, 70]
    assert np.array_equal(r2, np.array([b, a]))


def test_fewer_rows_than_groups():
    rows = np.array([[0.0, 1.0], [2.0, 0.0], [5.0, 5.0]])
    # initial rows floor(g * 3 / 4) = 0, 0, 1, 2: group 1 duplicates group 0 and stays empty
    reps, sizes = cluster_block(rows, 4, 3)
    assert list(sizes) == [1, 0, 1, 1]
    assert np.array_equal(reps, np.array([rows[0], [0.0, 0.0], rows[1], rows[2]]))


def _separated(rng, groups, d=16, n=128, spread=3.0):
    """n rows around ``groups`` centres in contiguous runs, so the initial rows floor(g n / G) start
    in different clusters; unit Gaussian noise."""
    centres = rng.standard_normal((groups, d)) * spread
    return centres[(np.arange(n) * groups) // n] + rng.standard_normal((n, d))


LLOYD_CASES = ((4, 1), (4, 2), (4, 5), (2, 3), (8, 4), (3, 6))


def test_plain_lloyd_matches_scikit_learn_on_raw_rows():
    # the unrounded reading (plain fp64 Lloyd on the raw rows) against a library k-means
    KMeans = pytest.importorskip("sklearn.cluster").KMeans
    for groups, iters in LLOYD_CASES:
        rng = np.random.default_rng(100 + 10 * groups + iters)
        rows = _separated(rng, groups, spread=2.0)
        reps, sizes = lloyd_block(rows, groups, iters)
        assert sizes.min() > 0  # scikit-learn relocates empty clusters; keep them out of the comparison
        init = rows[[(g * 128) // groups for g in range(groups)]]
        km = KMeans(n_clusters=groups, init=init, n_init=1, max_iter=iters, tol=0.0,
                    algorithm="lloyd").fit(rows)
        # scikit-learn's centres are the means of its last assignment, as the representatives are
        assert np.allclose(reps, km.cluster_centers_, rtol=1e-9, atol=1e-9), (groups, iters)


def test_fixed_point_reading_matches_scikit_learn_on_certified_raw_rows():
    # the kernel's reading (rows and centroids on the 2^(e-11) grid) on raw, unsnapped rows: where every
    # assignment clears the derived rounding margin, its groups are scikit-learn's Lloyd groups
    KMeans = pytest.importorskip("sklearn.cluster").KMeans
    checked = 0
    for groups, iters in LLOYD_CASES:
        for seed in range(4):
            rng = np.random.default_rng(1000 * seed + 10 * groups + iters)
            rows = _separated(rng, groups)
            if not certified_agreement(rows, groups, iters):
                continue
            reps, sizes = cluster_block(rows, groups, iters)
            if sizes.min() == 0:
                continue
            init = rows[[(g * 128) // groups for g in range(groups)]]
            km = KMeans(n_clusters=groups, init=init, n_init=1, max_iter=iters, tol=0.0,
                        algorithm="lloyd").fit(rows)
            assert np.allclose(reps, km.cluster_centers_, rtol=1e-9, atol=1e-9), (groups, iters, seed)
            checked += 1
    assert checked >= 12, checked


def test_fixed_point_reading_equals_plain_lloyd_when_certified():
    # certified blocks: identical sizes and bit-identical representatives (same members, same sums)
    certified = 0
    for case in range(60):
        rng = np.random.default_rng(5000 + case)
        groups = (2, 4, 8)[case % 3]
        iters = (1, 3, 5)[(case // 3) % 3]
        spread = (3.0, 4.0, 6.0, 8.0)[(case // 9) % 4]
        d = (16, 64, 128)[case % 3]
        rows = _separated(rng, groups, d=d, n=(128, 97, 64)[case % 3], spread=spread)
        rows *= 10.0 ** rng.uniform(-3, 3)  # the grid follows the block's own magnitude
        if not certified_agreement(rows, groups, iters):
            continue
        certified += 1
        r1, s1 = cluster_block(rows, groups, iters)
        r2, s2 = lloyd_block(rows, groups, iters)
        assert np.array_equal(s1, s2), case
        assert np.array_equal(r1, r2), case
    assert certified >= 30, certified


def test_certification_bound_is_not_vacuous():
    # two rows a grid step apart from a third, with the centroid rounding able to swap them: the rule
    # must refuse to certify a block whose margins are below the rounding scale
    rows = np.array([[1.0, 0.0], [1.0 + 2.0 ** -12, 0.0], [1.0 + 2.0 ** -11, 0.0], [-1.0, 0.0]])
    assert not certified_agreement(rows, 2, 2)
    far = np.array([[1.0, 0.0], [1.01, 0.0], [-1.0, 0.0], [-1.01, 0.0]])
    assert certified_agreement(far, 2, 3)


def test_kmeans_cost_bound_with_rounded_centroids():
    # Lloyd's cost cannot rise by more than the centroid rounding: at most n d / 4 per iteration
    rng = np.random.default_rng(4)
    rows = rng.standard_normal((128, 32)) + np.repeat(rng.standard_normal((4, 32)) * 2, 32, axis=0)
    rng.shuffle(rows)
    _, _, hist, qi = cluster_block(rows, 4, 8, history=True)
    cost = [int(((qi[:, None, :] - c[None]) ** 2).sum(-1).min(axis=1).sum()) for c in hist]
    assert all(c2 <= c1 + 128 * 32 // 4 for c1, c2 in zip(cost, cost[1:])), cost
    assert cost[-1] < cost[0]


def test_score_matrix_invariants():
    q, k = _tiny(seed=7, N=300, N_pad=512)   # query blocks 5..7 of 64 rows hold no valid row
    S, reps, sizes, _ = score_ibcs(q, k, 300, 64, 32, 1.3, 4, 3)
    n_q = valid_counts(300, 512, 64)
    n_j = valid_counts(300, 512, 32)
    assert np.allclose(S.astype(np.float64).sum(-1), 1.0, atol=1e-6)
    assert np.all(S[..., n_j == 0] == 0)
    assert np.array_equal(sizes.sum(-1), np.broadcast_to(n_q, sizes.shape[:-1]))
    # an empty query block scores like the plain scorer's empty block (zero mean: mass in proportion to n_j)
    S0, _, _ = score(q, k, 300, 64, 32, 1.3)
    assert np.allclose(S[:, :, 5:], S0[:, :, 5:], rtol=1e-6)
    assert not reps[:, :, 5:].any()
    # more groups than one actually split these blocks
    assert np.all((sizes[:, :, :4] > 0).sum(-1) >= 2)
    # the subset form returns the same rows
    rows, r_sub, s_sub = score_ibcs(q, k, 300, 64, 32, 1.3, 4, 3, blocks=[(0, 1, 2), (0, 0, 6)])
    assert np.array_equal(rows[0], S[0, 1, 2]) and np.array_equal(rows[1], S[0, 0, 6])
    assert np.array_equal(s_sub[0], sizes[0, 1, 2]) and np.array_equal(r_sub[0], reps[0, 1, 2])


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
    S, reps, sizes, _ = score_ibcs(q, k, N, 64, 32, 0.6, 2, 2)
    assert list(sizes[0, 0, 0]) == [30, 34]
    n_j = np.array([min(32, max(0, N - 32 * j)) for j in range(Np // 32)], dtype=np.float64)
    kb = np.array([k[0, 0, 32 * j: 32 * j + int(n)].mean(axis=0) if n else np.zeros(d)
                   for j, n in enumerate(n_j)])
    logn = np.where(n_j > 0, np.log(np.maximum(n_j, 1)), -np.inf)
    want = 30 / 64 * softmax(0.6 * kb @ a + logn) + 34 / 64 * softmax(0.6 * kb @ b + logn)
    assert np.allclose(S[0, 0, 0], want, rtol=1e-6, atol=1e-9)


def test_centroid_rounding_half_up():
    # one group: the centroid after one iteration is the rounded mean of the fixed-point rows
    rows = np.array([[1.0, 1.0 / 1024, -1.0], [1.0, 0.0, -1.0], [0.0, 0.0, 0.0]])
    _, _, hist, qi = cluster_block(rows, 1, 1, history=True)
    assert qi.tolist() == [[1024, 1, -1024], [1024, 0, -1024], [0, 0, 0]]
    # means 682.67 -> 683, 0.33 -> 0, -682.67 -> -683
    assert hist[0][0].tolist() == [683, 0, -683]
    _, _, hist, _ = cluster_block(rows[:2], 1, 1, history=True)
    # means 1024, 0.5 -> 1 (half up), -1024
    assert hist[0][0].tolist() == [1024, 1, -1024]
    _, _, hist, _ = cluster_block(-rows[:2], 1, 1, history=True)
    assert hist[0][0].tolist() == [-1024, 0, 1024]  # -0.5 -> 0 (half up)
