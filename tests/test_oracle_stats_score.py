"""Pins for the oracle's statistics-aware scorer (CPU only): units of identical
keys reduce it to the plain scorer; the per-dimension variance against a
scalar brute force; its Gaussian moment-generating-function logit against the
Monte Carlo mean of exp over many Gaussian keys; spread raises a unit's score;
rows sum to 1 and invalid units score 0."""

import math

import numpy as np

from oracle import score, valid_counts
from oracle.stats_score import block_variances, score_stats


def test_identical_keys_give_the_plain_scorer():
    rng = np.random.default_rng(0)
    N, Np, d, bk = 200, 256, 8, 32
    q = rng.standard_normal((1, 2, Np, d))
    unit_vals = rng.standard_normal((1, 2, Np // bk, d))
    k = np.repeat(unit_vals, bk, axis=2)
    q[..., N:, :] = 0
    k[..., N:, :] = 0
    S, _, _, var = score_stats(q, k, N, 64, bk, 0.8)
    S0, _, _ = score(q, k, N, 64, bk, 0.8)
    assert np.all(var < 1e-25)  # the mean of equal values may round in its last bit
    assert np.allclose(S, S0, rtol=1e-7, atol=1e-12)


def test_variance_matches_scalar_brute_force():
    rng = np.random.default_rng(1)
    N, Np, d, bk = 70, 96, 3, 32
    k = rng.standard_normal((1, 1, Np, d))
    var = block_variances(k, N, bk)
    for j in range(Np // bk):
        n = max(0, min(bk, N - j * bk))
        for c in range(d):
            xs = [k[0, 0, j * bk + r, c] for r in range(n)]
            if n == 0:
                assert var[0, 0, j, c] == 0
                continue
            m = sum(xs) / n
            assert math.isclose(var[0, 0, j, c], sum((x - m) ** 2 for x in xs) / n, rel_tol=1e-12)


def test_logit_is_the_gaussian_mean_of_exp():
    # one query block (all rows the same vector qv) against two units of many Gaussian keys:
    # log of the empirical mean of exp(s <qv, k>) over a unit approaches the scorer's logit
    rng = np.random.default_rng(2)
    d, n, s = 6, 1 << 16, 0.9
    qv = rng.standard_normal(d) * 0.8
    mu = rng.standard_normal((2, d)) * 0.5
    sd = np.array([0.3, 0.6])[:, None] * np.ones(d)
    keys = mu[:, None, :] + sd[:, None, :] * rng.standard_normal((2, n, d))
    q = np.broadcast_to(qv, (1, 1, 2 * n, d)).copy()
    k = keys.reshape(1, 1, 2 * n, d)
    S, qb, kb, kv = score_stats(q, k, 2 * n, 2 * n, n, s)
    logit = s * kb[0, 0] @ qb[0, 0, 0] + 0.5 * s * s * kv[0, 0] @ (qb[0, 0, 0] ** 2)
    emp = np.log(np.exp(s * keys @ qv).mean(axis=1))
    assert np.allclose(logit, emp, atol=0.02), (logit, emp)
    # the second-moment term is large here: leaving it out misses by far more than the tolerance
    assert np.all(np.abs(s * kb[0, 0] @ qb[0, 0, 0] - emp)[1:] > 0.1)
    # and the score ratio of the two units follows the logit difference
    assert math.isclose(S[0, 0, 0, 1] / S[0, 0, 0, 0], math.exp(logit[1] - logit[0]), rel_tol=1e-5)


def test_spread_raises_a_units_score():
    rng = np.random.default_rng(3)
    d, bk = 4, 16
    base = rng.standard_normal(d)
    k = np.zeros((1, 1, 2 * bk, d))
    k[0, 0, :bk] = base                                   # unit 0: no spread
    k[0, 0, bk:] = base + 0.5 * rng.standard_normal((bk, d))
    k[0, 0, bk:] += base - k[0, 0, bk:].mean(axis=0)      # unit 1: same mean, spread
    q = np.tile(rng.standard_normal(d), (1, 1, 2 * bk, 1))
    S, _, kb, kv = score_stats(q, k, 2 * bk, 2 * bk, bk, 1.0)
    assert np.allclose(kb[0, 0, 0], kb[0, 0, 1])
    assert S[0, 0, 0, 1] > S[0, 0, 0, 0]


def test_rows_sum_to_one_and_invalid_units_score_zero():
    rng = np.random.default_rng(4)
    N, Np = 300, 512
    q = rng.standard_normal((2, 2, Np, 16)) * 0.5
    k = rng.standard_normal((2, 2, Np, 16)) * 0.5
    q[..., N:, :] = 0
    k[..., N:, :] = 0
    S, _, _, _ = score_stats(q, k, N, 64, 32, 1.2)
    n_j = valid_counts(N, Np, 32)
    assert np.allclose(S.astype(np.float64).sum(-1), 1.0, atol=1e-6)
    assert np.all(S[..., n_j == 0] == 0)
