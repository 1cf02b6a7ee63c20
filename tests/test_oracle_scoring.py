"""Pins for the oracle's block scoring (CPU only): closed forms and scalar brute force."""

import math

import numpy as np

from oracle import block_means, score, valid_counts


def _brute_score(q, k, N, bq, bk, sm):
    """Scalar Python loops over one head: means, logits, n_j-weighted softmax."""
    Np, d = len(q), len(q[0])
    def mean(x, lo, n):
        return [sum(x[r][c] for r in range(lo, lo + n)) / n for c in range(d)] if n else [0.0] * d
    qb = [mean(q, i * bq, max(0, min(bq, N - i * bq))) for i in range(Np // bq)]
    nj = [max(0, min(bk, N - j * bk)) for j in range(Np // bk)]
    kb = [mean(k, j * bk, nj[j]) for j in range(Np // bk)]
    S = []
    for i in range(len(qb)):
        lg = [sm * sum(a * b for a, b in zip(qb[i], kb[j])) for j in range(len(kb))]
        L = max(lg[j] for j in range(len(kb)) if nj[j] > 0)
        mass = [nj[j] * math.exp(lg[j] - L) if nj[j] > 0 else 0.0 for j in range(len(kb))]
        z = sum(mass)
        S.append([x / z for x in mass])
    return S


def test_score_matches_scalar_brute_force():
    rng = np.random.default_rng(0)
    N, Np, d, bq, bk, sm = 50, 64, 4, 16, 8, 0.7
    q = np.zeros((1, 1, Np, d)); k = np.zeros((1, 1, Np, d))
    q[0, 0, :N] = rng.standard_normal((N, d))
    k[0, 0, :N] = rng.standard_normal((N, d))
    S, _, _ = score(q, k, N, bq, bk, sm)
    ref = np.array(_brute_score(q[0, 0].tolist(), k[0, 0].tolist(), N, bq, bk, sm), dtype=np.float32)
    assert np.array_equal(S[0, 0], ref)


def test_identical_tokens_give_that_token_as_mean():
    d, Np, N = 8, 96, 80
    x = np.full((1, 1, Np, d), 99.0)  # padded rows hold junk that must be ignored
    tok = np.arange(d, dtype=np.float64) - 3.5
    x[0, 0, :N] = tok
    m = block_means(x, N, 32)
    assert np.array_equal(m[0, 0, 0], tok) and np.array_equal(m[0, 0, 2], tok)  # block 2 has 16 valid rows


def test_equal_key_means_give_count_proportional_scores():
    # every key unit has the same mean -> S_ij = n_j / N exactly (up to fp32 rounding)
    rng = np.random.default_rng(1)
    N, Np, d = 300, 320, 16
    q = np.zeros((1, 2, Np, d)); k = np.zeros((1, 2, Np, d))
    q[..., :N, :] = rng.standard_normal((1, 2, N, d))
    k[..., :N, :] = rng.standard_normal(d)
    S, _, _ = score(q, k, N, 64, 32, 1.3)
    nj = valid_counts(N, Np, 32)
    ref = (nj / N).astype(np.float32)
    assert np.allclose(S, np.broadcast_to(ref, S.shape), rtol=1e-6, atol=0)
    assert np.isclose(S[0, 0, 0, -1], 12 / 300, rtol=1e-6)  # tail unit 9 holds 12 valid keys


def test_invalid_units_score_zero_and_rows_sum_to_one():
    rng = np.random.default_rng(2)
    N, Np, d = 130, 256, 8
    q = np.zeros((1, 1, Np, d)); k = np.zeros((1, 1, Np, d))
    q[..., :N, :] = rng.standard_normal((N, d)); k[..., :N, :] = rng.standard_normal((N, d))
    S, _, _ = score(q, k, N, 64, 32, 2.0)
    assert np.all(S[0, 0, :, 5:] == 0)  # units 5..7 start at >= 160 > N
    assert np.allclose(S.astype(np.float64).sum(-1), 1.0, atol=1e-6)


def test_scores_are_rows_of_query_blocks_not_columns():
    # query block i is aligned with key unit sigma(i): argmax_j S_ij == sigma(i)
    d, nb, blk = 32, 6, 16
    Np = nb * blk
    sigma = [3, 0, 5, 1, 4, 2]
    basis = np.eye(d)[:nb] * 6.0
    q = np.zeros((1, 1, Np, d)); k = np.zeros((1, 1, Np, d))
    for i in range(nb):
        q[0, 0, i * blk:(i + 1) * blk] = basis[i]
        k[0, 0, sigma[i] * blk:(sigma[i] + 1) * blk] = basis[i]
    S, _, _ = score(q, k, Np, blk, blk, 1.0)
    assert S[0, 0].argmax(axis=1).tolist() == sigma


def test_two_unit_ratio_closed_form():
    d, Np = 2, 8
    q = np.zeros((1, 1, Np, d)); k = np.zeros((1, 1, Np, d))
    q[0, 0, :4] = [1.0, 2.0]
    k[0, 0, :4] = [0.5, 0.0]
    k[0, 0, 4:7] = [0.0, 0.25]  # unit 1 has 3 valid keys (N = 7)
    S, _, _ = score(q, k, 7, 4, 4, 1.5)
    ratio = (4 * math.exp(1.5 * 0.5)) / (3 * math.exp(1.5 * 0.5))
    assert math.isclose(float(S[0, 0, 0, 0]) / float(S[0, 0, 0, 1]), ratio, rel_tol=1e-6)
