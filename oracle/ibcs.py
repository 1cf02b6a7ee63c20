"""Intra-block clustering scorer (IBCS), fp64 CPU oracle.

Test infrastructure: part of the CPU oracle (see ``oracle/__init__.py``).

What it computes (AB-Attention, Abstract: the Intra-Block Clustering Selector
clusters the queries of each query block only, without permuting tokens;
podcast transcript, the passage on how blocks are chosen: similar queries of a
query block are grouped, every group gets a representative and a weight that
reflects how many queries it holds, and the representatives score the key
blocks; the passage after it: one block mean can hide preferences that only
part of the block holds).

The pages give no algorithm, initialisation, group count or mixing rule. The
readings taken here:

* clustering is Lloyd's k-means with squared Euclidean distance on the query
  vectors of the block's n valid rows, G groups and T iterations;
* the initial centroid of group g is row floor(g n / G) of the block (in the
  block's own row order, after the optional permutation);
* one iteration assigns every row to its nearest centroid (ties: the lower
  group) and then replaces every centroid by the mean of its rows; a group
  with no rows keeps its centroid;
* the representative of group g is its final centroid c_g and its weight is
  n_g / n, n_g being its row count after the last assignment;
* S[i, j] = sum_g (n_g / n) n_j exp(l_gj - L_g) / sum_{j' in V} n_j' exp(l_gj' - L_g)
  with l_gj = sm_scale <c_g, k_bar_j> and L_g = max_{j in V} l_gj: the mixture,
  by group size, of every group's estimated attention mass. Rows still sum to
  1 and S = 0 for units with no valid key;
* a query block with no valid row scores like the plain scorer's empty block:
  one group with the zero centroid and weight 1 (its sizes are all 0).

With G = 1 the one centroid is the block mean, so this is the plain scorer.
"""

from __future__ import annotations

import numpy as np

from .scoring import apply_perm, block_means, valid_counts


def cluster_block(rows: np.ndarray, groups: int, iters: int):
    """k-means of one block's valid rows ([n, d], n >= 1) into ``groups`` groups.

    Returns (centroids [G, d] fp64, sizes int64 [G], margin). ``margin`` is the
    smallest relative gap (d2 - d1) / (d2 + d1) seen in any assignment between
    a row's nearest centroid (d1) and the nearest centroid that differs from it
    (d2); inf when every assignment was between identical centroids. A small
    margin marks a near tie that a lower-precision computation may resolve
    the other way.
    """
    rows = np.asarray(rows, dtype=np.float64)
    n = rows.shape[0]
    c = rows[[(g * n) // groups for g in range(groups)]].copy()
    margin = np.inf
    lab = np.zeros(n, dtype=np.int64)
    for _ in range(iters):
        d2 = ((rows[:, None, :] - c[None, :, :]) ** 2).sum(axis=-1)  # [n, G]
        lab = np.argmin(d2, axis=1)  # first minimum: the lower group on ties
        same = np.all(c[:, None, :] == c[None, :, :], axis=-1)     # [G, G] identical centroids
        best = d2[np.arange(n), lab]
        other = np.where(same[lab], np.inf, d2)
        second = other.min(axis=1)
        fin = np.isfinite(second)
        if fin.any():
            margin = min(margin, float(((second[fin] - best[fin]) / (second[fin] + best[fin])).min()))
        for g in range(groups):
            members = rows[lab == g]
            if members.shape[0]:
                c[g] = members.sum(axis=0) / members.shape[0]
    sizes = np.bincount(lab, minlength=groups).astype(np.int64)
    return c, sizes, margin


def group_mixture(cent: np.ndarray, weights: np.ndarray, k_bar: np.ndarray, n_j: np.ndarray,
                  sm_scale: float) -> np.ndarray:
    """One score row: sum_g weights[g] * (n_j-weighted softmax of sm_scale <c_g, k_bar_j> over V)."""
    valid = n_j > 0
    out = np.zeros(k_bar.shape[0], dtype=np.float64)
    for g in range(cent.shape[0]):
        if weights[g] == 0:
            continue
        lv = np.where(valid, sm_scale * (k_bar @ cent[g]), -np.inf)
        mass = np.where(valid, n_j * np.exp(lv - lv.max()), 0.0)
        out += weights[g] * mass / mass.sum()
    return out


def score_ibcs(q, k, N: int, block_q: int, block_k: int, sm_scale: float, groups: int, iters: int,
               perm=None, blocks=None):
    """IBCS score matrix.

    With ``blocks`` None: returns (S float32 [B, H, nQB, nKU], centroids fp64
    [B, H, nQB, G, d], sizes int64 [B, H, nQB, G], margins [B, H, nQB], k_bar).
    With ``blocks`` a list of (b, h, i): the same quantities for those query
    blocks only, as lists in that order (S rows, centroids, sizes, margins).
    """
    qp = apply_perm(np.asarray(q, dtype=np.float64), perm)
    k_bar = block_means(k, N, block_k, perm)
    B, H, N_pad, d = qp.shape
    nQB = N_pad // block_q
    counts = valid_counts(N, N_pad, block_q)
    n_j = valid_counts(N, N_pad, block_k).astype(np.float64)

    def one(b, h, i):
        n = int(counts[i])
        if n == 0:
            cent = np.zeros((groups, d))
            sizes = np.zeros(groups, dtype=np.int64)
            row = group_mixture(cent[:1], np.ones(1), k_bar[b, h], n_j, sm_scale)
            return row, cent, sizes, np.inf
        rows = qp[b, h, i * block_q: i * block_q + n]
        cent, sizes, margin = cluster_block(rows, groups, iters)
        row = group_mixture(cent, sizes / n, k_bar[b, h], n_j, sm_scale)
        return row, cent, sizes, margin

    if blocks is not None:
        res = [one(b, h, i) for (b, h, i) in blocks]
        return ([r[0].astype(np.float32) for r in res], [r[1] for r in res], [r[2] for r in res],
                [r[3] for r in res])
    S = np.zeros((B, H, nQB, k_bar.shape[2]), dtype=np.float64)
    cents = np.zeros((B, H, nQB, groups, d))
    sizes = np.zeros((B, H, nQB, groups), dtype=np.int64)
    margins = np.zeros((B, H, nQB))
    for b in range(B):
        for h in range(H):
            for i in range(nQB):
                S[b, h, i], cents[b, h, i], sizes[b, h, i], margins[b, h, i] = one(b, h, i)
    return S.astype(np.float32), cents, sizes, margins, k_bar
