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
* the distances that decide the groups are exact integers: every row is
  rounded to fixed point, q_int = rint(q 2^s) with s = 11 - e and e the
  exponent of the block's largest magnitude (max |q| = f 2^e, f in [0.5, 1)),
  so |q_int| <= 2^11 and a squared distance over d <= 128 dimensions is at
  most 2^31 (an exact unsigned 32-bit sum); rounding is to nearest, ties to
  even. The assignment is then a
  decision that any implementation reproduces exactly;
* the initial centroid of group g is q_int of row floor(g n / G) of the block
  (in the block's own row order, after the optional permutation);
* one iteration assigns every row to the nearest centroid (ties: the lower
  group) and then replaces every centroid by the rounded mean of its rows,
  floor((2 sum + n_g) / (2 n_g)) per dimension; a group with no rows keeps its
  centroid;
* the representative of group g is the mean of its member rows' original
  values after the last assignment, its weight n_g / n; an empty group has the
  zero representative and weight 0;
* S[i, j] = sum_g (n_g / n) n_j exp(l_gj - L_g) / sum_{j' in V} n_j' exp(l_gj' - L_g)
  with l_gj = sm_scale <c_g, k_bar_j> and L_g = max_{j in V} l_gj: the mixture,
  by group size, of every group's estimated attention mass. Rows still sum to
  1 and S = 0 for units with no valid key;
* a query block with no valid row scores like the plain scorer's empty block:
  one group with the zero representative and weight 1 (its sizes are all 0).

With G = 1 the one representative is the block mean, so this is the plain
scorer.

The fixed-point width is set by exactness on the GPU's f16 matrix cores
(every integer up to 2^11 is exact in f16, partial sums stay below 2^24).
``lloyd_block`` is the unrounded reading -- plain Lloyd k-means in fp64 on
the raw rows with the same initial rows, iteration count and tie rule -- and
``certified_agreement`` states when the two must give the same groups: the
rounding of rows (half a grid step e = 2^-(s+1) per coordinate) and of
centroids (at most e more per coordinate against the mean of the rounded rows)
moves a squared distance D over d dimensions by at most
    6 e sqrt(d D) + 9 e^2 d   (centroids after an update),
    4 e sqrt(d D) + 4 e^2 d   (initial centroids, themselves rounded rows),
so an assignment whose plain-Lloyd margin over every other group exceeds the
sum of the two groups' bounds is taken identically; when every assignment of
every iteration clears that margin, both readings hold the same members
throughout and return the same sizes and representatives.
"""

from __future__ import annotations

import math

import numpy as np

from .scoring import apply_perm, block_means, valid_counts


FIXED_BITS = 11  # |q_int| <= 2^11: d <= 128 squared differences sum to at most 2^31


def fixed_point(rows: np.ndarray):
    """Block rows -> (q_int int64, s): q_int = rint(rows 2^s), s = 11 - e(max |rows|)."""
    mx = float(np.abs(rows).max()) if rows.size else 0.0
    s = FIXED_BITS - math.frexp(mx)[1] if mx > 0 else 0
    return np.rint(np.ldexp(rows, s)).astype(np.int64), s


def cluster_block(rows: np.ndarray, groups: int, iters: int, history: bool = False):
    """k-means of one block's valid rows ([n, d], n >= 1) into ``groups`` groups.

    Returns (representatives [G, d] fp64, sizes int64 [G]); with ``history``
    also the fixed-point centroids after every iteration and the block's q_int.
    """
    rows = np.asarray(rows, dtype=np.float64)
    n = rows.shape[0]
    qi, _ = fixed_point(rows)
    c = qi[[(g * n) // groups for g in range(groups)]].copy()
    lab = np.zeros(n, dtype=np.int64)
    hist = []
    for _ in range(iters):
        d2 = ((qi[:, None, :] - c[None, :, :]) ** 2).sum(axis=-1)  # [n, G], exact integers
        lab = np.argmin(d2, axis=1)  # first minimum: the lower group on ties
        for g in range(groups):
            members = qi[lab == g]
            ng = members.shape[0]
            if ng:
                c[g] = (2 * members.sum(axis=0) + ng) // (2 * ng)  # floor division: round half up
        hist.append(c.copy())
    sizes = np.bincount(lab, minlength=groups).astype(np.int64)
    reps = np.zeros((groups, rows.shape[1]))
    for g in range(groups):
        if sizes[g]:
            reps[g] = rows[lab == g].sum(axis=0) / sizes[g]
    if history:
        return reps, sizes, hist, qi
    return reps, sizes


def lloyd_block(rows: np.ndarray, groups: int, iters: int, history: bool = False):
    """Plain Lloyd k-means of one block's rows in fp64, no rounding.

    Initial centroid g is row floor(g n / G); each iteration assigns every row
    to its nearest centroid in squared Euclidean distance (ties: the lower
    group) and moves every non-empty group's centroid to the mean of its rows.
    Returns (representatives [G, d], sizes [G]) like ``cluster_block``; with
    ``history`` also, per iteration, the [n, G] squared distances that decided
    the assignment and the centroids they were measured against.
    """
    rows = np.asarray(rows, dtype=np.float64)
    n = rows.shape[0]
    c = rows[[(g * n) // groups for g in range(groups)]].copy()
    lab = np.zeros(n, dtype=np.int64)
    hist = []
    for _ in range(iters):
        d2 = ((rows[:, None, :] - c[None, :, :]) ** 2).sum(axis=-1)
        hist.append((d2, c.copy()))
        lab = np.argmin(d2, axis=1)
        for g in range(groups):
            if (lab == g).any():
                c[g] = rows[lab == g].mean(axis=0)
    sizes = np.bincount(lab, minlength=groups).astype(np.int64)
    reps = np.zeros((groups, rows.shape[1]))
    for g in range(groups):
        if sizes[g]:
            reps[g] = rows[lab == g].sum(axis=0) / sizes[g]
    if history:
        return reps, sizes, hist
    return reps, sizes


def certified_agreement(rows: np.ndarray, groups: int, iters: int) -> bool:
    """True when every plain-Lloyd assignment clears the rounding bound of the
    fixed-point reading in every iteration (see the module notes), so that
    ``cluster_block`` and ``lloyd_block`` must agree on this block."""
    rows = np.asarray(rows, dtype=np.float64)
    _, s = fixed_point(rows)
    e = math.ldexp(0.5, -s)
    d = rows.shape[1]
    _, _, hist = lloyd_block(rows, groups, iters, history=True)
    for it, (d2, _) in enumerate(hist):
        a, b = (4.0, 4.0) if it == 0 else (6.0, 9.0)
        bound = a * e * np.sqrt(d * d2) + b * e * e * d
        bound *= 1 + 1e-9  # fp64 evaluation of the distances themselves
        best = np.argmin(d2, axis=1)
        r = np.arange(d2.shape[0])
        gap = d2 - d2[r, best][:, None]
        need = bound + bound[r, best][:, None]
        other = np.ones_like(d2, dtype=bool)
        other[r, best] = False
        if np.any(other & (gap <= need)):
            return False
    return True


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

    With ``blocks`` None: returns (S float32 [B, H, nQB, nKU], representatives
    fp64 [B, H, nQB, G, d], sizes int64 [B, H, nQB, G], k_bar). With ``blocks``
    a list of (b, h, i): the same quantities for those query blocks only, as
    lists in that order (S rows, representatives, sizes).
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
            reps = np.zeros((groups, d))
            sizes = np.zeros(groups, dtype=np.int64)
            row = group_mixture(reps[:1], np.ones(1), k_bar[b, h], n_j, sm_scale)
            return row, reps, sizes
        reps, sizes = cluster_block(qp[b, h, i * block_q: i * block_q + n], groups, iters)
        row = group_mixture(reps, sizes / n, k_bar[b, h], n_j, sm_scale)
        return row, reps, sizes

    if blocks is not None:
        res = [one(b, h, i) for (b, h, i) in blocks]
        return [r[0].astype(np.float32) for r in res], [r[1] for r in res], [r[2] for r in res]
    S = np.zeros((B, H, nQB, k_bar.shape[2]), dtype=np.float64)
    reps = np.zeros((B, H, nQB, groups, d))
    sizes = np.zeros((B, H, nQB, groups), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for i in range(nQB):
                S[b, h, i], reps[b, h, i], sizes[b, h, i] = one(b, h, i)
    return S.astype(np.float32), reps, sizes, k_bar
