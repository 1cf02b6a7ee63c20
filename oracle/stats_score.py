"""Statistics-aware scorer, fp64 CPU oracle.

Test infrastructure: part of the CPU oracle (see ``oracle/__init__.py``).

What it computes (Veda, Abstract: tile selection posed as reconstructing full
attention, with statistics-aware tile scoring). The page names the idea and no
formula; the reading taken here scores a key unit by the attention mass its
keys would receive if they were Gaussian with the unit's first two moments:

* k_bar[j] and var[j] = mean and population variance (per dimension) of the
  n_j valid keys of unit j;
* the mean of exp(s <q, k>) over such keys is exp(s <q, k_bar> + s^2/2 sum_d
  q_d^2 var_d) (the moment-generating function of a diagonal Gaussian), so
  l[i, j] = s <q_bar_i, k_bar_j> + (s^2 / 2) <q_bar_i^2, var_j> with s =
  sm_scale and q_bar_i the block mean of the queries;
* S[i, j] = n_j exp(l[i, j] - L_i) / sum_{j' in V} n_j' exp(l[i, j'] - L_i),
  S = 0 for units with no valid key, exactly as the plain scorer.

A unit whose keys are all equal has zero variance and scores as in the plain
scorer; spread within a unit raises its estimated mass, since a few aligned
keys can dominate an average of exponentials.
"""

from __future__ import annotations

import numpy as np

from .scoring import apply_perm, block_means, valid_counts


def block_variances(x: np.ndarray, N: int, block: int, perm=None) -> np.ndarray:
    """Population variance (per dimension) of the valid rows of every block, fp64."""
    xp = apply_perm(np.asarray(x, dtype=np.float64), perm)
    B, H, N_pad, d = xp.shape
    counts = valid_counts(N, N_pad, block)
    out = np.zeros((B, H, N_pad // block, d))
    for blk, n in enumerate(counts):
        if n:
            out[:, :, blk, :] = xp[:, :, blk * block: blk * block + n, :].var(axis=2)
    return out


def score_stats(q, k, N: int, block_q: int, block_k: int, sm_scale: float, perm=None):
    """Statistics-aware score matrix: (S float32 [B, H, nQB, nKU], q_bar, k_bar, k_var)."""
    q_bar = block_means(q, N, block_q, perm)
    k_bar = block_means(k, N, block_k, perm)
    k_var = block_variances(k, N, block_k, perm)
    n_j = valid_counts(N, q.shape[-2], block_k).astype(np.float64)
    valid = n_j > 0
    logits = (sm_scale * np.einsum("bhid,bhjd->bhij", q_bar, k_bar)
              + 0.5 * sm_scale ** 2 * np.einsum("bhid,bhjd->bhij", q_bar ** 2, k_var))
    lv = np.where(valid, logits, -np.inf)
    L = lv.max(axis=-1, keepdims=True)
    mass = np.where(valid, n_j * np.exp(lv - L), 0.0)
    S = mass / mass.sum(axis=-1, keepdims=True)
    return S.astype(np.float32), q_bar, k_bar, k_var
