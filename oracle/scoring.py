"""Block scoring, fp64 CPU oracle.

Test infrastructure: part of the CPU oracle (see ``oracle/__init__.py``).

What it computes (AB-Attention, Abstract: key blocks are rated from cheap
per-block summaries; InstaGen, Abstract: the sampling chance of a block follows
its estimated share of attention):

* q_bar[i] = mean of the valid rows of query block i (rows r < N of the
  permuted sequence); a block with no valid row gets the zero vector;
* k_bar[j] = mean of the n_j valid keys of key unit j; units with n_j = 0 are
  not in the population V;
* l[i, j] = sm_scale * <q_bar[i], k_bar[j]>;
* S[i, j] = n_j exp(l[i, j] - L_i) / sum_{j' in V} n_j' exp(l[i, j'] - L_i) with
  L_i = max_{j in V} l[i, j]; S[i, j] = 0 for j not in V. The factor n_j makes
  a half-filled tail unit count only its real keys. S is the estimated share
  of query block i's attention mass that falls in unit j, rounded once to fp32.
"""

from __future__ import annotations

import numpy as np


def apply_perm(x: np.ndarray, perm) -> np.ndarray:
    """Gather rows of [..., N_pad, d] by ``perm`` (X'[r] = X[perm[r]]); identity if None."""
    if perm is None:
        return x
    return x[..., np.asarray(perm, dtype=np.int64), :]


def unpermute(x: np.ndarray, perm) -> np.ndarray:
    """Scatter rows back: out[perm[r]] = x[r]."""
    if perm is None:
        return x
    out = np.empty_like(x)
    out[..., np.asarray(perm, dtype=np.int64), :] = x
    return out


def valid_counts(N: int, N_pad: int, block: int) -> np.ndarray:
    """n_b = number of rows r < N inside each block of ``block`` rows."""
    starts = np.arange(0, N_pad, block)
    return np.clip(N - starts, 0, block).astype(np.int64)


def block_means(x: np.ndarray, N: int, block: int, perm=None) -> np.ndarray:
    """Mean of the valid rows of every block: [B, H, N_pad, d] -> [B, H, N_pad/block, d] in fp64."""
    xp = apply_perm(np.asarray(x, dtype=np.float64), perm)
    B, H, N_pad, d = xp.shape
    counts = valid_counts(N, N_pad, block)
    nb = N_pad // block
    out = np.zeros((B, H, nb, d), dtype=np.float64)
    for blk in range(nb):
        n = counts[blk]
        if n == 0:
            continue
        rows = xp[:, :, blk * block: blk * block + n, :]
        out[:, :, blk, :] = rows.sum(axis=2) / n
    return out


def score(q, k, N: int, block_q: int, block_k: int, sm_scale: float, perm=None):
    """Score matrix S (float32 [B, H, nQB, nKU]) plus the fp64 block means.

    Returns (S, q_bar, k_bar).
    """
    q_bar = block_means(q, N, block_q, perm)
    k_bar = block_means(k, N, block_k, perm)
    N_pad = q.shape[-2]
    n_j = valid_counts(N, N_pad, block_k).astype(np.float64)
    valid = n_j > 0
    logits = sm_scale * np.einsum("bhid,bhjd->bhij", q_bar, k_bar)
    lv = np.where(valid, logits, -np.inf)
    L = lv.max(axis=-1, keepdims=True)
    mass = np.where(valid, n_j * np.exp(lv - L), 0.0)
    S = mass / mass.sum(axis=-1, keepdims=True)
    return S.astype(np.float32), q_bar, k_bar
