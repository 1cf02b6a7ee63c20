"""Weighted block-sparse attention and dense attention, fp64 CPU oracle.

Test infrastructure: part of the CPU oracle (see ``oracle/__init__.py``).

What it computes. For a query row r of block i with the list of (unit j,
weight w_j) chosen for that block, logits a_rt = sm_scale <Q'_r, K'_t> over the
valid keys t of each listed unit, and

    N_hat_r = sum_j w_j sum_t exp(a_rt - M_r) V'_t
    D_hat_r = sum_j w_j sum_t exp(a_rt - M_r)
    O'_r    = N_hat_r / D_hat_r,    lse_r = M_r + ln D_hat_r.

The weight enters numerator and denominator alike, so one sparse pass
estimates the dense sums instead of dropping the unlisted blocks
(AB-Attention, Abstract; InstaGen, Abstract). Multiplying a block's terms by
w_j is the same as adding ln w_j to its logits before the softmax
(AB-Attention, transcript: weights as pre-softmax shifts). The numerator and
denominator estimates are each unbiased over the sampler's randomness; their
ratio is not (AB-Attention, transcript: unbiasedness of the two sums).

Readings: Q', K', V' are the rows gathered by the optional permutation and
validity is positional (r < N); padded query rows output 0 with lse = -inf;
the list is used as given, a repeated entry counting twice. M_r is any
per-row constant: ``attend`` uses the max over the listed logits, and
``weighted_sums`` takes it from the caller (the dense row max, which does not
depend on the seed) so that the sums can be averaged over seeds.
Dense attention is the same computation with every valid unit listed at
weight 1, i.e. a masked softmax(sm_scale Q K^T) V.
"""

from __future__ import annotations

import numpy as np

from .scoring import apply_perm, unpermute


def _unit_keys(j: int, block_k: int, N: int) -> np.ndarray:
    lo = j * block_k
    hi = min(lo + block_k, N)
    return np.arange(lo, max(lo, hi))


def _block_rows(i: int, block_q: int, N: int) -> np.ndarray:
    lo = i * block_q
    hi = min(lo + block_q, N)
    return np.arange(lo, max(lo, hi))


def attend_block(qp, kp, vp, i, idx_row, w_row, N, block_q, block_k, sm_scale):
    """One query block of one head, inputs already permuted ([N_pad, d] each).

    Returns (O' rows [block_q, d], lse [block_q]) in fp64.
    """
    d = qp.shape[-1]
    o = np.zeros((block_q, d), dtype=np.float64)
    lse = np.full(block_q, -np.inf, dtype=np.float64)
    rows = _block_rows(i, block_q, N)
    if rows.size == 0:
        return o, lse
    qr = qp[rows]
    parts = []
    for j, wj in zip(np.asarray(idx_row).tolist(), np.asarray(w_row, dtype=np.float64).tolist()):
        keys = _unit_keys(int(j), block_k, N)
        if keys.size == 0:
            continue
        parts.append((sm_scale * (qr @ kp[keys].T), wj, keys))
    M = np.max(np.concatenate([a for a, _, _ in parts], axis=1), axis=1)
    num = np.zeros((rows.size, d))
    den = np.zeros(rows.size)
    for a, wj, keys in parts:
        e = np.exp(a - M[:, None])
        num += wj * (e @ vp[keys])
        den += wj * e.sum(axis=1)
    o[: rows.size] = num / den[:, None]
    lse[: rows.size] = M + np.log(den)
    return o, lse


def attend(q, k, v, N, block_q, block_k, sm_scale, idx, w, perm=None, blocks=None):
    """Weighted sparse attention.

    q, k, v: [B, H, N_pad, d] (any float dtype; widened to fp64); idx, w: [B, H, nQB, L].
    With ``blocks`` None returns (O [B, H, N_pad, d], lse [B, H, N_pad]) un-permuted.
    With ``blocks`` a list of (b, h, i), returns a list of (O' rows, lse rows) for those
    blocks in the permuted order (compare with the kernel's output gathered by perm).
    """
    qp = apply_perm(np.asarray(q, dtype=np.float64), perm)
    kp = apply_perm(np.asarray(k, dtype=np.float64), perm)
    vp = apply_perm(np.asarray(v, dtype=np.float64), perm)
    if blocks is not None:
        return [attend_block(qp[b, h], kp[b, h], vp[b, h], i, idx[b, h, i], w[b, h, i],
                             N, block_q, block_k, sm_scale) for b, h, i in blocks]
    B, H, N_pad, d = qp.shape
    nqb = N_pad // block_q
    O = np.zeros((B, H, N_pad, d))
    L = np.full((B, H, N_pad), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                o, l = attend_block(qp[b, h], kp[b, h], vp[b, h], i, idx[b, h, i], w[b, h, i],
                                    N, block_q, block_k, sm_scale)
                O[b, h, i * block_q:(i + 1) * block_q] = o
                L[b, h, i * block_q:(i + 1) * block_q] = l
    return unpermute(O, perm), unpermute(L[..., None], perm)[..., 0]


def dense_block(qp, kp, vp, rows, N, sm_scale):
    """Masked softmax attention for the given (permuted-space) rows of one head."""
    d = qp.shape[-1]
    rows = np.asarray(rows)
    o = np.zeros((rows.size, d))
    lse = np.full(rows.size, -np.inf)
    ok = rows < N
    if not ok.any():
        return o, lse
    a = sm_scale * (qp[rows[ok]] @ kp[:N].T)
    M = a.max(axis=1)
    e = np.exp(a - M[:, None])
    den = e.sum(axis=1)
    o[ok] = (e @ vp[:N]) / den[:, None]
    lse[ok] = M + np.log(den)
    return o, lse


def attend_dense(q, k, v, N, sm_scale, perm=None, block_rows=1024, blocks=None, block_q=128):
    """Dense masked attention.

    With ``blocks`` None: (O, lse) over the full tensors, un-permuted. With ``blocks`` a
    list of (b, h, i): list of (O' rows, lse rows) for query block i (rows of ``block_q``)
    in the permuted order.
    """
    qp = apply_perm(np.asarray(q, dtype=np.float64), perm)
    kp = apply_perm(np.asarray(k, dtype=np.float64), perm)
    vp = apply_perm(np.asarray(v, dtype=np.float64), perm)
    if blocks is not None:
        return [dense_block(qp[b, h], kp[b, h], vp[b, h],
                            np.arange(i * block_q, (i + 1) * block_q), N, sm_scale)
                for b, h, i in blocks]
    B, H, N_pad, d = qp.shape
    O = np.zeros((B, H, N_pad, d))
    L = np.full((B, H, N_pad), -np.inf)
    for b in range(B):
        for h in range(H):
            for s in range(0, N_pad, block_rows):
                rows = np.arange(s, min(s + block_rows, N_pad))
                o, l = dense_block(qp[b, h], kp[b, h], vp[b, h], rows, N, sm_scale)
                O[b, h, rows] = o
                L[b, h, rows] = l
    return unpermute(O, perm), unpermute(L[..., None], perm)[..., 0]


def dense_row_max(qp_h, kp_h, rows, N, sm_scale) -> np.ndarray:
    """M_r = max over all valid keys of a_rt, for the given rows of one (permuted) head."""
    return (sm_scale * (qp_h[rows] @ kp_h[:N].T)).max(axis=1)


def unit_sums(qp_h, kp_h, vp_h, rows, N, block_k, sm_scale, M) -> tuple:
    """Per-unit exact contributions for the given rows of one head.

    Returns (num [n_units, len(rows), d], den [n_units, len(rows)]) with
    num_j = sum_{t in j} exp(a_rt - M_r) V_t and den_j = sum_{t in j} exp(a_rt - M_r).
    """
    n_units = -(-N // block_k)
    d = vp_h.shape[-1]
    num = np.zeros((n_units, len(rows), d))
    den = np.zeros((n_units, len(rows)))
    for j in range(n_units):
        keys = _unit_keys(j, block_k, N)
        e = np.exp(sm_scale * (qp_h[rows] @ kp_h[keys].T) - M[:, None])
        num[j] = e @ vp_h[keys]
        den[j] = e.sum(axis=1)
    return num, den


def weighted_sums(qp_h, kp_h, vp_h, rows, N, block_k, sm_scale, idx_row, w_row, M):
    """N_hat and D_hat for the given rows of one head with a caller-fixed M_r."""
    d = vp_h.shape[-1]
    num = np.zeros((len(rows), d))
    den = np.zeros(len(rows))
    for j, wj in zip(np.asarray(idx_row).tolist(), np.asarray(w_row, dtype=np.float64).tolist()):
        keys = _unit_keys(int(j), block_k, N)
        e = np.exp(sm_scale * (qp_h[rows] @ kp_h[keys].T) - M[:, None])
        num += wj * (e @ vp_h[keys])
        den += wj * e.sum(axis=1)
    return num, den
