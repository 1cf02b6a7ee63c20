"""Block selection (exact set + fixed-size weighted sample), CPU oracle.

Test infrastructure: part of the CPU oracle (see ``oracle/__init__.py``).

What the pages fix:

* each query block attends exactly to its highest-scoring key blocks; every
  other block can enter only through a random draw whose chance grows with the
  block's estimated attention, and a drawn block is scaled up by one over that
  chance (InstaGen, Abstract; AB-Attention, Abstract);
* scores set per-block inclusion probabilities, the most important blocks can
  be taken with certainty while every other block keeps a nonzero chance, and
  the sampler returns a fixed number of distinct blocks so the budget is
  predictable (AB-Attention, transcript: the inclusion-probability sampler);
* a block kept with probability 1/4 counts four times (AB-Attention,
  transcript: the inverse-probability weighting example).

Readings where the pages leave the step open (each one is listed with its
reason in the design notes):

* inclusion probabilities pi_j = min(1, c * s_j) over the non-exact valid
  units R, with c chosen so that sum_R pi_j = m (so sum over all valid units is
  k + m, the exact set having pi = 1);
* to make every sum order-free and hence reproducible bit for bit on any
  hardware, scores are first quantised to integers q_j in [1, 2^Fs) relative
  to the row maximum (Fs = 20), the water-filling that finds c runs on exact
  integers, and pi is held in fixed point with F = 32 fractional bits and
  sum_R pi_int = m * 2^F exactly;
* the design is systematic probability-proportional-to-size sampling over R
  in ascending unit order with one uniform 32-bit offset per query block from
  Philox4x32-10 keyed by the seed and counted by (query block, head, batch);
* the sample is drawn from R only; units capped at pi = 1 inside R appear in
  the sample part of the list with weight 1.

Everything here is exact integer arithmetic except two IEEE fp64 divisions
(one per uncapped unit for pi, one per sampled unit for its weight) and the
final fp64 -> fp32 rounding of the weight.
"""

from __future__ import annotations

import math

import numpy as np

from .philox import block_offset

F_BITS = 32   # fixed-point fraction bits of pi
FS_BITS = 20  # score quantisation bits
FLT_MAX = float(np.finfo(np.float32).max)


def sanitize(s32) -> np.ndarray:
    """fp32 scores widened to fp64; NaN, zero and negative -> 0, +inf -> FLT_MAX."""
    s = np.asarray(s32, dtype=np.float32).astype(np.float64)
    out = np.where(s > 0, s, 0.0)          # NaN compares false -> 0
    out = np.where(np.isinf(out), FLT_MAX, out)
    return out


def exact_set(s: np.ndarray, n_valid: int, k: int) -> list:
    """First k valid units ordered by (score descending, index ascending); returned ascending."""
    order = sorted(range(n_valid), key=lambda j: (-s[j], j))
    return sorted(order[:k])


def quantise(s_r: np.ndarray, fs: int = FS_BITS) -> list:
    """Integer scores q_j = max(1, floor(s_j * 2^(fs - e))), e the binary exponent of max s.

    If every score is zero all q_j are 1 (uniform). Result lies in [1, 2^fs).
    """
    smax = float(np.max(s_r)) if len(s_r) else 0.0
    if smax <= 0.0:
        return [1] * len(s_r)
    _, e = math.frexp(smax)  # smax = f * 2^e, f in [0.5, 1)
    return [max(1, math.floor(math.ldexp(float(x), fs - e))) for x in s_r]


def water_fill(q: list, m: int):
    """Capped set of pi_j = min(1, c q_j) with sum pi = m, by exact integer rounds.

    Each round takes every uncapped unit with (m - t) q_j >= Q_U (that is,
    c q_j >= 1 for the current c = (m - t)/Q_U) into the capped set; it stops
    when a round adds nothing. Returns (capped flags, t, Q_U).
    """
    capped = [False] * len(q)
    while True:
        t = sum(capped)
        q_u = sum(qj for qj, c in zip(q, capped) if not c)
        new = [j for j, qj in enumerate(q) if not capped[j] and (m - t) * qj >= q_u]
        if not new:
            return capped, t, q_u
        for j in new:
            capped[j] = True


def fixed_point_pi(q: list, capped: list, t: int, q_u: int, m: int, f: int = F_BITS) -> list:
    """pi_int_j in [1, 2^f] with sum exactly m * 2^f.

    Capped units get 2^f. An uncapped unit gets floor(2^f * fl64((m - t) q_j) / fl64(Q_U))
    using one IEEE fp64 division; the shortfall delta = m 2^f - sum (0 <= delta < |U|)
    is paid as +1 to the first delta uncapped units in ascending order.
    """
    one = 1 << f
    pi = []
    for qj, c in zip(q, capped):
        if c:
            pi.append(one)
        else:
            ratio = float((m - t) * qj) / float(q_u)
            pi.append(math.floor(math.ldexp(ratio, f)))
    delta = m * one - sum(pi)
    for j in range(len(pi)):
        if delta == 0:
            break
        if not capped[j]:
            pi[j] += 1
            delta -= 1
    return pi


def systematic_sample(pi: list, u: int, f: int = F_BITS) -> list:
    """Systematic PPS sampling: points u, u + 2^f, u + 2*2^f, ... on the cumulative pi axis.

    Unit j (in list order) is taken iff a point falls in [C_{j-1}, C_j), C being the
    prefix sums of pi_int. Returns a list of (position in R, slot), slot in [0, m).
    """
    def n_points_below(x):
        return ((x - u - 1) >> f) + 1 if x > u else 0

    out = []
    c_prev = 0
    for pos, p in enumerate(pi):
        c = c_prev + p
        a, b = n_points_below(c_prev), n_points_below(c)
        if b > a:
            out.append((pos, a))
        c_prev = c
    return out


def inverse_weight(pi_int: int, f: int = F_BITS) -> np.float32:
    """w = fp32(fl64(2^f) / fl64(pi_int))."""
    return np.float32(float(1 << f) / float(pi_int))


def select_row(s32, n_valid: int, k: int, m: int, u: int, f: int = F_BITS, fs: int = FS_BITS,
               details: bool = False):
    """Selection for one query block.

    s32: the fp32 score row (length >= n_valid); n_valid: valid units are 0..n_valid-1;
    u: the uniform 32-bit offset (use ``block_offset``). Returns (idx int32[k+m],
    w float32[k+m]) and, with ``details``, a dict of the intermediate quantities.
    """
    s = sanitize(np.asarray(s32)[:n_valid])
    K = exact_set(s, n_valid, k)
    in_k = set(K)
    R = [j for j in range(n_valid) if j not in in_k]
    if m > len(R):
        raise ValueError("m exceeds the number of non-exact valid units")
    idx = np.zeros(k + m, dtype=np.int32)
    w = np.zeros(k + m, dtype=np.float32)
    idx[:k] = K
    w[:k] = 1.0
    info = {"K": K, "R": R}
    if m > 0:
        q = quantise(s[R], fs)
        capped, t, q_u = water_fill(q, m)
        pi = fixed_point_pi(q, capped, t, q_u, m, f)
        taken = systematic_sample(pi, u, f)
        for pos, slot in taken:
            idx[k + slot] = R[pos]
            w[k + slot] = inverse_weight(pi[pos], f)
        info.update(q=q, capped=capped, t=t, q_u=q_u, pi=pi, taken=taken)
    return (idx, w, info) if details else (idx, w)


def select(S, N: int, block_k: int, k: int, m: int, seed: int, rows=None):
    """Selection for every (b, h, i) row of S [B, H, nQB, nKU] (or only ``rows``).

    Returns (idx int32[B, H, nQB, k+m], w float32[...]); with ``rows`` given (a list of
    (b, h, i)), returns lists of per-row results in that order.
    """
    S = np.asarray(S, dtype=np.float32)
    n_valid = -(-N // block_k)
    if rows is not None:
        out = []
        for b, h, i in rows:
            u = block_offset(seed, b, h, i)
            out.append(select_row(S[b, h, i], n_valid, k, m, u))
        return out
    B, H, nQB, _ = S.shape
    idx = np.zeros((B, H, nQB, k + m), dtype=np.int32)
    w = np.zeros((B, H, nQB, k + m), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            for i in range(nQB):
                u = block_offset(seed, b, h, i)
                idx[b, h, i], w[b, h, i] = select_row(S[b, h, i], n_valid, k, m, u)
    return idx, w
