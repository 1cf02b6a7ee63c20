"""Pins for the oracle's block selection (CPU only).

Each test checks the oracle against something other than itself: a library
sort, an independent exact-rational water-filling, brute-force enumeration of
the sampler's uniform offset, the pages' worked example, and special cases
with a closed form.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (exact_set, quantise, water_fill, fixed_point_pi, systematic_sample,
                    select_row, sanitize, inverse_weight, block_offset, F_BITS)

HERE = os.path.dirname(os.path.abspath(__file__))


def _rows(seed, n, count):
    """Score rows with assorted shapes: softmax-like, heavy-tailed, tied, sparse."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(count):
        kind = c % 5
        if kind == 0:
            x = rng.standard_normal(n) * 2
            s = np.exp(x - x.max())
        elif kind == 1:
            s = rng.pareto(1.2, n)
        elif kind == 2:
            s = rng.integers(0, 4, n).astype(np.float64)
        elif kind == 3:
            s = np.where(rng.random(n) < 0.2, rng.random(n), 0.0)
        else:
            s = rng.random(n) ** 8
        s = s / max(s.sum(), 1e-300)
        out.append(s.astype(np.float32))
    return out


def _fraction_waterfill(q, m):
    """Exact water-filling by sorting: the c with sum_j min(1, c q_j) = m (rationals)."""
    n = len(q)
    order = sorted(range(n), key=lambda j: -q[j])
    for t in range(0, m + 1):
        if t == n:
            return None, set(order)
        rest = sum(q[j] for j in order[t:])
        c = Fraction(m - t, rest)
        top_ok = all(c * q[order[s]] >= 1 for s in range(t))
        next_ok = c * q[order[t]] < 1
        if top_ok and next_ok:
            return c, set(order[:t])
    raise AssertionError("no water level found")


def test_exact_set_matches_lexsort():
    for s in _rows(1, 97, 40):
        k = 11
        ref = np.lexsort((np.arange(97), -s.astype(np.float64)))[:k]
        assert exact_set(sanitize(s), 97, k) == sorted(ref.tolist())


def test_exact_set_tie_break_lower_index():
    s = np.array([0.1, 0.3, 0.3, 0.3, 0.0], dtype=np.float32)
    assert exact_set(sanitize(s), 5, 2) == [1, 2]


def test_sanitize_degenerate_scores():
    s = np.array([np.nan, -1.0, 0.0, -0.0, np.inf, 1e-45, 2.0], dtype=np.float32)
    out = sanitize(s)
    assert out[:4].tolist() == [0.0, 0.0, 0.0, 0.0]
    assert out[4] == float(np.finfo(np.float32).max)
    assert out[5] > 0 and out[6] == 2.0


def test_quantise_range_and_scale():
    s = np.array([1.0, 0.5, 0.25, 0.9999999, 1e-30], dtype=np.float64)
    q = quantise(s, 20)
    # max 1.0 = 0.5 * 2^1 -> e = 1; q = floor(s * 2^19)
    assert q == [2**19, 2**18, 2**17, math.floor(0.9999999 * 2**19), 1]
    assert all(1 <= x < 2**20 for x in q)
    assert quantise(np.zeros(4), 20) == [1, 1, 1, 1]


@pytest.mark.parametrize("m", [1, 2, 5, 17, 40])
def test_waterfill_matches_exact_rationals(m):
    for s in _rows(2 + m, 60, 25):
        q = quantise(sanitize(s).astype(np.float64), 20)
        capped, t, q_u = water_fill(q, m)
        c, ref_capped = _fraction_waterfill(q, m)
        assert {j for j, f in enumerate(capped) if f} == ref_capped
        pi = fixed_point_pi(q, capped, t, q_u, m)
        for j, p in enumerate(pi):
            if j in ref_capped:
                assert p == 2**F_BITS
            else:
                exact = Fraction(2**F_BITS) * c * q[j]
                assert abs(Fraction(p) - exact) < 2


@pytest.mark.parametrize("m", [1, 3, 8, 31])
def test_pi_sums_to_m_exactly(m):
    for s in _rows(10 + m, 64, 40):
        q = quantise(sanitize(s).astype(np.float64), 20)
        capped, t, q_u = water_fill(q, m)
        pi = fixed_point_pi(q, capped, t, q_u, m)
        assert sum(pi) == m * 2**F_BITS
        assert all(1 <= p <= 2**F_BITS for p in pi)
        # the integer-rounding shortfall is smaller than the number of uncapped units
        raw = [2**F_BITS if c else math.floor(math.ldexp(float((m - t) * qj) / float(q_u), F_BITS))
               for qj, c in zip(q, capped)]
        delta = m * 2**F_BITS - sum(raw)
        assert 0 <= delta < max(1, len(q) - t) or (delta == 0)


def test_pi_sum_with_exact_set_is_k_plus_m():
    # sum over all valid units of pi (exact set at 1) equals k + m
    for s in _rows(99, 200, 10):
        k, m = 12, 30
        _, _, info = select_row(s, 200, k, m, u=0, details=True)
        assert k * 2**F_BITS + sum(info["pi"]) == (k + m) * 2**F_BITS


@pytest.mark.parametrize("f,fs,n,m", [(8, 4, 16, 3), (12, 6, 40, 7), (16, 10, 48, 12)])
def test_bruteforce_inclusion_equals_pi(f, fs, n, m):
    """Enumerate every offset u in [0, 2^f): each unit is drawn exactly pi_int times."""
    for s in _rows(f, n, 6):
        q = quantise(sanitize(s).astype(np.float64), fs)
        capped, t, q_u = water_fill(q, m)
        pi = fixed_point_pi(q, capped, t, q_u, m, f)
        assert sum(pi) == m << f
        counts = [0] * n
        for u in range(1 << f):
            taken = systematic_sample(pi, u, f)
            pos = [p for p, _ in taken]
            assert len(pos) == m and len(set(pos)) == m
            assert sorted(sl for _, sl in taken) == list(range(m))
            for j in range(n):
                if capped[j]:
                    assert j in pos
            for p in pos:
                counts[p] += 1
        assert counts == pi


def test_breakpoint_enumeration_inclusion_at_32_bits():
    """At F = 32, the draw only changes where u crosses C_j mod 2^32: exact probabilities."""
    F = F_BITS
    for s in _rows(5, 120, 8):
        m = 20
        q = quantise(sanitize(s).astype(np.float64), 20)
        capped, t, q_u = water_fill(q, m)
        pi = fixed_point_pi(q, capped, t, q_u, m, F)
        cum = np.cumsum([0] + pi).tolist()
        cuts = sorted({c % (1 << F) for c in cum} | {0, 1 << F})
        mass = [0] * len(pi)
        for a, b in zip(cuts[:-1], cuts[1:]):
            ta = systematic_sample(pi, a, F)
            tb = systematic_sample(pi, b - 1, F)
            assert ta == tb  # constant over the interval
            for p, _ in ta:
                mass[p] += b - a
        assert mass == pi


def test_worked_example_quarter_probability_weight_four():
    gold = json.load(open(os.path.join(HERE, "golden", "pi_quarter_weight.json")))
    p, wgt = gold["inclusion_probability"], gold["weight"]
    # one sample from four equally scored units: each has pi = 1/4
    for m, n in [(1, 4), (2, 8), (5, 20)]:
        s = np.full(n, 1.0 / n, dtype=np.float32)
        idx, w, info = select_row(s, n, 0, m, u=123456789, details=True)
        assert all(x == int(p * 2**F_BITS) for x in info["pi"])
        assert all(float(x) == wgt for x in w)
        assert np.float32(wgt).tobytes() == inverse_weight(2**30).tobytes()


def test_uniform_scores_give_m_over_r():
    for n, m in [(10, 3), (37, 5), (591, 40)]:
        s = np.full(n, 0.5, dtype=np.float32)
        _, _, info = select_row(s, n, 0, m, u=0, details=True)
        base = (m << F_BITS) // n
        assert all(p in (base, base + 1) for p in info["pi"])


def test_all_capped_gives_every_unit_weight_one():
    s = _rows(3, 30, 1)[0]
    idx, w = select_row(s, 30, 10, 20, u=77)
    assert sorted(idx.tolist()) == list(range(30))
    assert np.all(w == 1.0)


def test_zero_nan_negative_scores_are_uniform():
    s = np.array([0, np.nan, -3, 0, 0, 0, 0, 0], dtype=np.float32)
    idx, w, info = select_row(s, 8, 2, 3, u=5, details=True)
    assert info["K"] == [0, 1]  # all tie at 0: lowest indices
    assert info["q"] == [1] * 6
    assert len(set(idx.tolist())) == 5


def test_dominant_unit_is_capped_and_always_drawn():
    s = np.full(50, 1e-4, dtype=np.float32)
    s[7] = 1.0
    s[3] = 2.0
    for u in [0, 2**31, 2**32 - 1, 12345]:
        idx, w, info = select_row(s, 50, 1, 4, u=u, details=True)
        assert idx[0] == 3  # exact set
        assert 7 in idx[1:].tolist()
        assert w[list(idx).index(7)] == 1.0


def test_select_row_list_shape_and_distinctness():
    for s in _rows(77, 300, 12):
        for seed in range(3):
            u = block_offset(seed, 0, 1, 2)
            idx, w = select_row(s, 300, 8, 18, u)
            assert idx.shape == (26,) and w.shape == (26,)
            assert len(set(idx.tolist())) == 26
            assert np.all(w[:8] == 1.0) and np.all(w >= 1.0)


def test_m_zero_is_top_k():
    s = _rows(8, 40, 1)[0]
    idx, w = select_row(s, 40, 6, 0, u=0)
    ref = np.lexsort((np.arange(40), -s.astype(np.float64)))[:6]
    assert idx.tolist() == sorted(ref.tolist()) and np.all(w == 1.0)


def test_k_exceeding_budget_rejected():
    with pytest.raises(ValueError):
        select_row(np.ones(5, np.float32), 5, 3, 3, u=0)
