"""The estimator study on the GPU: at the dense limit (k + m = every valid unit)
every estimator must reproduce dense attention; below it every estimator gives
a finite, positive error and the score mass of the best units lies in (0, 1];
and the study's numbers (relative L2 error against dense attention, D_hat / D)
are recomputed with the oracle on the very lists the study fed bsa_attend
(InstaGen, Abstract: sampling against top-k at high entropy; AB-Attention,
transcript: the ablation without the inverse-probability weights)."""

import math

import numpy as np
import pytest
import torch

import oracle

from block_sparse_attention_27_amd.inputs import Workload, generate
from block_sparse_attention_27_amd.study import run_temperature
from gpu_util import host_f64, print_case

pytestmark = pytest.mark.gpu


def _wl(k, m, tau=1.0):
    return Workload("study", B=1, H=2, grid=(3, 16, 24), d=128, dtype="bf16", block_q=128, block_k=128,
                    k_exact=k, m_sample=m, clusters=6, temperature=tau)


def test_study_dense_limit():
    print_case("estimator study, k + m = all valid units")
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w = _wl(2, 7)
    assert w.list_len == w.n_valid_units
    r = run_temperature(w, [0, 1], log=lambda m: None)
    for name in ("truncation", "unweighted", "weighted", "sample_only", "truncation_ibcs", "weighted_ibcs",
                 "truncation_stats", "weighted_stats"):
        assert r[name] < 1e-4, (name, r[name])
    assert abs(r["top_mass"] - 1.0) < 1e-5


@pytest.mark.parametrize("tau", [0.5, 2.0])
def test_study_sparse_finite(tau):
    print_case(f"estimator study, k=1 m=3 tau={tau}")
    r = run_temperature(_wl(1, 3, tau), [0, 1, 2], log=lambda m: None)
    for name in ("truncation", "unweighted", "weighted", "sample_only", "truncation_ibcs", "weighted_ibcs",
                 "truncation_stats", "weighted_stats"):
        assert math.isfinite(r[name]) and r[name] > 0, (name, r[name])
    assert 0 < r["top_mass"] <= 1 + 1e-6


@pytest.mark.parametrize("values", ["noise", "clustered"])
def test_study_numbers_against_the_oracle(values):
    # 2 heads on a 3 x 16 x 24 grid, k = 2, m = 4, tau = 1: every estimator's error and D_hat / D
    # recomputed in fp64 from the lists the study used must match the study's within 1e-3
    print_case(f"estimator study vs the oracle, values={values}")
    w = _wl(2, 4).replace(value_mode=values)
    seeds = [0, 1, 2]
    r = run_temperature(w, seeds, log=lambda m: None, keep_lists=True)
    g = generate(w)
    q, k, v = (host_f64(g[x]) for x in ("q", "k", "v"))
    O_d, L_d = oracle.attend_dense(q, k, v, w.N, w.sm_scale, g["perm"])
    per = {}
    for name, seed, p, idx, wt in r["lists"]:
        O, L = oracle.attend(q, k, v, w.N, p.block_q, p.block_k, w.sm_scale, idx, wt, g["perm"])
        diff = (O - O_d)[..., : w.N, :]
        err = np.mean([np.linalg.norm(diff[0, h]) / np.linalg.norm(O_d[0, h, : w.N]) for h in range(w.H)])
        dr = float(np.mean(np.exp(L[..., : w.N] - L_d[..., : w.N])))
        per.setdefault(name, []).append((err, dr))
    assert set(per) == {"truncation", "weighted", "unweighted", "sample_only"}
    assert len(per["weighted"]) == len(seeds) and len(per["truncation"]) == 1
    for name, vals in per.items():
        e_ref = float(np.mean([e for e, _ in vals]))
        d_ref = float(np.mean([d for _, d in vals]))
        print_case(f"  {name}: study {r[name]:.5f} / {r[name + '_dr']:.5f}, oracle {e_ref:.5f} / {d_ref:.5f}")
        assert abs(r[name] - e_ref) <= 1e-3, (name, r[name], e_ref)
        assert abs(r[name + "_dr"] - d_ref) <= 1e-3, (name, r[name + "_dr"], d_ref)
    # the pages' claims in this regime: the weighted estimators keep the denominator (D_hat / D near 1)
    # while truncation and the unweighted sample lose part of it
    assert per["truncation"][0][1] < 1.0 and np.mean([d for _, d in per["unweighted"]]) < 1.0


def test_statistics_aware_scorer_reranks_units_with_unequal_spread():
    # Veda, Abstract (statistics-aware tile scoring): with key units of unequal within-unit spread the
    # second-moment term changes which units are exact far more often than with a uniform spread; the
    # true (dense) attention mass its picks hold is reported, not asserted: at these spreads it moves by
    # about 1e-4 either way
    from block_sparse_attention_27_amd.inputs import WORKLOADS
    print_case("statistics-aware vs plain scorer, uniform and clustered key spread")
    base = WORKLOADS["wan14b_480p"].replace(H=4, temperature=0.5, value_mode="clustered")
    r_u = run_temperature(base, [0], log=lambda m: None)
    r_c = run_temperature(base.replace(key_spread="clustered"), [0], log=lambda m: None)
    print_case(f"  exact sets differ: uniform {r_u['exact_diff_stats']:.4f}, clustered {r_c['exact_diff_stats']:.4f}; "
               f"true mass plain/stats {r_c['mass_plain']:.5f}/{r_c['mass_stats']:.5f}")
    assert r_c["exact_diff_stats"] > 2 * r_u["exact_diff_stats"] and r_c["exact_diff_stats"] > 0.05
    assert r_c["mass_plain"] <= r_c["mass_best"] + 1e-6 and r_c["mass_stats"] <= r_c["mass_best"] + 1e-6
