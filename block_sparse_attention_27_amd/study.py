"""Estimator quality at matched density, on synthetic clustered-token layers.

InstaGen (Abstract) claims that an exact set plus an inverse-probability
weighted sample estimates dense attention where top-k truncation fails, above
all when attention has high entropy. AB-Attention (podcast transcript, the
ablation passage) reports that dropping the inverse-probability weights, or
selecting deterministically by top-k, costs about the same quality at equal
sparsity. This study measures the same comparison on the library's kernels,
with no trained weights: for each logit temperature of a workload it runs

    truncation   the top-(k+m) units, w = 1            (select with k+m, 0)
    unweighted   exact k + systematic sample of m, w = 1 for every entry
    weighted     exact k + systematic sample of m, w = 1/pi   (the method)
    sample_only  no exact set, a weighted sample of k+m units
    *_ibcs       truncation and weighted again, with the scores of the
                 intra-block clustering scorer (4 groups, 3 iterations)
    *_stats      the same with the statistics-aware scorer

through ``bsa_attend`` (fp32 output) and reports, against
``bsa_attend_dense`` over the valid rows:

    <name>        relative L2 error of the output, per head, then averaged
    <name>_dr     mean over rows of exp(lse - lse_dense) = D_hat / D, the
                  estimated softmax denominator over the dense one; the
                  weighted estimators are unbiased for D (their mean over
                  seeds tends to 1), truncation and the unweighted sample
                  are biased low

For each scorer (plain, ibcs, stats) the study also reports how well its
ranking finds the heavy units: ``mass_<scorer>`` is the mean share of a query
block's true attention (dense softmax over the valid keys, summed per key unit,
averaged over the block's rows) held by the scorer's top-(k+m) units, next to
``mass_best``, the share the true top-(k+m) units hold; ``exact_diff_stats``
is the fraction of query blocks whose top-k set under the statistics-aware
scorer differs from the plain scorer's. The true masses come from fp32
softmax(Q K^T) in PyTorch, a reporting aid outside the library's path.
``--key-spread clustered`` gives key units unequal within-unit spread, the
case the statistics-aware scorer is built for.

The sampled estimators are averaged over several selection seeds (``_std`` is
the standard deviation of the error over seeds). ``top_mass`` is the mean
share of a query block's estimated attention mass (its score row) held by its
k+m best units: near 1 means low entropy, where truncation is already
accurate. ``--values clustered`` draws values that follow the token clusters
(V ~ N(0, 1) noise averages out under high-entropy attention, so the dense
output is near zero and every sparse estimate is far from it in relative
terms).

    python -m block_sparse_attention_27_amd.study --workload wan14b_480p --temps 0.5 1 2 --seeds 8

Needs a GPU; the numbers are printed as one JSON object per temperature.
"""

from __future__ import annotations

import argparse
import json
import statistics
import sys
import time


def _device_inputs(g):
    import numpy as np
    import torch

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    perm = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    return dev(g["q"]), dev(g["k"]), dev(g["v"]), perm


def _d_ratio(lse, lse_ref, n_valid):
    """Mean over valid rows of exp(lse - lse_ref)."""
    import torch

    return float(torch.exp((lse[..., :n_valid] - lse_ref[..., :n_valid]).double()).mean())


def _rel_err_per_head(o, ref, n_valid):
    """Relative L2 error of o against ref over rows < n_valid, one value per (b, h)."""
    import torch

    diff = (o[..., :n_valid, :] - ref[..., :n_valid, :]).double()
    num = torch.linalg.vector_norm(diff, dim=(-2, -1))
    den = torch.linalg.vector_norm(ref[..., :n_valid, :].double(), dim=(-2, -1))
    return (num / den).flatten().tolist()


def unit_mass(w, q, k, perm, rows_per_chunk=2048):
    """True attention mass per (b, h, query block, key unit): the dense softmax of
    sm_scale <q, k> over the valid keys, summed over each unit's keys and averaged
    over the block's valid rows (fp32, in chunks of query rows)."""
    import torch

    B, H, Np, d = q.shape
    if perm is not None:
        q = q.index_select(2, perm.long())
        k = k.index_select(2, perm.long())
    nqb, nku = Np // w.block_q, Np // w.block_k
    M = torch.zeros((B, H, nqb, nku), dtype=torch.float32, device=q.device)
    key_ok = torch.arange(Np, device=q.device) < w.N
    for b in range(B):
        for h in range(H):
            kt = k[b, h].float().t().contiguous()  # [d, Np], contiguous right operand
            for r0 in range(0, Np, rows_per_chunk):
                r1 = min(Np, r0 + rows_per_chunk)
                logits = torch.matmul(q[b, h, r0:r1].float(), kt) * w.sm_scale
                logits.masked_fill_(~key_ok, float("-inf"))
                p = torch.softmax(logits, dim=-1)
                pu = p.view(r1 - r0, nku, w.block_k).sum(-1)  # [rows, units]
                rows = torch.arange(r0, r1, device=q.device)
                pu = pu * (rows < w.N).float()[:, None]
                blk = pu.view(-1, w.block_q, nku).sum(1)
                cnt = (rows < w.N).float().view(-1, w.block_q).sum(1).clamp(min=1)
                M[b, h, r0 // w.block_q: r1 // w.block_q] = blk / cnt[:, None]
    return M


def run_temperature(w, seeds, log=print, keep_lists=False):
    """All estimators for one workload (one temperature). Returns a result dict.

    With ``keep_lists`` the dict also holds, under "lists", every (estimator,
    seed, problem, idx, w) that was fed to ``bsa_attend`` (host copies), so
    that the numbers can be recomputed independently.
    """
    import torch

    import block_sparse_attention_27_amd as bsa
    from block_sparse_attention_27_amd.inputs import generate

    t0 = time.perf_counter()
    g = generate(w)
    q, k, v, perm = _device_inputs(g)
    log(f"  inputs for tau={w.temperature} in {time.perf_counter() - t0:.1f} s")
    L = w.list_len
    base = bsa.problem_for(w, out_fp32=1)
    dense, lse_d = bsa.attend_dense(base, q, k, v, perm, with_lse=True)
    S, _, _ = bsa.score(base, q, k, perm)

    top = torch.topk(S, min(L, S.shape[-1]), dim=-1).values.sum(-1)
    top_mass = float(top.mean())

    kept = []

    def err(p, idx, wt, name=None, seed=None):
        o, lse = bsa.attend(p, q, k, v, idx, wt, perm, with_lse=True)
        if keep_lists and name is not None:
            kept.append((name, seed, bsa.Problem.from_buffer_copy(p), idx.cpu().numpy(), wt.cpu().numpy()))
        return statistics.mean(_rel_err_per_head(o, dense, w.N)), _d_ratio(lse, lse_d, w.N)

    res = {"workload": w.name, "values": w.value_mode, "key_spread": w.key_spread, "temperature": w.temperature,
           "k_exact": w.k_exact, "m_sample": w.m_sample, "density": round(w.density, 4),
           "top_mass": round(top_mass, 4), "seeds": len(seeds)}

    S_ib = bsa.score_ibcs(base, q, k, perm, groups=4, iters=3)[0]
    S_st = bsa.score_stats(base, q, k, perm)[0]

    M = unit_mass(w, q, k, perm)
    n_l = min(L, S.shape[-1])
    res["mass_best"] = float(torch.topk(M, n_l, dim=-1).values.sum(-1).mean())
    for name, Sx in (("plain", S), ("ibcs", S_ib), ("stats", S_st)):
        top = torch.topk(Sx, n_l, dim=-1).indices
        res["mass_" + name] = float(M.gather(-1, top).sum(-1).mean())
    if w.k_exact > 0:
        ex_p = torch.topk(S, w.k_exact, dim=-1).indices.sort(-1).values
        ex_s = torch.topk(S_st, w.k_exact, dim=-1).indices.sort(-1).values
        res["exact_diff_stats"] = float((ex_p != ex_s).any(-1).float().mean())
    del M

    p_tr = bsa.problem_for(w, out_fp32=1, k_exact=L, m_sample=0)
    idx, wt = bsa.select(p_tr, S)
    res["truncation"], res["truncation_dr"] = err(p_tr, idx, wt, "truncation")
    idx, wt = bsa.select(p_tr, S_ib)
    res["truncation_ibcs"], res["truncation_ibcs_dr"] = err(p_tr, idx, wt)
    idx, wt = bsa.select(p_tr, S_st)
    res["truncation_stats"], res["truncation_stats_dr"] = err(p_tr, idx, wt)

    runs = {"unweighted": [], "weighted": [], "sample_only": [], "weighted_ibcs": [], "weighted_stats": []}
    for s in seeds:
        p = bsa.problem_for(w, seed=s, out_fp32=1)
        idx, wt = bsa.select(p, S)
        runs["weighted"].append(err(p, idx, wt, "weighted", s))
        runs["unweighted"].append(err(p, idx, torch.ones_like(wt), "unweighted", s))
        p0 = bsa.problem_for(w, seed=s, out_fp32=1, k_exact=0, m_sample=L)
        idx0, wt0 = bsa.select(p0, S)
        runs["sample_only"].append(err(p0, idx0, wt0, "sample_only", s))
        idx, wt = bsa.select(p, S_ib)
        runs["weighted_ibcs"].append(err(p, idx, wt))
        idx, wt = bsa.select(p, S_st)
        runs["weighted_stats"].append(err(p, idx, wt))
    for name, vals in runs.items():
        errs = [e for e, _ in vals]
        res[name] = statistics.mean(errs)
        res[name + "_std"] = statistics.pstdev(errs) if len(errs) > 1 else 0.0
        res[name + "_dr"] = statistics.mean(r for _, r in vals)
    torch.cuda.synchronize()
    out = {key: round(val, 5) if isinstance(val, float) else val for key, val in res.items()}
    if keep_lists:
        out["lists"] = kept
    return out


def main(argv=None):
    from block_sparse_attention_27_amd.inputs import WORKLOADS

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="wan14b_480p", choices=sorted(WORKLOADS))
    ap.add_argument("--temps", type=float, nargs="+", default=[0.5, 1.0, 2.0])
    ap.add_argument("--seeds", type=int, default=8, help="selection seeds per sampled estimator")
    ap.add_argument("--values", nargs="+", default=["noise", "clustered"], choices=["noise", "clustered"])
    ap.add_argument("--key-spread", default="uniform", choices=["uniform", "clustered"])
    args = ap.parse_args(argv)

    import torch
    if not torch.cuda.is_available():
        print("the estimator study runs the library's GPU kernels; no GPU is visible", file=sys.stderr)
        return 2
    base = WORKLOADS[args.workload]
    for vm in args.values:
        for tau in args.temps:
            w = base.replace(temperature=tau, value_mode=vm, key_spread=args.key_spread)
            print(f"[study] {w.name} values={vm} tau={tau}", file=sys.stderr, flush=True)
            res = run_temperature(w, list(range(args.seeds)),
                                  log=lambda m: print(m, file=sys.stderr, flush=True))
            print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
