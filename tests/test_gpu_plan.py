"""Sampling-plan reuse on the GPU: lists built from one step's activations are
reused for a later step's attention, which must equal the oracle's attention
on the later activations with those lists (same bars as test_gpu_parity);
refreshing the plan must give the oracle's selection on the new scores."""

import numpy as np
import pytest
import torch

import block_sparse_attention_27_amd as bsa
import oracle
from block_sparse_attention_27_amd.inputs import Workload, generate
from gpu_util import to_device, host_f64, rel_l2, print_case

pytestmark = pytest.mark.gpu


def _wl(seed, perm):
    return Workload("plan", B=1, H=2, grid=(3, 16, 24), d=128, dtype="bf16", block_q=128, block_k=64,
                    k_exact=3, m_sample=6, clusters=6, temperature=1.0, permute=perm, seed=seed,
                    select_seed=7)


@pytest.mark.parametrize("perm", [False, True])
def test_plan_reuse_across_steps(perm):
    print_case(f"sampling plan reused across two steps, permuted={perm}")
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w1, w2 = _wl(0, perm), _wl(1, perm)
    g1, g2 = generate(w1), generate(w2)
    pm = g1["perm"]                      # the token order is part of the plan's geometry
    pm_d = torch.from_numpy(pm).cuda() if pm is not None else None
    p = bsa.problem_for(w1, out_fp32=1)
    q1, k1 = to_device(g1["q"]), to_device(g1["k"])
    q2, k2, v2 = (to_device(g2[x]) for x in ("q", "k", "v"))

    plan = bsa.SamplingPlan(p, q1, k1, pm_d)
    S1, _, _ = bsa.score(p, q1, k1, pm_d)
    out = plan.attend(q2, k2, v2, pm_d)
    torch.cuda.synchronize()
    idx, wt = plan.idx.cpu().numpy(), plan.w.cpu().numpy()
    i_ref, w_ref = oracle.select(S1.cpu().numpy(), w1.N, w1.block_k, w1.k_exact, w1.m_sample, w1.select_seed)
    assert np.array_equal(idx, i_ref)
    assert np.array_equal(wt.view(np.uint32), w_ref.view(np.uint32))

    qh, kh, vh = (host_f64(g2[x]) for x in ("q", "k", "v"))
    O_ref, _ = oracle.attend(qh, kh, vh, w1.N, w1.block_q, w1.block_k, w1.sm_scale, i_ref, w_ref, pm)
    o = out.cpu().numpy().astype(np.float64)
    assert rel_l2(o[..., :w1.N, :], O_ref[..., :w1.N, :]) < 2e-3
    assert np.max(np.abs(o - O_ref)) < 1e-2

    plan.refresh(q2, k2, pm_d)
    S2, _, _ = bsa.score(p, q2, k2, pm_d)
    torch.cuda.synchronize()
    i2, w2r = oracle.select(S2.cpu().numpy(), w1.N, w1.block_k, w1.k_exact, w1.m_sample, w1.select_seed)
    assert np.array_equal(plan.idx.cpu().numpy(), i2)
    assert np.array_equal(plan.w.cpu().numpy().view(np.uint32), w2r.view(np.uint32))
    assert not np.array_equal(i2, i_ref)  # new activations, new plan
