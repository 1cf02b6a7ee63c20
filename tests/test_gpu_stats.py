"""bsa_score_stats on the GPU against the oracle's statistics-aware scorer:
scores within the score bar (|dS| <= 1e-3 S_ref + 1e-12 max_j S_ref), the key
means and variances within 1e-5 relative L2, over small whole tensors (d, Bq,
Bk, dtype, permutation) and sampled heads of the 720p and HunyuanVideo layers.
Units of identical keys must score as in bsa_score."""

import numpy as np
import pytest
import torch

import block_sparse_attention_27_amd as bsa
import oracle
from block_sparse_attention_27_amd.inputs import Workload, WORKLOADS, generate
from gpu_util import to_device, host_f64, rel_l2, print_case

pytestmark = pytest.mark.gpu


def _check(S, S_ref):
    got = S.astype(np.float64)
    ref = S_ref.astype(np.float64)
    tol = 1e-3 * ref + 1e-12 * ref.max(axis=-1, keepdims=True)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(got - ref) / np.maximum(ref, 1e-30))))


@pytest.mark.parametrize("d,bq,bk,dtype,perm", [(128, 128, 128, "bf16", False), (128, 128, 32, "bf16", True),
                                                (64, 64, 64, "bf16", False), (128, 64, 128, "fp32", True),
                                                (64, 128, 32, "fp32", False)])
def test_stats_small_whole_tensors(d, bq, bk, dtype, perm):
    print_case(f"stats scorer d={d} bq={bq} bk={bk} {dtype} perm={perm}")
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    w = Workload("stats", B=2, H=2, grid=(3, 17, 23), d=d, dtype=dtype, block_q=bq, block_k=bk,
                 k_exact=2, m_sample=3, clusters=6, temperature=0.8, permute=perm, seed=5)
    g = generate(w)
    pd = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    p = bsa.problem_for(w)
    S, qm, km, kv = bsa.score_stats(p, to_device(g["q"]), to_device(g["k"]), pd)
    torch.cuda.synchronize()
    S_ref, qb, kb, kvar = oracle.score_stats(host_f64(g["q"]), host_f64(g["k"]), w.N, bq, bk, w.sm_scale, g["perm"])
    _check(S.cpu().numpy(), S_ref)
    assert rel_l2(km.cpu().numpy(), kb) < 1e-5 and rel_l2(qm.cpu().numpy(), qb) < 1e-5
    assert rel_l2(kv.cpu().numpy(), kvar) < 1e-5


def test_stats_identical_keys_match_plain_scorer():
    print_case("stats scorer: units of identical keys")
    rng = np.random.default_rng(6)
    B, H, N, Np, d, bk = 1, 2, 1000, 1024, 128, 64
    q = (rng.standard_normal((B, H, Np, d)) * 0.3).astype(np.float32)
    k = np.repeat((rng.standard_normal((B, H, Np // bk, d)) * 0.3).astype(np.float32), bk, axis=2)
    q[..., N:, :] = 0
    k[..., N:, :] = 0
    p = bsa.Problem(B=B, H=H, N=N, N_pad=Np, d=d, block_q=128, block_k=bk, k_exact=1, m_sample=1,
                    dtype=bsa.BSA_FP32, out_fp32=0, seed=0, sm_scale=1.0, kv_permuted=0)
    qd, kd = to_device(q), to_device(k)
    S1, _, _, kv = bsa.score_stats(p, qd, kd)
    S0, _, _ = bsa.score(p, qd, kd)
    torch.cuda.synchronize()
    assert float(kv.abs().max()) < 1e-10
    a, b = S1.cpu().numpy().astype(np.float64), S0.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(a - b) <= 1e-5 * b + 1e-12 * b.max(-1, keepdims=True))


@pytest.mark.parametrize("name,heads", [("wan14b_720p", [0, 39]), ("hunyuan", [7])])
def test_stats_full_size_sampled_heads(name, heads):
    print_case(f"{name}: bsa_score_stats at full size, heads {heads}")
    w = WORKLOADS[name]
    g = generate(w)
    pd = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    p = bsa.problem_for(w)
    S, _, _, kv = bsa.score_stats(p, to_device(g["q"]), to_device(g["k"]), pd)
    torch.cuda.synchronize()
    S, kv = S.cpu().numpy(), kv.cpu().numpy()
    for h in heads:
        S_ref, _, _, kvar = oracle.score_stats(host_f64(g["q"][:, h:h + 1]), host_f64(g["k"][:, h:h + 1]), w.N,
                                               w.block_q, w.block_k, w.sm_scale, g["perm"])
        _check(S[:, h:h + 1], S_ref)
        assert rel_l2(kv[:, h:h + 1], kvar) < 1e-5
