"""The GPU pass is a Horvitz-Thompson estimator of the dense sums.

For a query row, the weighted denominator sum_j w_j sum_t e^{a_rt} is exp(lse)
and the weighted numerator is out * exp(lse). Over the sampler's randomness
(one offset per query block, from the seed) each is unbiased for the dense
sum (InstaGen, Abstract: sampled blocks reweighted by the inverse of their
chance; AB-Attention transcript: unbiasedness of the two sums). With
bsa_select and bsa_attend on the GPU over 2,000 seeds, their averages must meet
the dense sums of bsa_attend_dense within six standard errors (about 32,000
values are checked). fp32 inputs keep the kernels' rounding far below the
statistical resolution.
"""

import pytest
import torch

import block_sparse_attention_27_amd as bsa
from block_sparse_attention_27_amd.inputs import Workload, generate
from gpu_util import to_device, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bsa.load_library()


def test_sums_are_unbiased_over_seeds():
    print_case("Horvitz-Thompson over 2,000 seeds (fp32, 2 heads, 4 query blocks, 8 units of 32)")
    w = Workload("ht", B=1, H=2, grid=(2, 8, 16), d=64, dtype="fp32", block_q=64, block_k=32, k_exact=2,
                 m_sample=3, clusters=4, temperature=1.0, permute=False, seed=21, select_seed=0)
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    p = bsa.problem_for(w)
    S, _, _ = bsa.score(p, q, k)
    out_d, lse_d = bsa.attend_dense(p, q, k, v, with_lse=True)
    n_seeds = 2000
    idx = torch.empty((w.B, w.H, w.n_qblocks, w.list_len), dtype=torch.int32, device="cuda")
    wt = torch.empty_like(idx, dtype=torch.float32)
    out = torch.empty_like(q)
    lse = torch.empty_like(lse_d)
    valid = slice(0, w.N)
    den = torch.zeros_like(lse_d[..., valid], dtype=torch.float64)
    den2 = torch.zeros_like(den)
    num = torch.zeros_like(out_d[..., valid, :], dtype=torch.float64)
    num2 = torch.zeros_like(num)
    for s in range(n_seeds):
        p.seed = (s * 0x9E3779B97F4A7C15 + 1) % (1 << 64)
        bsa.bsa_select(p, S, idx, wt)
        bsa.bsa_attend(p, q, k, v, None, idx, wt, out, lse)
        r = torch.exp(lse[..., valid].double() - lse_d[..., valid].double())  # denominator / dense denominator
        x = out[..., valid, :].double() * r[..., None]                      # numerator / dense denominator
        den += r
        den2 += r * r
        num += x
        num2 += x * x
    torch.cuda.synchronize()
    n = float(n_seeds)
    for name, m1, m2, target in (("denominator", den, den2, torch.ones_like(den)),
                                 ("numerator", num, num2, out_d[..., valid, :].double())):
        mean = m1 / n
        se = torch.sqrt(torch.clamp(m2 / n - mean * mean, min=0.0) / (n - 1))
        dev = (mean - target).abs()
        bad = dev > 6 * se + 1e-5
        assert not bool(bad.any()), (name, float(dev.max()), float(se.max()))
    print_case("  both sums within 6 standard errors of the dense sums on every row")
