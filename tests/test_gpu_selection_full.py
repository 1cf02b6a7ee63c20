"""bsa_select on the GPU against the oracle on whole layers and over many seeds.

Bar: idx and the bit patterns of w equal the oracle's, fed the same fp32 S
(InstaGen, Abstract: one random draw per query block, shared by its queries;
the draw is word 0 of Philox4x32-10 at counter (i, h, b, 0) and key = seed).

* every row of the Wan2.1-1.3B (3,072 rows of 256 units), 480p (10,240 rows),
  720p (23,640 rows of 591 units) and HunyuanVideo (22,296 rows of 3,713 valid
  32-key units, the long-row kernel) layers, S from bsa_score on the GPU;
* a sweep of 20 seeds over a 2-head 480p-shaped layer: 10,240 (counter, key)
  pairs;
* 10,000 seeds on four 16-unit rows, every (seed, row) bit-exact, and the
  empirical inclusion frequency of every unit against its pi (systematic
  sampling takes unit j with probability pi_j whatever the offset's seed).
The oracle's selection runs in CPU worker processes (tests/oracle_pool.py).
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_27_amd as bsa
from block_sparse_attention_27_amd.inputs import WORKLOADS, generate
from gpu_util import print_case, to_device
from oracle_pool import select_rows, select_seeds

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bsa.load_library()


def _gpu_scores_and_lists(w, p):
    g = generate(w)
    q, k = to_device(g["q"]), to_device(g["k"])
    perm = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    S, _, _ = bsa.score(p, q, k, perm)
    idx, wt = bsa.select(p, S)
    torch.cuda.synchronize()
    del q, k
    return S, idx, wt


def _compare(w, p, S, idx, wt, rows, seed):
    S_h = S.cpu().numpy()
    i_ref, w_ref = select_rows(S_h, w.N, w.block_k, p.k_exact, p.m_sample, seed, rows)
    idx_h, wt_h = idx.cpu().numpy(), wt.cpu().numpy()
    got_i = np.stack([idx_h[b, h, i] for b, h, i in rows])
    got_w = np.stack([wt_h[b, h, i] for b, h, i in rows])
    bad = np.nonzero(~(np.all(got_i == i_ref, axis=1) & np.all(got_w.view(np.uint32) == w_ref.view(np.uint32), axis=1)))[0]
    assert bad.size == 0, (f"{bad.size} of {len(rows)} rows differ; first {rows[bad[0]]}: "
                           f"gpu {got_i[bad[0]][:8]}.. ref {i_ref[bad[0]][:8]}..")
    print_case(f"  {len(rows)} rows bit-exact")


@pytest.mark.parametrize("name", ["wan13b", "wan14b_480p", "wan14b_720p", "hunyuan"])
def test_selection_every_row_of_the_layer(name):
    w = WORKLOADS[name]
    p = bsa.problem_for(w)
    print_case(f"{name}: score + select on the GPU, all {w.B * w.H * w.n_qblocks} rows "
               f"({w.n_valid_units} valid units each) vs the oracle")
    S, idx, wt = _gpu_scores_and_lists(w, p)
    rows = [(b, h, i) for b in range(w.B) for h in range(w.H) for i in range(w.n_qblocks)]
    _compare(w, p, S, idx, wt, rows, w.select_seed)


def test_selection_seed_sweep():
    w = WORKLOADS["wan14b_480p"].replace(H=2)
    p = bsa.problem_for(w)
    print_case("480p-shaped, 2 heads: 20 seeds x 512 rows = 10,240 (counter, key) pairs")
    S, _, _ = _gpu_scores_and_lists(w, p)
    rows = [(0, h, i) for h in range(w.H) for i in range(w.n_qblocks)]
    seeds = [0, 1, 2, 3, 0xFFFFFFFF, 1 << 32, (1 << 64) - 1, 0x9E3779B97F4A7C15] + list(range(1000, 1012))
    for seed in seeds:
        ps = bsa.Problem.from_buffer_copy(p)
        ps.seed = seed
        idx, wt = bsa.select(ps, S)
        torch.cuda.synchronize()
        _compare(w, ps, S, idx, wt, rows, seed)


def test_selection_ten_thousand_seeds_and_inclusion_frequencies():
    """Four query blocks of 16 units (2 exact + 5 sampled): scores with a dominant
    unit (capped at pi = 1), a zero, and a spread of gamma-distributed values."""
    print_case("10,000 seeds x 4 rows of 16 units, k = 2, m = 5")
    rng = np.random.default_rng(2024)
    S_rows = rng.gamma(0.6, size=(4, 16)).astype(np.float32)
    S_rows[0, 3] = 40.0   # dominant: capped
    S_rows[1, 5] = 0.0    # quantised to the minimum
    S_rows[2, :] = 1.0    # uniform row
    S_rows /= S_rows.sum(axis=1, keepdims=True)
    n_seeds = 10_000
    p = bsa.Problem(B=1, H=1, N=512, N_pad=512, d=128, block_q=128, block_k=32, k_exact=2, m_sample=5,
                    dtype=bsa.BSA_BF16, out_fp32=0, seed=0, sm_scale=1.0, kv_permuted=0)
    S = torch.from_numpy(S_rows.reshape(1, 1, 4, 16)).cuda()
    idx_all = torch.empty((n_seeds, 1, 1, 4, 7), dtype=torch.int32, device="cuda")
    w_all = torch.empty((n_seeds, 1, 1, 4, 7), dtype=torch.float32, device="cuda")
    for s in range(n_seeds):
        p.seed = s * 0x9E3779B97F4A7C15 % (1 << 64)  # seeds spread over all 64 bits
        bsa.bsa_select(p, S, idx_all[s], w_all[s])
    torch.cuda.synchronize()
    gi = idx_all.cpu().numpy().reshape(n_seeds, 4, 7)
    gw = w_all.cpu().numpy().reshape(n_seeds, 4, 7)
    seeds = [s * 0x9E3779B97F4A7C15 % (1 << 64) for s in range(n_seeds)]
    ri, rw, pis = select_seeds(S_rows, 512, 32, 2, 5, seeds)
    assert np.array_equal(gi, ri)
    assert np.array_equal(gw.view(np.uint32), rw.view(np.uint32))
    # empirical inclusion frequency of every unit of R in the sample part against pi
    for i, (R, pi) in enumerate(pis):
        counts = np.zeros(16)
        for row in gi[:, i, 2:]:
            counts[row] += 1
        for pos, j in enumerate(R):
            pj = pi[pos] / 2.0 ** 32
            f = counts[j] / n_seeds
            sigma = np.sqrt(pj * (1 - pj) / n_seeds)
            assert abs(f - pj) <= 5 * sigma + 1e-12, (i, j, f, pj)
        assert counts.sum() == 5 * n_seeds
    print_case("  40,000 (seed, row) selections bit-exact; inclusion frequencies within 5 sigma of pi")
