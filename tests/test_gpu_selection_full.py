"""bsa_select on the GPU against the oracle on whole layers and over many seeds.

Bar: idx and the bit patterns of w equal the oracle's, fed the same fp32 S
(InstaGen, Abstract: one random draw per query block, shared by its queries;
the draw is word 0 of Philox4x32-10 at counter (i, h, b, 0) and key = seed).

* every one of the 23,640 rows of the Wan2.1-14B 720p layer (40 heads x 591
  query blocks, 591 units per row), S from bsa_score on the GPU;
* 10,220 rows of the HunyuanVideo layer (every query block of 11 heads, 3,713
  valid 32-key units per row, the long-row kernel), S from bsa_score;
* a sweep of 20 seeds over a 2-head 480p-shaped layer: 10,240 (counter, key)
  pairs.
The oracle's selection runs in CPU worker processes (tests/oracle_pool.py).
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_27_amd as bsa
from block_sparse_attention_27_amd.inputs import WORKLOADS, generate
from gpu_util import print_case, to_device
from oracle_pool import select_rows

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


def test_selection_every_row_of_the_720p_layer():
    w = WORKLOADS["wan14b_720p"]
    p = bsa.problem_for(w)
    print_case(f"720p: score + select on the GPU, all {w.B * w.H * w.n_qblocks} rows vs the oracle")
    S, idx, wt = _gpu_scores_and_lists(w, p)
    rows = [(b, h, i) for b in range(w.B) for h in range(w.H) for i in range(w.n_qblocks)]
    _compare(w, p, S, idx, wt, rows, w.select_seed)


def test_selection_hunyuan_ten_thousand_rows():
    w = WORKLOADS["hunyuan"]
    p = bsa.problem_for(w)
    print_case("hunyuan: score + select on the GPU, every query block of heads 0..10 vs the oracle")
    S, idx, wt = _gpu_scores_and_lists(w, p)
    rows = [(0, h, i) for h in range(11) for i in range(w.n_qblocks)]
    rows.append((0, w.H - 1, w.n_qblocks - 1))
    assert len(rows) >= 10_000
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
