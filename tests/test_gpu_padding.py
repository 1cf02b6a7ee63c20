"""Padding is never read: NaN in the padding rows of Q, K and V, and garbage in
the permutation entries past N, leave every output bit-identical.

The C ABI states that rows N..N_pad-1 of Q, K and V are never read and that
permutation entries r >= N are not read. Each case runs the whole library on a
ragged shape twice -- once with the generator's zero padding and an identity
tail of the permutation, once with NaN in every padding row and out-of-range
values in the permutation's tail -- and compares every output bit for bit:
block means and scores of all three scorers, the lists, sparse attention
(fp32 and bf16 output, and with K and V permuted first), dense attention, lse
and the permuted K and V.
"""

import numpy as np
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


CASES = [
    # d, block_q, block_k, dtype, permuted
    (128, 128, 128, "bf16", False),
    (128, 128, 32, "bf16", True),
    (128, 128, 64, "bf16", False),
    (64, 64, 64, "bf16", True),
    (128, 64, 32, "fp32", False),
    (64, 128, 64, "fp32", True),
]


def _bits(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _run(w, q, k, v, perm):
    p = bsa.problem_for(w)
    p32 = bsa.problem_for(w, out_fp32=1)
    r = {}
    r["S"], r["q_mean"], r["k_mean"] = bsa.score(p, q, k, perm)
    r["idx"], r["w"] = bsa.select(p, r["S"])
    r["out"], r["lse"] = bsa.attend(p32, q, k, v, r["idx"], r["w"], perm, with_lse=True)
    if w.dtype == "bf16":
        r["out_bf16"] = bsa.attend(p, q, k, v, r["idx"], r["w"], perm)
    r["dense"], r["dense_lse"] = bsa.attend_dense(p32, q, k, v, perm, with_lse=True)
    if perm is not None:
        r["k_perm"] = bsa.permute_rows(p, k, perm)
        r["v_perm"] = bsa.permute_rows(p, v, perm)
        r["out_kv_permuted"] = bsa.attend(bsa.with_kv_permuted(p32), q, r["k_perm"], r["v_perm"], r["idx"], r["w"],
                                          perm)
    r["S_ibcs"], r["q_cent"], r["q_size"], r["k_mean_ibcs"] = bsa.score_ibcs(p, q, k, perm, groups=4, iters=3)
    r["S_stats"], r["q_mean_stats"], r["k_mean_stats"], r["k_var"] = bsa.score_stats(p, q, k, perm)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("d,bq,bk,dtype,permuted", CASES)
def test_padding_rows_and_permutation_tail_are_never_read(d, bq, bk, dtype, permuted):
    w = Workload("pad", B=1, H=2, grid=(3, 17, 29), d=d, dtype=dtype, block_q=bq, block_k=bk, k_exact=3,
                 m_sample=5, clusters=6, temperature=1.0, permute=permuted, seed=4, select_seed=8)
    assert w.N % 128 != 0 and w.N_pad > w.N
    print_case(f"padding never read: d={d} Bq={bq} Bk={bk} {dtype} permuted={permuted} N={w.N} N_pad={w.N_pad}")
    g = generate(w)
    clean = [to_device(g[x]) for x in ("q", "k", "v")]
    dirty = [t.clone() for t in clean]
    for t in dirty:
        t[:, :, w.N:, :] = float("nan")
    perm_clean = perm_dirty = None
    if permuted:
        perm_clean = torch.from_numpy(g["perm"]).cuda()
        tail = np.array([-7, 1 << 30, w.N_pad + 3, w.N_pad, -1], dtype=np.int32)
        pd = g["perm"].copy()
        pd[w.N:] = np.resize(tail, w.N_pad - w.N)
        perm_dirty = torch.from_numpy(pd).cuda()
    a = _run(w, *clean, perm_clean)
    b = _run(w, *dirty, perm_dirty)
    for name in a:
        assert torch.equal(_bits(a[name]), _bits(b[name])), name
        if a[name].is_floating_point():
            assert not torch.isnan(a[name]).any(), name
    print_case(f"  {len(a)} outputs bit-identical")
