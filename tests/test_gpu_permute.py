"""GPU tests of bsa_permute_rows and of the kv_permuted mode.

bsa_permute_rows moves bytes only, so it is compared bit for bit with the
oracle's row gather. With kv_permuted = 1 the kernels take K' = K[perm] and
V' = V[perm] as given and gather only the query rows (and scatter the output
rows): every sum and product then sees the same values in the same order as
when the kernels gather K and V themselves, so S, the lists, out and lse must
equal those of kv_permuted = 0 bit for bit. The oracle comparison of the
gather-inside path is in test_gpu_edges and test_gpu_parity; the permuted
pass through the convenience wrapper is checked against the oracle here too."""

import itertools

import numpy as np
import pytest
import torch

import block_sparse_attention_27_amd as bsa
import oracle
from block_sparse_attention_27_amd.inputs import Workload, generate
from gpu_util import to_device, to_f64, host_f64, rel_l2, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bsa.load_library()


def _small(d, bq, bk, dtype, grid=(3, 17, 23), k=3, m=5, H=3, B=2, seed=0):
    return Workload("perm", B=B, H=H, grid=grid, d=d, dtype=dtype, block_q=bq, block_k=bk,
                    k_exact=k, m_sample=m, clusters=6, temperature=1.0, permute=True, seed=seed,
                    select_seed=seed + 11)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


@pytest.mark.parametrize("d,dtype,grid", [(128, "bf16", (3, 17, 23)), (64, "bf16", (2, 9, 11)),
                                          (128, "fp32", (2, 9, 11)), (64, "fp32", (1, 1, 37))])
def test_permute_rows_is_the_row_gather(d, dtype, grid):
    print_case(f"permute_rows d={d} {dtype} grid={grid}")
    w = _small(d, 128, 64, dtype, grid=grid)
    g = generate(w)
    p = bsa.problem_for(w)
    perm = torch.from_numpy(g["perm"]).cuda()
    for name in ("q", "k", "v"):
        x = to_device(g[name])
        xp = bsa.permute_rows(p, x, perm)
        torch.cuda.synchronize()
        got = _bits(xp)
        host = g[name] if g[name].dtype == np.uint16 else g[name].view(np.uint32)
        ref = oracle.apply_perm(host, g["perm"])
        assert np.array_equal(got[..., : w.N, :], ref[..., : w.N, :])
        assert not got[..., w.N:, :].any()  # rows past N are zeros


def test_permute_rows_entry_outside_the_rows_gives_a_zero_row():
    print_case("permute_rows with out-of-range entries")
    w = _small(128, 128, 64, "bf16", grid=(2, 9, 11))
    g = generate(w)
    p = bsa.problem_for(w)
    pm = g["perm"].copy()
    pm[7] = w.N_pad + 5
    pm[9] = -3
    x = to_device(g["k"])
    xp = bsa.permute_rows(p, x, torch.from_numpy(pm).cuda())
    torch.cuda.synchronize()
    got = _bits(xp)
    ref = oracle.apply_perm(g["k"], np.clip(pm, 0, w.N_pad - 1))
    bad = np.zeros(w.N_pad, dtype=bool)
    bad[[7, 9]] = True
    bad[w.N:] = True
    assert np.array_equal(got[..., ~bad, :], ref[..., ~bad, :])
    assert not got[..., bad, :].any()


COMBOS = list(itertools.product([64, 128], [64, 128], [32, 64, 128], ["bf16", "fp32"]))


@pytest.mark.parametrize("d,bq,bk,dtype", COMBOS)
def test_kv_permuted_equals_gathering_inside(d, bq, bk, dtype):
    print_case(f"kv_permuted d={d} bq={bq} bk={bk} {dtype}")
    w = _small(d, bq, bk, dtype)
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    perm = torch.from_numpy(g["perm"]).cuda()
    p = bsa.problem_for(w)
    p32 = bsa.Problem.from_buffer_copy(p)
    p32.out_fp32 = 1
    kp, vp = bsa.permute_rows(p, k, perm), bsa.permute_rows(p, v, perm)
    pk, pk32 = bsa.with_kv_permuted(p), bsa.with_kv_permuted(p32)

    S0, qm0, km0 = bsa.score(p, q, k, perm)
    S1, qm1, km1 = bsa.score(pk, q, kp, perm)
    T0 = bsa.score_stats(p, q, k, perm)
    T1 = bsa.score_stats(pk, q, kp, perm)
    C0 = bsa.score_ibcs(p, q, k, perm, groups=4, iters=3)
    C1 = bsa.score_ibcs(pk, q, kp, perm, groups=4, iters=3)
    idx0, w0 = bsa.select(p, S0)
    idx1, w1 = bsa.select(pk, S1)
    o0, l0 = bsa.attend(p32, q, k, v, idx0, w0, perm, with_lse=True)
    o1, l1 = bsa.attend(pk32, q, kp, vp, idx1, w1, perm, with_lse=True)
    outs = [(o0, o1), (l0, l1)]
    if dtype == "bf16":
        outs.append((bsa.attend(p, q, k, v, idx0, w0, perm), bsa.attend(pk, q, kp, vp, idx1, w1, perm)))
    od1, ld1 = bsa.attend_dense(pk32, q, kp, vp, perm, with_lse=True)
    torch.cuda.synchronize()
    for a, b in [(S0, S1), (qm0, qm1), (km0, km1), *zip(T0, T1), *zip(C0, C1), (idx0, idx1), (w0, w1), *outs]:
        assert np.array_equal(_bits(a) if a.dtype != torch.int32 else a.cpu().numpy(),
                              _bits(b) if b.dtype != torch.int32 else b.cpu().numpy())
    # dense attention on the permuted K' and V' against the oracle (token-order K, V and perm)
    qh, kh, vh = (host_f64(g[x]) for x in ("q", "k", "v"))
    Od_ref, Ld_ref = oracle.attend_dense(qh, kh, vh, w.N, w.sm_scale, g["perm"])
    tol = (2e-3, 1e-2) if dtype == "bf16" else (1e-5, 1e-5)
    og = to_f64(od1)
    assert rel_l2(og, Od_ref) <= tol[0] and np.max(np.abs(og - Od_ref)) <= tol[1]
    lg = ld1.cpu().numpy().astype(np.float64)
    assert np.all(np.isneginf(lg[..., w.N:]))
    assert np.max(np.abs(lg[..., : w.N] - Ld_ref[..., : w.N])) < 2e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_sparse_attention_wrapper_on_a_permuted_sequence(dtype):
    """The wrapper gathers K and V once and runs the steps with kv_permuted = 1."""
    print_case(f"sparse_attention wrapper permuted {dtype}")
    w = _small(128, 128, 32, dtype, grid=(4, 18, 24), k=6, m=10, H=2, B=1, seed=3)
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    perm = torch.from_numpy(g["perm"]).cuda()
    p = bsa.problem_for(w, out_fp32=1)
    out, lse, idx, wt = bsa.sparse_attention(p, q, k, v, perm, with_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh = (host_f64(g[x]) for x in ("q", "k", "v"))
    S_ref, _, _ = oracle.score(qh, kh, w.N, w.block_q, w.block_k, w.sm_scale, g["perm"])
    S = bsa.score(p, q, k, perm)[0].cpu().numpy()
    assert np.all(np.abs(S.astype(np.float64) - S_ref) <= 1e-3 * S_ref + 1e-12 * S_ref.max(-1, keepdims=True))
    i_ref, w_ref = oracle.select(S, w.N, w.block_k, w.k_exact, w.m_sample, w.select_seed)
    assert np.array_equal(idx.cpu().numpy(), i_ref)
    assert np.array_equal(wt.cpu().numpy().view(np.uint32), w_ref.view(np.uint32))
    O_ref, L_ref = oracle.attend(qh, kh, vh, w.N, w.block_q, w.block_k, w.sm_scale, i_ref, w_ref, g["perm"])
    tol = (2e-3, 1e-2) if dtype == "bf16" else (1e-5, 1e-5)
    og = to_f64(out)
    assert rel_l2(og, O_ref) <= tol[0] and np.max(np.abs(og - O_ref)) <= tol[1]
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - L_ref[fin])) < 2e-3
