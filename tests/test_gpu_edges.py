"""GPU edge cases against the oracle: ragged shapes, every (d, block_q, block_k,
dtype, permutation) combination, hostile score rows for the selection, list
entries the kernel must ignore, repeated entries, m = 0, the dense limit, and
run-to-run determinism. Same bars as test_gpu_parity."""

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


def _small(d, bq, bk, dtype, perm, grid=(3, 17, 23), k=3, m=5, H=3, B=2, tau=1.0, seed=0):
    return Workload("edge", B=B, H=H, grid=grid, d=d, dtype=dtype, block_q=bq, block_k=bk,
                    k_exact=k, m_sample=m, clusters=6, temperature=tau, permute=perm, seed=seed,
                    select_seed=seed + 11)


def _run_and_check(w, tol_out):
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    perm = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    p = bsa.problem_for(w)
    S, qm, km = bsa.score(p, q, k, perm)
    idx, wt = bsa.select(p, S)
    p32 = bsa.Problem.from_buffer_copy(p)
    p32.out_fp32 = 1
    out, lse = bsa.attend(p32, q, k, v, idx, wt, perm, with_lse=True)
    outd, lsed = bsa.attend_dense(p32, q, k, v, perm, with_lse=True)
    if w.dtype == "bf16":
        o16 = bsa.attend(p, q, k, v, idx, wt, perm)
        od16 = bsa.attend_dense(p, q, k, v, perm)
        torch.cuda.synchronize()
        assert torch.equal(o16.view(torch.int16), out.to(torch.bfloat16).view(torch.int16))
        assert torch.equal(od16.view(torch.int16), outd.to(torch.bfloat16).view(torch.int16))
    torch.cuda.synchronize()
    qh, kh, vh = (host_f64(g[x]) for x in ("q", "k", "v"))
    S_ref, qb, kb = oracle.score(qh, kh, w.N, w.block_q, w.block_k, w.sm_scale, g["perm"])
    Sg = S.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Sg - S_ref) <= 1e-3 * S_ref + 1e-12 * S_ref.max(-1, keepdims=True))
    assert rel_l2(qm.cpu().numpy(), qb) < 1e-5 and rel_l2(km.cpu().numpy(), kb) < 1e-5
    i_ref, w_ref = oracle.select(S.cpu().numpy(), w.N, w.block_k, w.k_exact, w.m_sample, w.select_seed)
    assert np.array_equal(idx.cpu().numpy(), i_ref)
    assert np.array_equal(wt.cpu().numpy().view(np.uint32), w_ref.view(np.uint32))
    O_ref, L_ref = oracle.attend(qh, kh, vh, w.N, w.block_q, w.block_k, w.sm_scale, i_ref, w_ref, g["perm"])
    Od_ref, Ld_ref = oracle.attend_dense(qh, kh, vh, w.N, w.sm_scale, g["perm"])
    for o, l, oref, lref in ((out, lse, O_ref, L_ref), (outd, lsed, Od_ref, Ld_ref)):
        og = to_f64(o)
        assert rel_l2(og, oref) <= tol_out[0] and np.max(np.abs(og - oref)) <= tol_out[1]
        lg = l.cpu().numpy().astype(np.float64)
        assert np.all(np.isneginf(lg[..., w.N:]))
        fin = np.isfinite(lref)
        assert np.array_equal(np.isfinite(lg), fin)
        assert np.max(np.abs(lg[fin] - lref[fin])) < 2e-3
    return g, p, (q, k, v, perm), (S, idx, wt, out)


COMBOS = list(itertools.product([64, 128], [64, 128], [32, 64, 128], ["bf16", "fp32"], [False, True]))


@pytest.mark.parametrize("d,bq,bk,dtype,perm", COMBOS)
def test_ragged_shapes_all_variants(d, bq, bk, dtype, perm):
    print_case(f"ragged d={d} bq={bq} bk={bk} {dtype} perm={perm}")
    w = _small(d, bq, bk, dtype, perm)
    tol = (2e-3, 1e-2) if dtype == "bf16" else (1e-5, 1e-5)
    _run_and_check(w, tol)


def test_tiny_n_single_partial_block():
    print_case("N = 45 tokens, one partial query block, one partial unit")
    _run_and_check(_small(128, 128, 128, "bf16", False, grid=(1, 5, 9), k=1, m=0), (2e-3, 1e-2))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dense_limit_matches_dense_kernel(dtype):
    print_case(f"dense limit {dtype}: k+m = all valid units")
    w = _small(128, 128, 32, dtype, True, grid=(2, 9, 14), k=4, m=0)
    n_valid = w.n_valid_units
    w = w.replace(k_exact=4, m_sample=n_valid - 4)
    g, p, (q, k, v, perm), (S, idx, wt, out) = _run_and_check(w, (2e-3, 1e-2) if dtype == "bf16" else (1e-5, 1e-5))
    assert np.all(wt.cpu().numpy() == 1.0)
    p32 = bsa.Problem.from_buffer_copy(p)
    p32.out_fp32 = 1
    # dense attention reads the keys in the order it is given them; on K' and V'
    # it meets them in the sparse pass's order (units ascending), so the two
    # round P to bf16 over the same tiles
    kp, vp = bsa.permute_rows(p, k, perm), bsa.permute_rows(p, v, perm)
    outd = bsa.attend_dense(bsa.with_kv_permuted(p32), q, kp, vp, perm)
    torch.cuda.synchronize()
    a, b = to_f64(out), to_f64(outd)
    assert rel_l2(a, b) <= 2e-3 and np.max(np.abs(a - b)) <= 1e-2


def test_top_k_only_m_zero():
    print_case("m = 0: exact set only")
    _run_and_check(_small(128, 128, 64, "bf16", False, k=4, m=0), (2e-3, 1e-2))


def test_ignored_and_repeated_list_entries():
    print_case("lists with out-of-range indices, non-positive / NaN / inf weights, repeats")
    w = _small(128, 128, 32, "bf16", False, k=2, m=6)
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    p = bsa.problem_for(w, out_fp32=1)
    rng = np.random.default_rng(5)
    shape = (w.B, w.H, w.n_qblocks, w.list_len)
    idx = rng.integers(0, w.n_valid_units, shape).astype(np.int32)
    wts = (1.0 + 3.0 * rng.random(shape)).astype(np.float32)
    bad_idx = rng.random(shape) < 0.15
    idx[bad_idx] = rng.choice([-1, -7, w.n_units, w.n_units + 100], bad_idx.sum())
    bad_w = (~bad_idx) & (rng.random(shape) < 0.15)
    wts[bad_w] = rng.choice(np.array([0.0, -1.0, np.nan, np.inf], np.float32), bad_w.sum())
    idx[..., 1] = idx[..., 0]  # repeats
    wts[..., 1] = wts[..., 0]
    out = bsa.attend(p, q, k, v, torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    ok = (idx >= 0) & (idx < w.n_units) & (wts > 0) & np.isfinite(wts)
    qh, kh, vh = (host_f64(g[x]) for x in ("q", "k", "v"))
    got = to_f64(out)
    ref = np.zeros_like(got)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(w.n_qblocks):
                keep = ok[b, h, i]
                rows = slice(i * w.block_q, (i + 1) * w.block_q)
                if not keep.any():
                    assert np.all(got[b, h, rows] == 0)
                    continue
                ref[b, h, rows], _ = oracle.attend_block(qh[b, h], kh[b, h], vh[b, h], i, idx[b, h, i][keep],
                                                         wts[b, h, i][keep], w.N, w.block_q, w.block_k,
                                                         w.sm_scale)
    # the bar applies to the output tensor as a whole
    assert rel_l2(got, ref) <= 2e-3 and np.max(np.abs(got - ref)) <= 1e-2


@pytest.mark.parametrize("bq", [64, 128])
@pytest.mark.parametrize("runs", [1, 2, 3, 4, 5, 12])
def test_list_made_of_ascending_runs(bq, runs):
    """The kernels rank a list of a few ascending runs by binary searches and any
    other list by a full scan; both must give the oracle's result, with units
    repeated inside and across runs (ties keep their list order)."""
    print_case(f"lists of {runs} ascending runs, bq={bq}")
    w = _small(128, bq, 32, "bf16", False, k=10, m=20)
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    p = bsa.problem_for(w, out_fp32=1)
    rng = np.random.default_rng(100 + runs)
    shape = (w.B, w.H, w.n_qblocks, w.list_len)
    idx = rng.integers(0, w.n_valid_units, shape).astype(np.int32)
    cuts = np.sort(rng.choice(np.arange(1, w.list_len), runs - 1, replace=False)) if runs > 1 else []
    for seg in np.split(np.arange(w.list_len), cuts):
        idx[..., seg] = np.sort(idx[..., seg], axis=-1)
    wts = (0.5 + 3.5 * rng.random(shape)).astype(np.float32)
    out = bsa.attend(p, q, k, v, torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    qh, kh, vh = (host_f64(g[x]) for x in ("q", "k", "v"))
    got = to_f64(out)
    ref = np.zeros_like(got)
    for b in range(w.B):
        for h in range(w.H):
            for i in range(w.n_qblocks):
                rows = slice(i * w.block_q, (i + 1) * w.block_q)
                ref[b, h, rows], _ = oracle.attend_block(qh[b, h], kh[b, h], vh[b, h], i, idx[b, h, i], wts[b, h, i],
                                                         w.N, w.block_q, w.block_k, w.sm_scale)
    assert rel_l2(got, ref) <= 2e-3 and np.max(np.abs(got - ref)) <= 1e-2


def _hostile_rows(n_rows, n_valid, n_units, rng):
    S = np.zeros((n_rows, n_units), dtype=np.float32)
    for r in range(n_rows):
        kind = r % 8
        if kind == 0:
            x = rng.standard_normal(n_valid) * 3
            s = np.exp(x - x.max())
        elif kind == 1:
            s = rng.integers(0, 3, n_valid).astype(np.float64)  # heavy ties
        elif kind == 2:
            s = np.zeros(n_valid)  # all zero
        elif kind == 3:
            s = rng.random(n_valid) * 1e-40  # subnormal
        elif kind == 4:
            s = rng.random(n_valid) ** 30  # huge dynamic range
        elif kind == 5:
            s = np.full(n_valid, 0.25)  # uniform
        elif kind == 6:
            s = rng.random(n_valid)
            s[rng.integers(0, n_valid, 3)] = [np.nan, -1.0, np.inf]
        else:
            s = np.where(rng.random(n_valid) < 0.05, 1.0, 1e-7)  # a few spikes
        S[r, :n_valid] = s
        S[r, n_valid:] = rng.random(n_units - n_valid)  # junk beyond the valid units: never read
    return S


@pytest.mark.parametrize("n_valid,k,m", [(1, 1, 0), (5, 0, 5), (7, 2, 3), (256, 8, 18), (257, 20, 40),
                                         (511, 1, 100), (591, 20, 40), (1024, 50, 300), (2047, 96, 200),
                                         (3713, 96, 200), (4096, 0, 4096), (4096, 300, 7)])
def test_selection_hostile_rows_bitexact(n_valid, k, m):
    print_case(f"selection hostile rows n_valid={n_valid} k={k} m={m}")
    bk = 32
    N = n_valid * bk - 5 if n_valid > 1 else 20
    N_pad = -(-N // 128) * 128
    n_units = N_pad // bk
    nqb = N_pad // 128
    H = 1
    rows_cap = 64 if n_valid > 1000 else 400
    p = bsa.Problem(B=1, H=H, N=N, N_pad=N_pad, d=128, block_q=128, block_k=bk, k_exact=k, m_sample=m,
                    dtype=bsa.BSA_BF16, seed=0xDEADBEEF12345678, sm_scale=1.0, kv_permuted=0)
    rng = np.random.default_rng(n_valid)
    S = _hostile_rows(nqb, n_valid, n_units, rng).reshape(1, H, nqb, n_units)
    idx, wt = bsa.select(p, torch.from_numpy(S).cuda())
    torch.cuda.synchronize()
    idx, wt = idx.cpu().numpy(), wt.cpu().numpy()
    rows = [(0, 0, i) for i in range(min(nqb, rows_cap))]
    for (b, h, i), (ri, rw) in zip(rows, oracle.select(S, N, bk, k, m, 0xDEADBEEF12345678, rows=rows)):
        assert np.array_equal(idx[b, h, i], ri), (i, idx[b, h, i][:12], ri[:12])
        assert np.array_equal(wt[b, h, i].view(np.uint32), rw.view(np.uint32)), i


def test_determinism_bitwise():
    print_case("two runs give identical bytes")
    w = _small(128, 128, 32, "bf16", True, grid=(4, 16, 24), k=6, m=10)
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    perm = torch.from_numpy(g["perm"]).cuda()
    p = bsa.problem_for(w)
    r1 = bsa.sparse_attention(p, q, k, v, perm, with_lse=True)
    r2 = bsa.sparse_attention(p, q, k, v, perm, with_lse=True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("d,bq,dtype,perm", [(64, 64, "fp32", False), (128, 128, "bf16", True)])
def test_scores_more_units_than_the_logit_cache(d, bq, dtype, perm):
    # 655 key units of 32 (the last holds 23 keys) is more than the 640 whose logits the one-representative
    # score kernel keeps in LDS: the score pass then runs on the kernel that stages the key means once per
    # workgroup, with a ragged last workgroup of query blocks
    print_case(f"scores with 655 units d={d} bq={bq} {dtype} perm={perm}")
    w = Workload("units", B=1, H=2, grid=(7, 41, 73), d=d, dtype=dtype, block_q=bq, block_k=32,
                 k_exact=2, m_sample=3, clusters=6, temperature=1.0, permute=perm, seed=12)
    assert w.n_valid_units == 655 and w.N % 32 == 23
    g = generate(w)
    q, k = to_device(g["q"]), to_device(g["k"])
    pm = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    p = bsa.problem_for(w)
    S, qm, km = bsa.score(p, q, k, pm)
    torch.cuda.synchronize()
    qh, kh = host_f64(g["q"]), host_f64(g["k"])
    S_ref, qb, kb = oracle.score(qh, kh, w.N, w.block_q, w.block_k, w.sm_scale, g["perm"])
    Sg = S.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(Sg - S_ref) <= 1e-3 * S_ref + 1e-12 * S_ref.max(-1, keepdims=True))
    assert np.all(Sg[..., w.n_valid_units:] == 0)
    assert rel_l2(qm.cpu().numpy(), qb) < 1e-5 and rel_l2(km.cpu().numpy(), kb) < 1e-5


@pytest.mark.parametrize("bq,dtype", [(128, "bf16"), (64, "bf16"), (128, "fp32")])
def test_extreme_weights(bq, dtype):
    # caller-built lists with weights from 2^-100 to FLT_MAX: the running maximum is kept on the
    # weighted logits, so nothing overflows and the result is the oracle's (fp64) weighted softmax
    print_case(f"extreme weights: bq={bq} {dtype}")
    w = _small(128, bq, 64, dtype, False, k=2, m=6, seed=3)
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    p = bsa.problem_for(w, out_fp32=1)
    rng = np.random.default_rng(13)
    shape = (w.B, w.H, w.n_qblocks, w.list_len)
    idx = rng.integers(0, w.n_valid_units, shape).astype(np.int32)
    wts = np.exp2(rng.uniform(-100, 100, shape)).astype(np.float32)
    wts[:, :, ::3, 0] = np.finfo(np.float32).max
    wts[:, :, 1::3, 1] = np.finfo(np.float32).tiny
    out, lse = bsa.attend(p, q, k, v, torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda(), with_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh = (host_f64(g[x]) for x in ("q", "k", "v"))
    O_ref, L_ref = oracle.attend(qh, kh, vh, w.N, w.block_q, w.block_k, w.sm_scale, idx, wts)
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    assert rel_l2(got, O_ref) <= 2e-3 and np.max(np.abs(got - O_ref)) <= 1e-2
    lg = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - L_ref[fin]) / np.maximum(1.0, np.abs(L_ref[fin]))) < 2e-3


@pytest.mark.parametrize("perm", [False, True])
def test_lists_longer_than_one_chunk(perm):
    # 1,100 list entries per query block: the attention kernel takes them in sorted chunks (of at
    # most 512 entries for 128-row query blocks; with a permutation, the gathered-row ring restarts
    # per chunk)
    print_case(f"lists of 1100 entries (two chunks), permuted={perm}")
    w = Workload("long", B=1, H=1, grid=(12, 50, 80), d=128, dtype="bf16", block_q=128, block_k=32,
                 k_exact=100, m_sample=1000, clusters=16, temperature=1.0, permute=perm, seed=9, select_seed=4)
    assert w.list_len > 1024 and w.n_valid_units > w.list_len
    g = generate(w)
    q, k, v = (to_device(g[x]) for x in ("q", "k", "v"))
    pm = torch.from_numpy(g["perm"]).cuda() if g["perm"] is not None else None
    p = bsa.problem_for(w, out_fp32=1)
    S, _, _ = bsa.score(p, q, k, pm)
    idx, wt = bsa.select(p, S)
    out, lse = bsa.attend(p, q, k, v, idx, wt, pm, with_lse=True)
    torch.cuda.synchronize()
    idx_h, wt_h = idx.cpu().numpy(), wt.cpu().numpy()
    assert len(np.unique(idx_h[0, 0, 3])) > 1024  # the lists really hold more than one chunk of units
    blocks = [0, 97, w.n_qblocks - 1]
    ref = oracle.attend(host_f64(g["q"]), host_f64(g["k"]), host_f64(g["v"]), w.N, w.block_q, w.block_k,
                        w.sm_scale, idx_h, wt_h, g["perm"], blocks=[(0, 0, i) for i in blocks])
    got_all, ref_all = [], []
    for i, (o_ref, l_ref) in zip(blocks, ref):
        rows = np.arange(i * w.block_q, (i + 1) * w.block_q)
        orows = np.where(rows < w.N, g["perm"][rows] if perm else rows, rows)
        got = out[0, 0, torch.from_numpy(orows).cuda()].cpu().numpy().astype(np.float64)
        gl = lse[0, 0, torch.from_numpy(orows).cuda()].cpu().numpy().astype(np.float64)
        ok = rows < w.N
        assert np.max(np.abs(gl[ok] - l_ref[ok])) < 2e-3
        got_all.append(got[ok]); ref_all.append(o_ref[ok])
    got_all, ref_all = np.concatenate(got_all), np.concatenate(ref_all)
    assert rel_l2(got_all, ref_all) < 2e-3 and np.max(np.abs(got_all - ref_all)) < 1e-2
