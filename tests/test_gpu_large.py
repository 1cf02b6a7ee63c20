"""Tensors past 2^31 elements: 64-bit offsets in every kernel of the pass.

34 heads of 523,904 rows (a 31 x 131 x 129 latent grid, N = 523,869, a ragged
last block) at d = 128: a head holds 67,059,712 elements, so the bf16 Q, K and
V pass 2^31 bytes at head 17 and 2^32 bytes (2^31 elements) in head 32; the
fp32 output passes 2^33 bytes, the score matrix (34 x 4,093 x 4,093 fp32)
2^31 bytes, and the 32-key-unit lists 2^25 entries. The head-0, head-17 and
head-33 inputs come from the clustered generator; every other head is a copy
of head 17, so a head read at a wrapped offset would return another head's
values. On the whole tensors, in the launch configuration of the full layers:

* bsa_score, bsa_select, bsa_attend (128-key units) and bsa_attend_dense,
  checked against the oracle on heads 0, 17 and 33 (scores whole; selection on
  sampled rows, bit-exact; attention on sampled query blocks including the
  ragged last one);
* bsa_permute_rows of K and V through the clustered gather index (sampled rows
  bit-exact) and bsa_attend on 32-key units with lists of 12 units, once with
  K and V permuted first (kv_permuted = 1) and once gathering inside: the two
  outputs are bit-identical over the whole tensor and match the oracle on
  sampled blocks;
* bsa_attend on 64-row query blocks and 64-key units, K and V gathered through
  the index inside (the 8-wave kernel);
* fp32 Q, K and V (9.1 GB each): scores, selection and the fp32 attention
  kernel, within 1e-5 of the oracle;
* the clustering scorer through the gather index (group sizes bit-exact) and
  the statistics-aware scorer.

Bars as in the full-layer parity tests: scores 1e-3 relative, selection
bit-exact, attention 2e-3 relative L2 and 1e-2 max-abs, lse 2e-3.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_27_amd as bsa
import oracle
from block_sparse_attention_27_amd.inputs import Workload, generate
from gpu_util import to_f64, host_f64, rel_l2, print_case

pytestmark = pytest.mark.gpu

W = Workload("past_2e31", B=1, H=34, grid=(31, 131, 129), d=128, dtype="bf16", block_q=128, block_k=128,
             k_exact=4, m_sample=4, clusters=128, temperature=1.0, permute=True, seed=11, select_seed=5)
MADE = (0, 17, 33)  # heads drawn by the generator; the rest copy head 17
SCORE_RTOL = 1e-3
OUT_REL_L2 = 2e-3
OUT_MAX_ABS = 1e-2
LSE_ABS = 2e-3


@pytest.fixture(scope="module")
def data():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bsa.load_library()
    assert W.H * W.N_pad * W.d > 2 ** 31 and 33 * W.N_pad * W.d > 2 ** 31
    print_case(f"{W.name}: generating heads {MADE} (N={W.N}, N_pad={W.N_pad})")
    g = generate(W, heads=MADE)
    dev = {}
    for name in ("q", "k", "v"):
        t = torch.empty((W.B, W.H, W.N_pad, W.d), dtype=torch.bfloat16, device="cuda")
        for j, h in enumerate(MADE):
            t[:, h] = torch.from_numpy(g[name][:, j].view(np.int16)).view(torch.bfloat16).cuda()
        for h in range(W.H):
            if h not in MADE:
                t[:, h] = t[:, 17]
        dev[name] = t
    torch.cuda.synchronize()
    yield g, dev
    del dev
    torch.cuda.empty_cache()


def _host_head(g, name, h):
    """fp64 [1, 1, N_pad, d] copy of one generated head."""
    j = MADE.index(h)
    return host_f64(g[name][:, j:j + 1])


def _check_rows(got_rows, ref_rows, what):
    got = np.concatenate(got_rows)
    ref = np.concatenate(ref_rows)
    r, m = rel_l2(got, ref), float(np.max(np.abs(got - ref)))
    print_case(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= OUT_REL_L2 and m <= OUT_MAX_ABS, (what, r, m)


def _check_blocks(out, lse, refs, h, blocks, block_q, perm=None):
    """Compare the GPU rows of query blocks (in the computed order) with the oracle's."""
    got_rows, ref_rows = [], []
    for i, (o_ref, l_ref) in zip(blocks, refs):
        rows = np.arange(i * block_q, (i + 1) * block_q)
        valid = rows < W.N
        orows = np.where(valid, perm[rows] if perm is not None else rows, rows)
        sel = torch.from_numpy(orows).cuda()
        got = to_f64(out[0, h, sel])
        assert np.all(got[~valid] == 0), (h, i)
        got_rows.append(got[valid])
        ref_rows.append(o_ref[valid])
        if lse is not None:
            gl = lse[0, h, sel].cpu().numpy().astype(np.float64)
            assert np.all(np.isneginf(gl[~valid])), (h, i)
            assert np.max(np.abs(gl[valid] - l_ref[valid]), initial=0) < LSE_ABS, (h, i)
    return got_rows, ref_rows


def test_pass_past_2e31_elements(data):
    g, dev = data
    q, k, v = dev["q"], dev["k"], dev["v"]
    p = bsa.problem_for(W, out_fp32=1)
    print_case(f"{W.name}: bsa_score, bsa_select, bsa_attend (128-key units) over {W.H} heads")
    S, _, _ = bsa.score(p, q, k)
    idx, wt = bsa.select(p, S)
    out, lse = bsa.attend(p, q, k, v, idx, wt, with_lse=True)
    torch.cuda.synchronize()

    nQB = W.n_qblocks
    blocks = [0, 1, nQB // 2, nQB - 1]
    rng = np.random.default_rng(3)
    S_rows = np.zeros(S.shape, dtype=np.float32)  # untouched pages stay unallocated
    rows = []
    got_rows, ref_rows = [], []
    for h in MADE:
        print_case(f"  head {h}: scores, selection and attention vs oracle")
        qh, kh, vh = (_host_head(g, x, h) for x in ("q", "k", "v"))
        S_ref, _, _ = oracle.score(qh, kh, W.N, W.block_q, W.block_k, W.sm_scale)
        got = S[0, h].cpu().numpy().astype(np.float64)
        ref = S_ref[0, 0].astype(np.float64)
        bad = np.abs(got - ref) > SCORE_RTOL * ref + 1e-12 * ref.max(axis=-1, keepdims=True)
        assert not bad.any(), (h, int(bad.sum()))
        S_rows[0, h] = S[0, h].cpu().numpy()
        rows += [(0, h, i) for i in sorted(set(blocks + rng.integers(0, nQB, 6).tolist()))]

        idx_h = idx[0:1, h:h + 1].cpu().numpy()
        wt_h = wt[0:1, h:h + 1].cpu().numpy()
        refs = oracle.attend(qh, kh, vh, W.N, W.block_q, W.block_k, W.sm_scale, idx_h, wt_h,
                             blocks=[(0, 0, i) for i in blocks])
        gr, rr = _check_blocks(out, lse, refs, h, blocks, W.block_q)
        got_rows += gr
        ref_rows += rr
    _check_rows(got_rows, ref_rows, "sparse attention")

    print_case(f"  selection bit-exactness on {len(rows)} rows")
    idx_all, wt_all = idx.cpu().numpy(), wt.cpu().numpy()
    for (b, h, i), (ri, rw) in zip(rows, oracle.select(S_rows, W.N, W.block_k, W.k_exact, W.m_sample,
                                                        W.select_seed, rows=rows)):
        assert np.array_equal(idx_all[b, h, i], ri), (b, h, i)
        assert np.array_equal(wt_all[b, h, i].view(np.uint32), rw.view(np.uint32)), (b, h, i)
    del S, idx, wt, out, lse, S_rows
    torch.cuda.empty_cache()

    print_case(f"{W.name}: bsa_attend_dense over {W.H} heads")
    out_d, lse_d = bsa.attend_dense(p, q, k, v, with_lse=True)
    torch.cuda.synchronize()
    got_rows, ref_rows = [], []
    for h, i in ((33, nQB - 1), (17, 0)):
        qh, kh, vh = (_host_head(g, x, h) for x in ("q", "k", "v"))
        refs = oracle.attend_dense(qh, kh, vh, W.N, W.sm_scale, blocks=[(0, 0, i)], block_q=W.block_q)
        gr, rr = _check_blocks(out_d, lse_d, refs, h, [i], W.block_q)
        got_rows += gr
        ref_rows += rr
    _check_rows(got_rows, ref_rows, "dense attention")
    del out_d, lse_d
    torch.cuda.empty_cache()


def test_permuted_32_key_units_past_2e31_elements(data):
    g, dev = data
    q, k, v = dev["q"], dev["k"], dev["v"]
    perm = g["perm"]
    perm_d = torch.from_numpy(perm).cuda()
    p = bsa.problem_for(W, block_k=32, k_exact=6, m_sample=6, out_fp32=1)
    n_valid = -(-W.N // 32)
    print_case(f"{W.name}: bsa_permute_rows of K and V ({W.H} heads)")
    kk = bsa.permute_rows(p, k, perm_d)
    vv = bsa.permute_rows(p, v, perm_d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    r = np.unique(np.concatenate([[0, W.N - 1, W.N, W.N_pad - 1], rng.integers(0, W.N_pad, 64)]))
    for h in MADE:
        j = MADE.index(h)
        for name, src, got in (("k", g["k"], kk), ("v", g["v"], vv)):
            rows = got[0, h, torch.from_numpy(r).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
            want = np.where((r < W.N)[:, None], src[0, j, np.where(r < W.N, perm[r], 0)], 0)
            assert np.array_equal(rows, want), (name, h)

    idx, wt = _explicit_lists(rng, (W.B, W.H, W.n_qblocks), n_valid, 12, 1361)
    idx_d, wt_d = torch.from_numpy(idx).cuda(), torch.from_numpy(wt).cuda()

    print_case(f"{W.name}: bsa_attend on 32-key units, K and V permuted first and gathered inside")
    out_a, lse_a = bsa.attend(bsa.with_kv_permuted(p), q, kk, vv, idx_d, wt_d, perm_d, with_lse=True)
    del kk, vv
    out_b = bsa.attend(p, q, k, v, idx_d, wt_d, perm_d)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32))
    del out_b
    torch.cuda.empty_cache()

    nQB = W.n_qblocks
    blocks = [0, nQB // 3, nQB - 1]
    got_rows, ref_rows = [], []
    for h in (0, 33):
        print_case(f"  head {h}: attention vs oracle")
        qh, kh, vh = (_host_head(g, x, h) for x in ("q", "k", "v"))
        refs = oracle.attend(qh, kh, vh, W.N, W.block_q, 32, W.sm_scale, idx[:, h:h + 1], wt[:, h:h + 1], perm,
                             blocks=[(0, 0, i) for i in blocks])
        gr, rr = _check_blocks(out_a, lse_a, refs, h, blocks, W.block_q, perm)
        got_rows += gr
        ref_rows += rr
    _check_rows(got_rows, ref_rows, "permuted sparse attention")


def _explicit_lists(rng, n_rows_shape, n_valid, L, step):
    """L distinct valid units per row (start + step e mod n_valid, L step < n_valid), shuffled; weights in [0.5, 4)."""
    assert L * step < n_valid
    shape = n_rows_shape + (L,)
    start = rng.integers(0, n_valid, n_rows_shape + (1,))
    idx = ((start + step * np.arange(L)) % n_valid).astype(np.int32)
    idx = np.take_along_axis(idx, np.argsort(rng.random(shape), axis=-1), axis=-1)
    wt = rng.uniform(0.5, 4.0, shape).astype(np.float32)
    return idx, wt


def test_64_row_blocks_gathered_past_2e31_elements(data):
    g, dev = data
    q, k, v = dev["q"], dev["k"], dev["v"]
    perm = g["perm"]
    bq = bk = 64
    p = bsa.problem_for(W, block_q=bq, block_k=bk, k_exact=4, m_sample=4, out_fp32=1)
    nQB = W.N_pad // bq
    n_valid = -(-W.N // bk)
    idx, wt = _explicit_lists(np.random.default_rng(5), (W.B, W.H, nQB), n_valid, 8, 1013)
    print_case(f"{W.name}: bsa_attend on 64-row query blocks, K and V gathered through perm inside")
    out, lse = bsa.attend(p, q, k, v, torch.from_numpy(idx).cuda(), torch.from_numpy(wt).cuda(),
                          torch.from_numpy(perm).cuda(), with_lse=True)
    torch.cuda.synchronize()
    blocks = [0, nQB // 2, nQB - 1]
    got_rows, ref_rows = [], []
    for h in (0, 33):
        qh, kh, vh = (_host_head(g, x, h) for x in ("q", "k", "v"))
        refs = oracle.attend(qh, kh, vh, W.N, bq, bk, W.sm_scale, idx[:, h:h + 1], wt[:, h:h + 1], perm,
                             blocks=[(0, 0, i) for i in blocks])
        gr, rr = _check_blocks(out, lse, refs, h, blocks, bq, perm)
        got_rows += gr
        ref_rows += rr
    _check_rows(got_rows, ref_rows, "64-row blocks")


def test_fp32_inputs_past_2e31_elements(data):
    """fp32 Q, K, V (9.1 GB each): block means, scores, selection and the fp32 attention kernel."""
    g, dev = data
    q, k, v = (dev[x].float() for x in ("q", "k", "v"))  # exact widening of the bf16 values
    p = bsa.problem_for(W, dtype=bsa.BSA_FP32)
    print_case(f"{W.name}: fp32 inputs, bsa_score, bsa_select, bsa_attend over {W.H} heads")
    S, _, _ = bsa.score(p, q, k)
    idx, wt = bsa.select(p, S)
    out, lse = bsa.attend(p, q, k, v, idx, wt, with_lse=True)
    torch.cuda.synchronize()
    del q, k, v
    nQB = W.n_qblocks
    blocks = [0, nQB // 2, nQB - 1]
    S_rows = np.zeros(S.shape, dtype=np.float32)
    rows = []
    for h in (0, 33):
        qh, kh, vh = (_host_head(g, x, h) for x in ("q", "k", "v"))
        S_ref, _, _ = oracle.score(qh, kh, W.N, W.block_q, W.block_k, W.sm_scale)
        got = S[0, h].cpu().numpy().astype(np.float64)
        ref = S_ref[0, 0].astype(np.float64)
        bad = np.abs(got - ref) > SCORE_RTOL * ref + 1e-12 * ref.max(axis=-1, keepdims=True)
        assert not bad.any(), (h, int(bad.sum()))
        S_rows[0, h] = S[0, h].cpu().numpy()
        rows += [(0, h, i) for i in blocks]
        refs = oracle.attend(qh, kh, vh, W.N, W.block_q, W.block_k, W.sm_scale, idx[0:1, h:h + 1].cpu().numpy(),
                             wt[0:1, h:h + 1].cpu().numpy(), blocks=[(0, 0, i) for i in blocks])
        gr, rr = _check_blocks(out, lse, refs, h, blocks, W.block_q)
        got = np.concatenate(gr)
        ref = np.concatenate(rr)
        r, m = rel_l2(got, ref), float(np.max(np.abs(got - ref)))
        print_case(f"  head {h}: fp32 attention rel_l2={r:.3e} max_abs={m:.3e}")
        assert r < 1e-5 and m < 1e-5, (h, r, m)
    idx_all, wt_all = idx.cpu().numpy(), wt.cpu().numpy()
    for (b, h, i), (ri, rw) in zip(rows, oracle.select(S_rows, W.N, W.block_k, W.k_exact, W.m_sample,
                                                        W.select_seed, rows=rows)):
        assert np.array_equal(idx_all[b, h, i], ri), (b, h, i)
        assert np.array_equal(wt_all[b, h, i].view(np.uint32), rw.view(np.uint32)), (b, h, i)


def test_alternative_scorers_past_2e31_elements(data):
    """bsa_score_ibcs (G = 4, T = 3, through the gather index) and bsa_score_stats on the whole tensors."""
    g, dev = data
    q, k = dev["q"], dev["k"]
    perm = g["perm"]
    p = bsa.problem_for(W)
    print_case(f"{W.name}: bsa_score_ibcs (G=4, T=3, permuted) and bsa_score_stats over {W.H} heads")
    S_i, qc, qs, _ = bsa.score_ibcs(p, q, k, torch.from_numpy(perm).cuda(), groups=4, iters=3)
    S_s, _, km, kv = bsa.score_stats(p, q, k)
    torch.cuda.synchronize()
    nQB = W.n_qblocks
    n_rows = oracle.valid_counts(W.N, W.N_pad, W.block_q)
    blocks = [0, nQB // 2, nQB - 1]
    for h in (0, 33):
        qh, kh = _host_head(g, "q", h), _host_head(g, "k", h)
        rows, reps, sizes = oracle.score_ibcs(qh, kh, W.N, W.block_q, W.block_k, W.sm_scale, 4, 3, perm,
                                              blocks=[(0, 0, i) for i in blocks])
        for i, s_ref, c_ref, z_ref in zip(blocks, rows, reps, sizes):
            z_got = qs[0, h, i].cpu().numpy()
            assert np.array_equal(z_got, z_ref) and z_got.sum() == n_rows[i], (h, i, z_got, z_ref)
            assert rel_l2(qc[0, h, i].cpu().numpy().astype(np.float64), c_ref) < 1e-5, (h, i)
            got = S_i[0, h, i].cpu().numpy().astype(np.float64)
            ref = s_ref.astype(np.float64)
            assert not (np.abs(got - ref) > SCORE_RTOL * ref + 1e-12 * ref.max()).any(), (h, i)
        S_ref, _, kb, kvar = oracle.score_stats(qh, kh, W.N, W.block_q, W.block_k, W.sm_scale)
        assert rel_l2(km[0, h].cpu().numpy().astype(np.float64), kb[0, 0]) < 1e-5, h
        assert rel_l2(kv[0, h].cpu().numpy().astype(np.float64), kvar[0, 0]) < 1e-5, h
        got = S_s[0, h].cpu().numpy().astype(np.float64)
        ref = S_ref[0, 0].astype(np.float64)
        bad = np.abs(got - ref) > SCORE_RTOL * ref + 1e-12 * ref.max(axis=-1, keepdims=True)
        assert not bad.any(), (h, int(bad.sum()))
        print_case(f"  head {h}: clustering scorer (3 blocks) and statistics-aware scorer (whole head) match")
