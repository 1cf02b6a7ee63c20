"""Runs the oracle's selection and attention over many rows or heads in worker processes (CPU only).

The workers import NumPy and the oracle, never torch or the HIP library: they
are fresh interpreters started as children (spawn), so they touch no GPU.
"""

import concurrent.futures
import multiprocessing
import os

import numpy as np

import oracle


def _select_chunk(args):
    slices, n_valid, k, m, seed, rows = args
    # the steps of oracle.select for each row: the row's Philox offset from its real (b, h, i), then select_row
    out = [oracle.select_row(slices[(b, h)][i], n_valid, k, m, oracle.block_offset(seed, b, h, i))
           for b, h, i in rows]
    return np.stack([r[0] for r in out]), np.stack([r[1] for r in out])


def select_rows(S: np.ndarray, N: int, block_k: int, k: int, m: int, seed: int, rows, workers: int = 8):
    """oracle selection over ``rows`` [(b, h, i), ...]; returns (idx [len, k+m], w [len, k+m]) in row order."""
    S = np.asarray(S, dtype=np.float32)
    n_valid = -(-N // block_k)
    workers = max(1, min(workers, len(os.sched_getaffinity(0))))
    n_chunks = max(1, min(len(rows), 4 * workers))
    # contiguous runs of the row list: rows listed head by head give each chunk one or two (b, h) slices
    bounds = [len(rows) * c // n_chunks for c in range(n_chunks + 1)]
    chunks = [rows[bounds[c]:bounds[c + 1]] for c in range(n_chunks)]
    # only the (b, h) slices a chunk reads travel to its worker
    jobs = [({(b, h): S[b, h] for b, h in {(b, h) for b, h, _ in ch}}, n_valid, k, m, seed, ch) for ch in chunks]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(workers, mp_context=ctx) as ex:
        outs = list(ex.map(_select_chunk, jobs))
    idx = np.empty((len(rows), k + m), dtype=np.int32)
    w = np.empty((len(rows), k + m), dtype=np.float32)
    for c, (ri, rw) in enumerate(outs):
        idx[bounds[c]:bounds[c + 1]] = ri
        w[bounds[c]:bounds[c + 1]] = rw
    return idx, w


def _seed_chunk(args):
    S_rows, n_valid, k, m, seeds = args
    idx = np.empty((len(seeds), len(S_rows), k + m), dtype=np.int32)
    w = np.empty((len(seeds), len(S_rows), k + m), dtype=np.float32)
    pis = None
    for a, seed in enumerate(seeds):
        for i, s in enumerate(S_rows):
            ri, rw, info = oracle.select_row(s, n_valid, k, m, oracle.block_offset(seed, 0, 0, i), details=True)
            idx[a, i], w[a, i] = ri, rw
            if pis is None or len(pis) <= i:
                pis = (pis or []) + [(info["R"], info["pi"])]
    return idx, w, pis


def select_seeds(S_rows: np.ndarray, N: int, block_k: int, k: int, m: int, seeds, workers: int = 8):
    """oracle selection of query blocks i = 0.. of (b, h) = (0, 0) for every seed.

    Returns (idx [seeds, rows, k+m], w [seeds, rows, k+m], [(R, pi_int) per row]).
    """
    S_rows = np.asarray(S_rows, dtype=np.float32)
    n_valid = -(-N // block_k)
    seeds = list(seeds)
    workers = max(1, min(workers, len(os.sched_getaffinity(0))))
    n_chunks = max(1, min(len(seeds), 4 * workers))
    chunks = [seeds[c::n_chunks] for c in range(n_chunks)]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(workers, mp_context=ctx) as ex:
        outs = list(ex.map(_seed_chunk, [(S_rows, n_valid, k, m, ch) for ch in chunks]))
    idx = np.empty((len(seeds), len(S_rows), k + m), dtype=np.int32)
    w = np.empty((len(seeds), len(S_rows), k + m), dtype=np.float32)
    for c, (ri, rw, _) in enumerate(outs):
        idx[c::n_chunks] = ri
        w[c::n_chunks] = rw
    return idx, w, outs[0][2]


def _f64_from_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exactly."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _attend_head(args):
    q, k, v, idx, w, out_gpu, lse_gpu, N, block_q, block_k, sm_scale, perm = args
    if q.dtype == np.uint16:
        q, k, v = _f64_from_bf16(q), _f64_from_bf16(k), _f64_from_bf16(v)
    O, L = oracle.attend(q[None, None], k[None, None], v[None, None], N, block_q, block_k, sm_scale,
                         idx[None, None], w[None, None], perm)
    O, L = O[0, 0], L[0, 0]
    rows = np.arange(O.shape[0]) < N  # un-permuted rows: the valid tokens are rows 0..N-1 either way
    got = out_gpu.astype(np.float64)
    d = got[rows] - O[rows]
    lg = lse_gpu.astype(np.float64)
    fin = np.isfinite(L[rows])
    return {"ss_diff": float(np.sum(d * d)), "ss_ref": float(np.sum(O[rows] ** 2)),
            "max_abs": float(np.max(np.abs(d), initial=0.0)),
            "max_lse": float(np.max(np.abs(lg[rows][fin] - L[rows][fin]), initial=0.0)),
            "lse_finite_match": bool(np.array_equal(np.isfinite(lg[rows]), fin)),
            "pad_zero": bool(np.all(got[~rows] == 0) and np.all(np.isneginf(lg[~rows])))}


def attend_heads(q, k, v, idx, w, out_gpu, lse_gpu, N, block_q, block_k, sm_scale, perm=None, heads=None,
                 workers: int = 16):
    """oracle attention over every query block of the given heads of batch 0, each head in a worker.

    q, k, v: host [B, H, N_pad, d] (uint16 bf16 bits or float); idx, w: [B, H, nQB, L]; out_gpu, lse_gpu: the
    kernel's outputs on the host ([B, H, N_pad, d] fp32 and [B, H, N_pad]). Returns one error record per head.
    """
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    workers = max(1, min(workers, len(os.sched_getaffinity(0)), len(heads)))
    jobs = [(q[0, h], k[0, h], v[0, h], idx[0, h], w[0, h], out_gpu[0, h], lse_gpu[0, h], N, block_q, block_k,
             sm_scale, perm) for h in heads]
    # one BLAS thread per worker: the workers already fill the cores
    knobs = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {n: os.environ.get(n) for n in knobs}
    os.environ.update({n: "1" for n in knobs})
    try:
        ctx = multiprocessing.get_context("spawn")
        with concurrent.futures.ProcessPoolExecutor(workers, mp_context=ctx) as ex:
            return list(ex.map(_attend_head, jobs))
    finally:
        for n, val in saved.items():
            if val is None:
                os.environ.pop(n, None)
            else:
                os.environ[n] = val
