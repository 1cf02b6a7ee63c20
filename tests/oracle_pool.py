"""Runs the oracle's selection over many rows in worker processes (CPU only).

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
    chunks = [rows[c::n_chunks] for c in range(n_chunks)]
    # only the (b, h) slices a chunk reads travel to its worker
    jobs = [({(b, h): S[b, h] for b, h in {(b, h) for b, h, _ in ch}}, n_valid, k, m, seed, ch) for ch in chunks]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(workers, mp_context=ctx) as ex:
        outs = list(ex.map(_select_chunk, jobs))
    idx = np.empty((len(rows), k + m), dtype=np.int32)
    w = np.empty((len(rows), k + m), dtype=np.float32)
    for c, (ri, rw) in enumerate(outs):
        idx[c::n_chunks] = ri
        w[c::n_chunks] = rw
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
