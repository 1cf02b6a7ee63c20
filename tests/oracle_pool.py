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
