"""Concurrent use: the library keeps no state, so passes on different streams,
enqueued from different host threads at the same time, give the results of
the same passes run one after another, bit for bit.

Two layers of different shapes (one permuted, with K and V put into the
permuted order first) each run score -> select -> attend -> dense on their own
stream (default priority), from their own host thread (ctypes releases the GIL
during each call), four times over; every output must equal the one from the
sequential run on the default stream.
"""

import threading

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


def _layer(name, bk, permute, seed):
    w = Workload(name, B=1, H=4, grid=(4, 24, 40), d=128, dtype="bf16", block_q=128, block_k=bk, k_exact=6,
                 m_sample=10, clusters=8, temperature=1.0, permute=permute, seed=seed, select_seed=seed + 1)
    g = generate(w)
    dev = [to_device(g[x]) for x in ("q", "k", "v")]
    perm = torch.from_numpy(g["perm"]).cuda() if permute else None
    return w, dev, perm


def _pass(w, q, k, v, perm, stream):
    p = bsa.problem_for(w, out_fp32=1)
    with torch.cuda.stream(stream):
        if perm is not None:
            k, v = bsa.permute_rows(p, k, perm, stream=stream), bsa.permute_rows(p, v, perm, stream=stream)
            p = bsa.with_kv_permuted(p)
        S, _, _ = bsa.score(p, q, k, perm, stream=stream)
        idx, wt = bsa.select(p, S, stream=stream)
        out, lse = bsa.attend(p, q, k, v, idx, wt, perm, with_lse=True, stream=stream)
        dense = bsa.attend_dense(p, q, k, v, perm, stream=stream)
    return [S, idx, wt, out, lse, dense]


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def test_two_streams_from_two_threads():
    print_case("two layers on two streams from two host threads, 4 rounds, against the sequential run")
    layers = [_layer("streamA", 64, False, 3), _layer("streamB", 32, True, 5)]
    ref = [_pass(w, *dev, perm, torch.cuda.current_stream()) for w, dev, perm in layers]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for rnd in range(4):
        results = [None, None]
        errors = []

        def work(j):
            try:
                w, dev, perm = layers[j]
                results[j] = _pass(w, *dev, perm, streams[j])
            except Exception as e:  # surfaced below, on the main thread
                errors.append(e)

        threads = [threading.Thread(target=work, args=(j,)) for j in range(2)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        assert not errors, errors
        for j in range(2):
            for name, a, b in zip(("S", "idx", "w", "out", "lse", "dense"), ref[j], results[j]):
                assert torch.equal(_bits(a), _bits(b)), (rnd, j, name)
    print_case("  every round bit-identical to the sequential run")
