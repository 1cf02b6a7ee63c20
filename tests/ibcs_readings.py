"""How far the clustering scorer's fixed-point reading departs from plain Lloyd k-means on layer-shaped blocks.

CPU only; calls the oracle and the seeded input generator, nothing of the HIP path. For every query
block of the chosen heads it runs both readings of the intra-block k-means (``oracle.cluster_block``:
rows and centroids on the 2^(e-11) grid; ``oracle.lloyd_block``: plain fp64 Lloyd on the raw rows; same
initial rows, iteration count and tie rule) and reports

* the blocks whose group sizes differ, and the blocks that the rounding margin certifies;
* over the blocks that differ, the change in the block's score row (the group-size-weighted mixture of
  the groups' estimated attention masses), elementwise relative and as an L1 distance.

usage: python tests/ibcs_readings.py wan14b_720p 0,1 [groups iters]
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_attention_27_amd.inputs import WORKLOADS, as_float32, generate  # noqa: E402
from oracle.ibcs import certified_agreement, cluster_block, group_mixture, lloyd_block  # noqa: E402
from oracle.scoring import apply_perm, block_means, valid_counts  # noqa: E402


def compare(name: str, heads, groups: int = 4, iters: int = 3) -> dict:
    w = WORKLOADS[name]
    g = generate(w, heads=heads)
    counts = valid_counts(w.N, w.N_pad, w.block_q)
    n_j = valid_counts(w.N, w.N_pad, w.block_k).astype(np.float64)
    tot = differ = cert = cert_differ = 0
    rel, l1 = [], []
    for hi in range(len(heads)):
        q = apply_perm(as_float32(g["q"][:, hi:hi + 1]).astype(np.float64), g["perm"])[0, 0]
        kb = block_means(as_float32(g["k"][:, hi:hi + 1]).astype(np.float64), w.N, w.block_k, g["perm"])[0, 0]
        for i in range(w.n_qblocks):
            n = int(counts[i])
            if n == 0:
                continue
            rows = q[i * w.block_q: i * w.block_q + n]
            r1, s1 = cluster_block(rows, groups, iters)
            r2, s2 = lloyd_block(rows, groups, iters)
            c = certified_agreement(rows, groups, iters)
            d = not np.array_equal(s1, s2)
            tot += 1
            cert += c
            differ += d
            cert_differ += c and d
            if d:
                S1 = group_mixture(r1, s1 / n, kb, n_j, w.sm_scale)
                S2 = group_mixture(r2, s2 / n, kb, n_j, w.sm_scale)
                rel.append(float(np.max(np.abs(S1 - S2) / np.maximum(S2, 1e-300))))
                l1.append(float(np.abs(S1 - S2).sum()))
    return {"workload": name, "heads": list(heads), "blocks": tot, "sizes_differ": differ, "certified": cert,
            "certified_but_differ": cert_differ,
            "score_rel_max": max(rel) if rel else 0.0, "score_rel_median": float(np.median(rel)) if rel else 0.0,
            "score_l1_max": max(l1) if l1 else 0.0}


if __name__ == "__main__":
    name = sys.argv[1] if len(sys.argv) > 1 else "wan14b_720p"
    heads = [int(x) for x in (sys.argv[2] if len(sys.argv) > 2 else "0,1").split(",")]
    G = int(sys.argv[3]) if len(sys.argv) > 3 else 4
    T = int(sys.argv[4]) if len(sys.argv) > 4 else 3
    r = compare(name, heads, G, T)
    print(r)
