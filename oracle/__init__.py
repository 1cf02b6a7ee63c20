"""CPU oracle for weighted dynamic block-sparse attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what the HIP path computes, written
from the pages' description (InstaGen: group-shared importance sampling;
AB-Attention: accurate block attention) and checked against closed forms,
brute force and library routines by the CPU tests under ``tests/``.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The library and its Python binding never do: the
product path has no CPU fallback. It shares no code with the HIP path; both
sides are fed from the seeded generator in the package's ``inputs`` module,
which holds none of the method's arithmetic.

Modules, in the order the method runs:
  scoring    block means and the estimated-attention score matrix S
  ibcs       the intra-block clustering scorer: k-means groups per query block,
             S as the size-weighted mixture of the groups' estimated masses
  stats_score  the statistics-aware scorer: key units scored by the mass of a
             Gaussian with their mean and per-dimension variance
  selection  exact top-k set, inclusion probabilities, systematic sample, 1/pi weights
  philox     the counter-based generator that supplies one offset per query block
  attention  weighted sparse attention, dense attention, and the two HT sums

Parity pins: every function here is pinned by at least one CPU test
(``tests/test_oracle_*.py``); the one that is only self-consistent is noted in
``philox`` (its canonical conformance is pinned by a cross-check against
rocRAND's host-callable Philox4x32-10).
"""

from .philox import philox4x32_10, philox4x32_10_np, block_offset
from .scoring import apply_perm, unpermute, valid_counts, block_means, score
from .ibcs import fixed_point, cluster_block, lloyd_block, certified_agreement, group_mixture, score_ibcs
from .stats_score import block_variances, score_stats
from .selection import (sanitize, exact_set, quantise, water_fill, fixed_point_pi,
                        systematic_sample, inverse_weight, select_row, select, F_BITS, FS_BITS)
from .attention import (attend, attend_block, attend_dense, dense_block, dense_row_max,
                        unit_sums, weighted_sums)

__all__ = [
    "philox4x32_10", "philox4x32_10_np", "block_offset",
    "apply_perm", "unpermute", "valid_counts", "block_means", "score",
    "fixed_point", "cluster_block", "lloyd_block", "certified_agreement", "group_mixture", "score_ibcs", "block_variances", "score_stats",
    "sanitize", "exact_set", "quantise", "water_fill", "fixed_point_pi",
    "systematic_sample", "inverse_weight", "select_row", "select", "F_BITS", "FS_BITS",
    "attend", "attend_block", "attend_dense", "dense_block", "dense_row_max",
    "unit_sums", "weighted_sums",
]
