"""Philox4x32-10 counter-based generator, written from its published definition.

Test infrastructure: part of the CPU oracle (see ``oracle/__init__.py``).

Definition (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11): a 4x32-bit counter is passed through 10 rounds keyed by a
2x32-bit key. One round multiplies counter words 0 and 2 by two fixed odd
constants, keeps the high and low 32-bit halves of each 64-bit product, and
recombines them as (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0). Between rounds
the key is advanced by two Weyl constants (the golden ratio and sqrt(3) - 1,
scaled to 32 bits).

Use in the method: one uniform 32-bit offset per (b, h, query block), the
counter being (query block, head, batch, 0) and the key the 64-bit seed split
into its low and high words. One draw per query block makes the sample shared
by every query of that block (InstaGen, Abstract: each query cluster draws one
sample for all its queries).
"""

from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85


def philox4x32_10(counter, key):
    """Ten Philox4x32 rounds on one counter; returns four Python ints."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """Same rounds, elementwise over numpy arrays (uint64 holding 32-bit words)."""
    m = np.uint64(MASK32)
    c = [np.asarray(x, dtype=np.uint64) & m for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & m
    k1 = np.asarray(k1, dtype=np.uint64) & m
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W0)) & m
            k1 = (k1 + np.uint64(PHILOX_W1)) & m
        p0 = np.uint64(PHILOX_M0) * c[0]
        p1 = np.uint64(PHILOX_M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return tuple(x.astype(np.uint32) for x in c)


def block_offset(seed: int, b: int, h: int, i: int) -> int:
    """The uniform offset u in [0, 2^32) drawn for query block i of head h, batch b."""
    key = (seed & MASK32, (seed >> 32) & MASK32)
    return philox4x32_10((i, h, b, 0), key)[0]
