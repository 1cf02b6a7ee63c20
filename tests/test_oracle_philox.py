"""Pins for the oracle's Philox4x32-10 (CPU only).

Canonical conformance: the oracle is compared with rocRAND's Philox4x32-10
engine (a library routine, compiled here for the host) on many counters and
keys. The vectorised form is compared with the scalar one.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox4x32_10, philox4x32_10_np, block_offset

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    cxx = shutil.which("amdclang++") or "/opt/rocm/llvm/bin/amdclang++"
    if not os.path.exists(cxx) and shutil.which(cxx) is None:
        pytest.skip("no ROCm host compiler for the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("philox") / "ref")
    src = os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp")
    subprocess.run([cxx, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-O1",
                    src, "-o", exe], check=True, capture_output=True)

    def run(cases):
        text = "".join(f"{s} {b} {h} {i}\n" for s, b, h, i in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [tuple(int(x) for x in line.split()) for line in out.strip().splitlines()]

    return run


def test_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(123)
    cases = [(0, 0, 0, 0), (2**64 - 1, 7, 39, 590), (0xDEADBEEFCAFEF00D, 0, 23, 928),
             (1, 0, 0, 1), (2**32, 0, 1, 0)]
    for _ in range(300):
        cases.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                      int(rng.integers(0, 4)), int(rng.integers(0, 64)), int(rng.integers(0, 4096))))
    ref = rocrand_ref(cases)
    assert len(ref) == len(cases)
    for (s, b, h, i), r in zip(cases, ref):
        key = (s & 0xFFFFFFFF, s >> 32)
        assert philox4x32_10((i, h, b, 0), key) == r, (s, b, h, i)
        assert block_offset(s, b, h, i) == r[0]


def test_vectorised_matches_scalar():
    rng = np.random.default_rng(7)
    c = rng.integers(0, 2**32, size=(4, 200), dtype=np.uint64)
    k = rng.integers(0, 2**32, size=(2, 200), dtype=np.uint64)
    vec = philox4x32_10_np(c[0], c[1], c[2], c[3], k[0], k[1])
    for n in range(200):
        ref = philox4x32_10([int(x) for x in c[:, n]], [int(x) for x in k[:, n]])
        assert tuple(int(v[n]) for v in vec) == ref


def test_counter_words_are_distinct_streams():
    # changing any one of (i, h, b) or the seed changes the draw
    base = block_offset(5, 0, 0, 0)
    assert len({base, block_offset(6, 0, 0, 0), block_offset(5, 1, 0, 0),
                block_offset(5, 0, 1, 0), block_offset(5, 0, 0, 1)}) == 5
