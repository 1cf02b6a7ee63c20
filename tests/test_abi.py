"""The C ABI without a GPU: exported symbols, struct layout, host-side validation.

Every rejected call returns before any HIP call, so these run on a machine
without a GPU (the library loads; nothing is launched).
"""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

import block_sparse_attention_27_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.library_path()):
        pytest.fail("libbsa.so is not built (run __graft_entry__.build())")
    return bsa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^(?:bsa_status|int32_t|const char\*)\s+(bsa_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_pipeline():
    names = _declared_functions()
    for n in ("bsa_score", "bsa_score_ibcs", "bsa_score_stats", "bsa_select", "bsa_permute_rows", "bsa_attend",
              "bsa_attend_dense", "bsa_status_string", "bsa_abi_version", "bsa_mfma_ceiling", "bsa_mfma_ceiling_random"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    nm = shutil.which("nm") or "nm"
    out = subprocess.run([nm, "-D", "--defined-only", bsa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_abi_version_and_status_strings(lib):
    assert lib.bsa_abi_version() == 7
    assert lib.bsa_status_string(0) == b"ok"
    assert lib.bsa_status_string(1) == b"invalid argument"
    assert lib.bsa_status_string(99) == b"unknown status"


def test_problem_struct_layout_matches_header(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "bsa.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(bsa_problem),'
                   ' offsetof(bsa_problem, dtype), offsetof(bsa_problem, seed),'
                   ' offsetof(bsa_problem, sm_scale), offsetof(bsa_problem, kv_permuted),'
                   ' offsetof(bsa_problem, out_fp32)); return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    c_vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    P = bsa.Problem
    assert c_vals == [ctypes.sizeof(P), P.dtype.offset, P.seed.offset, P.sm_scale.offset, P.kv_permuted.offset,
                      P.out_fp32.offset]


def _good(**kw):
    f = dict(B=1, H=2, N=1000, N_pad=1024, d=128, block_q=128, block_k=64, k_exact=2, m_sample=3,
             dtype=bsa.BSA_BF16, out_fp32=0, seed=1, sm_scale=1.0, kv_permuted=0)
    f.update(kw)
    return bsa.Problem(**f)


BAD = [
    dict(B=0), dict(H=0), dict(N=0), dict(N=2000), dict(d=96), dict(block_q=32), dict(block_k=16),
    dict(N_pad=1000), dict(dtype=7), dict(sm_scale=0.0), dict(sm_scale=float("inf")),
    dict(sm_scale=float("nan")), dict(kv_permuted=2), dict(kv_permuted=-1), dict(N_pad=1 << 29, N=1 << 29),
    dict(out_fp32=2),
]
BAD_BUDGET = [dict(k_exact=-1), dict(m_sample=-1), dict(k_exact=0, m_sample=0),
              dict(k_exact=10, m_sample=7)]  # 16 valid units of 64 keys in N = 1000


FAKE = ctypes.c_void_p(0x7F0000000000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("bad", BAD)
def test_invalid_problem_rejected_by_every_call(lib, bad):
    p = ctypes.byref(_good(**bad))
    assert lib.bsa_score(p, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_score_ibcs(p, 4, 3, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_score_stats(p, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_select(p, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_attend(p, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_attend_dense(p, FAKE, FAKE, FAKE, None, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_permute_rows(p, FAKE, FAKE, ctypes.c_void_p(0x7E0000000000), None) == bsa.BSA_ERR_INVALID_ARG


def test_kv_permuted_needs_a_permutation(lib):
    p = ctypes.byref(_good(kv_permuted=1))
    assert lib.bsa_score(p, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_score_ibcs(p, 4, 3, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_score_stats(p, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_attend(p, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_attend_dense(p, FAKE, FAKE, FAKE, None, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG


def test_permute_rows_argument_checks(lib):
    p = ctypes.byref(_good())
    other = ctypes.c_void_p(0x7E0000000000)
    bytes_ = 1 * 2 * 1024 * 128 * 2
    # null pointers, missing permutation, misalignment
    assert lib.bsa_permute_rows(p, None, FAKE, other, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_permute_rows(p, FAKE, None, other, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_permute_rows(p, FAKE, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_permute_rows(p, ctypes.c_void_p(0x7F0000000008), FAKE, other, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_permute_rows(p, FAKE, ctypes.c_void_p(0x7F0000000002), other, None) == bsa.BSA_ERR_INVALID_ARG
    # in place and overlapping buffers
    assert lib.bsa_permute_rows(p, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_permute_rows(p, FAKE, FAKE, ctypes.c_void_p(0x7F0000000000 + bytes_ - 16),
                                None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_permute_rows(p, FAKE, FAKE, ctypes.c_void_p(0x7F0000000000 - bytes_ + 16),
                                None) == bsa.BSA_ERR_INVALID_ARG


@pytest.mark.parametrize("groups,iters", [(0, 3), (3, 3), (16, 3), (-1, 3), (4, 0), (4, 17), (4, -2)])
def test_ibcs_groups_and_iterations_checked(lib, groups, iters):
    p = ctypes.byref(_good())
    assert lib.bsa_score_ibcs(p, groups, iters, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                              None) == bsa.BSA_ERR_INVALID_ARG


def test_stats_null_and_misaligned_outputs_rejected(lib):
    p = ctypes.byref(_good())
    odd = ctypes.c_void_p(0x7F0000000008)
    for args in ((None, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE), (FAKE, FAKE, None, FAKE),
                 (FAKE, FAKE, FAKE, None), (FAKE, FAKE, FAKE, odd), (FAKE, odd, FAKE, FAKE)):
        assert lib.bsa_score_stats(p, FAKE, FAKE, None, *args, None) == bsa.BSA_ERR_INVALID_ARG


def test_ibcs_null_and_misaligned_outputs_rejected(lib):
    p = ctypes.byref(_good())
    bad4 = ctypes.c_void_p(0x7F0000000002)
    odd = ctypes.c_void_p(0x7F0000000008)
    for args in ((None, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE), (FAKE, FAKE, None, FAKE),
                 (FAKE, FAKE, FAKE, None), (FAKE, odd, FAKE, FAKE), (FAKE, FAKE, bad4, FAKE),
                 (FAKE, FAKE, FAKE, odd)):
        assert lib.bsa_score_ibcs(p, 4, 3, FAKE, FAKE, None, *args, None) == bsa.BSA_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", BAD_BUDGET)
def test_invalid_budget_rejected(lib, bad):
    p = ctypes.byref(_good(**bad))
    assert lib.bsa_select(p, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_attend(p, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG


def test_null_and_misaligned_pointers_rejected(lib):
    p = ctypes.byref(_good())
    assert lib.bsa_score(None, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_score(p, None, FAKE, None, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_select(p, FAKE, None, FAKE, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_attend(p, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_attend_dense(p, FAKE, FAKE, None, None, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG
    odd = ctypes.c_void_p(0x7F0000000008)  # 8-byte aligned, not 16
    assert lib.bsa_attend(p, odd, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == bsa.BSA_ERR_INVALID_ARG
    bad4 = ctypes.c_void_p(0x7F0000000002)
    assert lib.bsa_select(p, FAKE, bad4, FAKE, None) == bsa.BSA_ERR_INVALID_ARG


def test_selection_unit_limit_is_unsupported(lib):
    # 5000 valid units of 32 keys exceed the fixed-point sampler's 4096-unit range
    p = ctypes.byref(_good(N=160000, N_pad=160000, block_k=32, block_q=128))
    assert lib.bsa_select(p, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_UNSUPPORTED


def test_scoring_key_unit_limit_is_unsupported(lib):
    # 2^22 units of 32 keys at d = 128: one head's key means span 2^31 bytes,
    # one more than the kernels' 32-bit range; at d = 64 the same shape passes
    # this check (and would launch, so it is not called here)
    p = ctypes.byref(_good(N=1 << 27, N_pad=1 << 27, block_k=32, block_q=128, H=1))
    assert lib.bsa_score(p, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_UNSUPPORTED
    assert lib.bsa_score_ibcs(p, 4, 3, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_UNSUPPORTED
    assert lib.bsa_score_stats(p, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == bsa.BSA_ERR_UNSUPPORTED


def test_mfma_ceiling_arguments_checked(lib):
    assert lib.bsa_mfma_ceiling(None, 10, 4, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_mfma_ceiling(ctypes.c_void_p(0x7F0000000002), 10, 4, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_mfma_ceiling(FAKE, 0, 4, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_mfma_ceiling(FAKE, 10, 0, None) == bsa.BSA_ERR_INVALID_ARG
    assert lib.bsa_mfma_ceiling(FAKE, -3, -1, None) == bsa.BSA_ERR_INVALID_ARG
    f = lib.bsa_mfma_ceiling_random
    assert f(None, 8, 4, None) == bsa.BSA_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(0x7F0000000002), 8, 4, None) == bsa.BSA_ERR_INVALID_ARG
    for iters in (0, 1, 2, 3, 6, -4):  # rounds come in fours
        assert f(FAKE, iters, 4, None) == bsa.BSA_ERR_INVALID_ARG
    assert f(FAKE, 8, 0, None) == bsa.BSA_ERR_INVALID_ARG
    assert f(FAKE, 8, (1 << 18) + 1, None) == bsa.BSA_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("BSA_LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(bsa, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        bsa.load_library()
