"""Weighted dynamic block-sparse attention for video DiTs on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libbsa.so`` (declared in
``include/bsa.h``). It only marshals torch tensors to device pointers and the
current HIP stream; every step runs in the library's HIP kernels. There is no
CPU fallback: if the library is missing, every call raises.

Mirrors of the C entry points (same names and argument order, outputs passed
in by the caller):
    bsa_score(problem, q, k, perm, S, q_mean, k_mean)
    bsa_score_ibcs(problem, groups, iters, q, k, perm, S, q_cent, q_size, k_mean)
    bsa_score_stats(problem, q, k, perm, S, q_mean, k_mean, k_var)
    bsa_select(problem, S, idx, w)
    bsa_permute_rows(problem, x, perm, x_perm)
    bsa_attend(problem, q, k, v, perm, idx, w, out, lse)
    bsa_attend_dense(problem, q, k, v, perm, out, lse)
Convenience wrappers that allocate their outputs: score, score_ibcs, score_stats, select,
permute_rows, attend, attend_dense, sparse_attention (the three steps in order; with a
permutation it first puts K and V into the permuted order and runs the steps with
kv_permuted = 1), and SamplingPlan, which keeps one score + select result for reuse by
later attend calls.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

from .inputs import Workload

__all__ = [
    "Problem", "BsaError", "load_library", "library_path", "problem_for", "out_dtype",
    "bsa_score", "bsa_score_ibcs", "bsa_score_stats", "bsa_select", "bsa_permute_rows", "bsa_attend",
    "bsa_attend_dense", "score", "score_ibcs", "score_stats", "select", "permute_rows", "with_kv_permuted",
    "attend", "attend_dense", "sparse_attention", "SamplingPlan", "bsa_mfma_ceiling", "bsa_mfma_ceiling_random", "MFMA_CEILING_FLOP",
    "BSA_OK", "BSA_ERR_INVALID_ARG", "BSA_ERR_UNSUPPORTED", "BSA_ERR_HIP", "BSA_BF16", "BSA_FP32",
]

BSA_OK, BSA_ERR_INVALID_ARG, BSA_ERR_UNSUPPORTED, BSA_ERR_HIP = 0, 1, 2, 3
BSA_BF16, BSA_FP32 = 0, 1

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("BSA_LIBRARY", os.path.join(_PKG, "libbsa.so"))


class Problem(ctypes.Structure):
    """ctypes mirror of ``bsa_problem``."""

    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("N_pad", ctypes.c_int32), ("d", ctypes.c_int32), ("block_q", ctypes.c_int32),
        ("block_k", ctypes.c_int32), ("k_exact", ctypes.c_int32), ("m_sample", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("out_fp32", ctypes.c_int32), ("kv_permuted", ctypes.c_int32),
        ("seed", ctypes.c_uint64), ("sm_scale", ctypes.c_float),
    ]

    @property
    def nQB(self) -> int:
        return self.N_pad // self.block_q

    @property
    def nKU(self) -> int:
        return self.N_pad // self.block_k

    @property
    def L(self) -> int:
        return self.k_exact + self.m_sample


class BsaError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed: {_status_text(status)} (status {status})")


_lib = None


def load_library():
    """Load libbsa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libbsa.so not found at {path}: build it first "
                           "(python -m block_sparse_attention_27_amd.build)")
    lib = ctypes.CDLL(path)
    vp, P = ctypes.c_void_p, ctypes.POINTER(Problem)
    lib.bsa_abi_version.restype = ctypes.c_int32
    lib.bsa_abi_version.argtypes = []
    lib.bsa_status_string.restype = ctypes.c_char_p
    lib.bsa_status_string.argtypes = [ctypes.c_int32]
    lib.bsa_score.restype = ctypes.c_int
    lib.bsa_score.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.bsa_score_ibcs.restype = ctypes.c_int
    lib.bsa_score_ibcs.argtypes = [P, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bsa_score_stats.restype = ctypes.c_int
    lib.bsa_score_stats.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bsa_select.restype = ctypes.c_int
    lib.bsa_select.argtypes = [P, vp, vp, vp, vp]
    lib.bsa_permute_rows.restype = ctypes.c_int
    lib.bsa_permute_rows.argtypes = [P, vp, vp, vp, vp]
    lib.bsa_attend.restype = ctypes.c_int
    lib.bsa_attend.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bsa_attend_dense.restype = ctypes.c_int
    lib.bsa_attend_dense.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.bsa_mfma_ceiling.restype = ctypes.c_int
    lib.bsa_mfma_ceiling.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
    lib.bsa_mfma_ceiling_random.restype = ctypes.c_int
    lib.bsa_mfma_ceiling_random.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp]
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().bsa_status_string(status).decode()
    except Exception:  # the library itself may be what is missing
        return "status"


def problem_for(w: Workload, seed: Optional[int] = None, **overrides) -> Problem:
    """A bsa_problem for a workload preset (overrides replace any field)."""
    f = dict(B=w.B, H=w.H, N=w.N, N_pad=w.N_pad, d=w.d, block_q=w.block_q, block_k=w.block_k,
             k_exact=w.k_exact, m_sample=w.m_sample,
             dtype=BSA_BF16 if w.dtype == "bf16" else BSA_FP32,
             out_fp32=0, seed=w.select_seed if seed is None else seed, sm_scale=w.sm_scale, kv_permuted=0)
    f.update(overrides)
    return Problem(**f)


# ---------------------------------------------------------------- marshalling

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(call: str, status: int):
    if status != BSA_OK:
        raise BsaError(call, status)


def _elem_dtype(p: Problem):
    import torch
    return torch.bfloat16 if p.dtype == BSA_BF16 else torch.float32


def out_dtype(p: Problem):
    """Element type of the attention output for this problem."""
    import torch
    return torch.bfloat16 if (p.dtype == BSA_BF16 and not p.out_fp32) else torch.float32


def _expect(name, t, shape, dtype):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def bsa_score(p: Problem, q, k, perm, S, q_mean, k_mean, stream=None):
    import torch
    et = _elem_dtype(p)
    qkv_shape = (p.B, p.H, p.N_pad, p.d)
    _expect("q", q, qkv_shape, et); _expect("k", k, qkv_shape, et)
    _expect("perm", perm, (p.N_pad,), torch.int32)
    _expect("S", S, (p.B, p.H, p.nQB, p.nKU), torch.float32)
    _expect("q_mean", q_mean, (p.B, p.H, p.nQB, p.d), torch.float32)
    _expect("k_mean", k_mean, (p.B, p.H, p.nKU, p.d), torch.float32)
    _check("bsa_score", load_library().bsa_score(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(perm), _ptr(S),
                                                 _ptr(q_mean), _ptr(k_mean), _stream(stream)))


def bsa_score_ibcs(p: Problem, groups: int, iters: int, q, k, perm, S, q_cent, q_size, k_mean, stream=None):
    import torch
    et = _elem_dtype(p)
    _expect("q", q, (p.B, p.H, p.N_pad, p.d), et)
    _expect("k", k, (p.B, p.H, p.N_pad, p.d), et)
    _expect("perm", perm, (p.N_pad,), torch.int32)
    _expect("S", S, (p.B, p.H, p.nQB, p.nKU), torch.float32)
    _expect("q_cent", q_cent, (p.B, p.H, p.nQB, groups, p.d), torch.float32)
    _expect("q_size", q_size, (p.B, p.H, p.nQB, groups), torch.int32)
    _expect("k_mean", k_mean, (p.B, p.H, p.nKU, p.d), torch.float32)
    _check("bsa_score_ibcs", load_library().bsa_score_ibcs(ctypes.byref(p), groups, iters, _ptr(q), _ptr(k),
                                                           _ptr(perm), _ptr(S), _ptr(q_cent), _ptr(q_size),
                                                           _ptr(k_mean), _stream(stream)))


def bsa_score_stats(p: Problem, q, k, perm, S, q_mean, k_mean, k_var, stream=None):
    import torch
    et = _elem_dtype(p)
    _expect("q", q, (p.B, p.H, p.N_pad, p.d), et)
    _expect("k", k, (p.B, p.H, p.N_pad, p.d), et)
    _expect("perm", perm, (p.N_pad,), torch.int32)
    _expect("S", S, (p.B, p.H, p.nQB, p.nKU), torch.float32)
    _expect("q_mean", q_mean, (p.B, p.H, p.nQB, p.d), torch.float32)
    _expect("k_mean", k_mean, (p.B, p.H, p.nKU, p.d), torch.float32)
    _expect("k_var", k_var, (p.B, p.H, p.nKU, p.d), torch.float32)
    _check("bsa_score_stats", load_library().bsa_score_stats(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(perm), _ptr(S),
                                                             _ptr(q_mean), _ptr(k_mean), _ptr(k_var),
                                                             _stream(stream)))


def bsa_select(p: Problem, S, idx, w, stream=None):
    import torch
    _expect("S", S, (p.B, p.H, p.nQB, p.nKU), torch.float32)
    _expect("idx", idx, (p.B, p.H, p.nQB, p.L), torch.int32)
    _expect("w", w, (p.B, p.H, p.nQB, p.L), torch.float32)
    _check("bsa_select", load_library().bsa_select(ctypes.byref(p), _ptr(S), _ptr(idx), _ptr(w),
                                                   _stream(stream)))


def bsa_permute_rows(p: Problem, x, perm, x_perm, stream=None):
    import torch
    et = _elem_dtype(p)
    _expect("x", x, (p.B, p.H, p.N_pad, p.d), et)
    _expect("perm", perm, (p.N_pad,), torch.int32)
    _expect("x_perm", x_perm, (p.B, p.H, p.N_pad, p.d), et)
    _check("bsa_permute_rows", load_library().bsa_permute_rows(ctypes.byref(p), _ptr(x), _ptr(perm), _ptr(x_perm),
                                                               _stream(stream)))


# floating-point operations of one wave-round of bsa_mfma_ceiling: 8 MFMAs of 32 x 32 x 16 multiply-adds
MFMA_CEILING_FLOP = 8 * 2 * 32 * 32 * 16


def bsa_mfma_ceiling(out, iters: int, n_wg: int, stream=None):
    """Measurement aid: n_wg workgroups of 4 waves, each wave `iters` rounds of 8 register-only MFMAs."""
    import torch
    _expect("out", out, (n_wg * 256,), torch.float32)
    _check("bsa_mfma_ceiling", load_library().bsa_mfma_ceiling(_ptr(out), iters, n_wg, _stream(stream)))


def bsa_mfma_ceiling_random(out, iters: int, n_wg: int, stream=None):
    """Measurement aid: as bsa_mfma_ceiling, with operands that change from one MFMA to the next."""
    import torch
    _expect("out", out, (n_wg * 256,), torch.float32)
    _check("bsa_mfma_ceiling_random",
           load_library().bsa_mfma_ceiling_random(_ptr(out), iters, n_wg, _stream(stream)))


def bsa_attend(p: Problem, q, k, v, perm, idx, w, out, lse=None, stream=None):
    import torch
    et = _elem_dtype(p)
    qkv_shape = (p.B, p.H, p.N_pad, p.d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(name, t, qkv_shape, et)
    _expect("out", out, qkv_shape, out_dtype(p))
    _expect("perm", perm, (p.N_pad,), torch.int32)
    _expect("idx", idx, (p.B, p.H, p.nQB, p.L), torch.int32)
    _expect("w", w, (p.B, p.H, p.nQB, p.L), torch.float32)
    _expect("lse", lse, (p.B, p.H, p.N_pad), torch.float32)
    _check("bsa_attend", load_library().bsa_attend(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(perm),
                                                   _ptr(idx), _ptr(w), _ptr(out), _ptr(lse),
                                                   _stream(stream)))


def bsa_attend_dense(p: Problem, q, k, v, perm, out, lse=None, stream=None):
    import torch
    et = _elem_dtype(p)
    qkv_shape = (p.B, p.H, p.N_pad, p.d)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(name, t, qkv_shape, et)
    _expect("out", out, qkv_shape, out_dtype(p))
    _expect("perm", perm, (p.N_pad,), torch.int32)
    _expect("lse", lse, (p.B, p.H, p.N_pad), torch.float32)
    _check("bsa_attend_dense", load_library().bsa_attend_dense(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                                               _ptr(perm), _ptr(out), _ptr(lse),
                                                               _stream(stream)))


# ---------------------------------------------------------------- convenience

def score(p: Problem, q, k, perm=None, stream=None):
    """Returns (S, q_mean, k_mean)."""
    import torch
    dev = q.device
    S = torch.empty((p.B, p.H, p.nQB, p.nKU), dtype=torch.float32, device=dev)
    qm = torch.empty((p.B, p.H, p.nQB, p.d), dtype=torch.float32, device=dev)
    km = torch.empty((p.B, p.H, p.nKU, p.d), dtype=torch.float32, device=dev)
    bsa_score(p, q, k, perm, S, qm, km, stream)
    return S, qm, km


def score_ibcs(p: Problem, q, k, perm=None, groups: int = 4, iters: int = 3, stream=None):
    """Returns (S, q_cent, q_size, k_mean)."""
    import torch
    dev = q.device
    S = torch.empty((p.B, p.H, p.nQB, p.nKU), dtype=torch.float32, device=dev)
    qc = torch.empty((p.B, p.H, p.nQB, groups, p.d), dtype=torch.float32, device=dev)
    qs = torch.empty((p.B, p.H, p.nQB, groups), dtype=torch.int32, device=dev)
    km = torch.empty((p.B, p.H, p.nKU, p.d), dtype=torch.float32, device=dev)
    bsa_score_ibcs(p, groups, iters, q, k, perm, S, qc, qs, km, stream)
    return S, qc, qs, km


def score_stats(p: Problem, q, k, perm=None, stream=None):
    """Returns (S, q_mean, k_mean, k_var)."""
    import torch
    dev = q.device
    S = torch.empty((p.B, p.H, p.nQB, p.nKU), dtype=torch.float32, device=dev)
    qm = torch.empty((p.B, p.H, p.nQB, p.d), dtype=torch.float32, device=dev)
    km = torch.empty((p.B, p.H, p.nKU, p.d), dtype=torch.float32, device=dev)
    kv = torch.empty((p.B, p.H, p.nKU, p.d), dtype=torch.float32, device=dev)
    bsa_score_stats(p, q, k, perm, S, qm, km, kv, stream)
    return S, qm, km, kv


def select(p: Problem, S, stream=None):
    """Returns (idx, w)."""
    import torch
    idx = torch.empty((p.B, p.H, p.nQB, p.L), dtype=torch.int32, device=S.device)
    w = torch.empty((p.B, p.H, p.nQB, p.L), dtype=torch.float32, device=S.device)
    bsa_select(p, S, idx, w, stream)
    return idx, w


def permute_rows(p: Problem, x, perm, stream=None):
    """x_perm with x_perm[b, h, r] = x[b, h, perm[r]] for r < N (zero rows past N)."""
    import torch
    x_perm = torch.empty_like(x)
    bsa_permute_rows(p, x, perm, x_perm, stream)
    return x_perm


def with_kv_permuted(p: Problem, flag: int = 1) -> Problem:
    """A copy of ``p`` with kv_permuted set (K and V passed as K[perm], V[perm])."""
    q = Problem.from_buffer_copy(p)
    q.kv_permuted = flag
    return q


def attend(p: Problem, q, k, v, idx, w, perm=None, with_lse=False, stream=None):
    """Returns out (and lse when ``with_lse``)."""
    import torch
    out = torch.empty(q.shape, dtype=out_dtype(p), device=q.device)
    lse = torch.empty((p.B, p.H, p.N_pad), dtype=torch.float32, device=q.device) if with_lse else None
    bsa_attend(p, q, k, v, perm, idx, w, out, lse, stream)
    return (out, lse) if with_lse else out


def attend_dense(p: Problem, q, k, v, perm=None, with_lse=False, stream=None):
    import torch
    out = torch.empty(q.shape, dtype=out_dtype(p), device=q.device)
    lse = torch.empty((p.B, p.H, p.N_pad), dtype=torch.float32, device=q.device) if with_lse else None
    bsa_attend_dense(p, q, k, v, perm, out, lse, stream)
    return (out, lse) if with_lse else out


def sparse_attention(p: Problem, q, k, v, perm=None, with_lse=False, stream=None):
    """score -> select -> attend on one stream; returns (out[, lse], idx, w).

    With a permutation (and K, V in token order, p.kv_permuted == 0) K and V are
    first gathered into the permuted order, so that the attention pass reads
    every key unit as contiguous rows; the results are those of the
    permutation applied inside each call.
    """
    if perm is not None and not p.kv_permuted:
        k, v = permute_rows(p, k, perm, stream), permute_rows(p, v, perm, stream)
        p = with_kv_permuted(p)
    S, _, _ = score(p, q, k, perm, stream)
    idx, w = select(p, S, stream)
    res = attend(p, q, k, v, idx, w, perm, with_lse, stream)
    return (res if isinstance(res, tuple) else (res,)) + (idx, w)


class SamplingPlan:
    """One query-block sampling plan (idx, w), built once and reused.

    AB-Attention (podcast transcript, the passage on reuse across nearby
    denoising steps): the plan -- which key blocks each query block reads and
    with what weight -- may be kept over nearby steps to save the selection
    work, while attention itself is recomputed from each step's activations.
    ``attend`` therefore runs only ``bsa_attend`` on the caller's current Q, K
    and V with the stored lists; ``refresh`` rebuilds the plan (score, then
    select) from new activations. The geometry (problem) is fixed per plan.
    """

    def __init__(self, p: Problem, q, k, perm=None, stream=None):
        self.p = p
        self.idx = None
        self.w = None
        self.refresh(q, k, perm, stream)

    def refresh(self, q, k, perm=None, stream=None):
        S, _, _ = score(self.p, q, k, perm, stream)
        self.idx, self.w = select(self.p, S, stream)
        return self

    def attend(self, q, k, v, perm=None, with_lse=False, stream=None):
        return attend(self.p, q, k, v, self.idx, self.w, perm, with_lse, stream)
