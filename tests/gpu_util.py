"""Helpers for the GPU tests: moving generated inputs to the device and back."""

import numpy as np
import torch

from block_sparse_attention_27_amd.inputs import f32_from_bf16_bits


def to_device(arr: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 tensor; float32 -> float32 tensor (on cuda:0)."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> fp64 numpy (bf16 widened exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return f32_from_bf16_bits(t.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return t.numpy().astype(np.float64)


def host_f64(arr: np.ndarray) -> np.ndarray:
    if arr.dtype == np.uint16:
        return f32_from_bf16_bits(arr).astype(np.float64)
    return arr.astype(np.float64)


def rel_l2(a, b) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def print_case(*parts):
    print("[case]", *parts, flush=True)
