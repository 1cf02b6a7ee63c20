"""Seeded synthetic workloads: clustered video-DiT attention layers.

This module only makes inputs. It holds none of the attention method's
arithmetic, so both the HIP path and the CPU oracle can be fed from it without
sharing any of the method's code.

Workloads
---------
The pages measure on trained video models (Wan2.1, HunyuanVideo) over prompt
benchmarks; none of that is available here, so every input is synthetic with
the layer shapes those models use:

* tokens sit on a (T, Hs, W) latent grid in row-major (t, y, x) order and are
  zero-padded from N to N_pad rows;
* every token belongs to one of C spatially coherent clusters: C seed points
  are drawn uniformly in the unit box and each token joins the nearest one,
  measured at its cell centre ((t+.5)/T, (y+.5)/Hs, (x+.5)/W), ties to the
  lower cluster id;
* per (b, h) a centroid mu_c ~ N(0, 2^2 I_d) is drawn for every cluster;
  Q = (mu_c + e_q)/sqrt(d) and K = (mu_c + e_k)/sqrt(d) with independent
  e ~ N(0, 0.5^2 I_d); V ~ N(0, 1) (value_mode "noise", every preset), or
  V = nu_c + e_v with a per-cluster value nu_c ~ N(0, I_d) and
  e_v ~ N(0, 0.5^2 I_d) (value_mode "clustered": values that follow the
  clusters, so that dense attention outputs are far from zero);
* key_spread "uniform" (every preset) gives every key the noise std above;
  key_spread "clustered" gives the keys of cluster c their own noise std
  noise_std * 2^u_c with u_c ~ U(0, 3) (0.5 to 4 at the default), so key
  units differ in their within-unit spread and not only in their means (Q, V
  and the centroids are the same draws as with "uniform");
* the logit scale is sm_scale = 1/temperature;
* bf16 workloads are drawn in fp32 and rounded to nearest-even bf16;
* the HunyuanVideo-shaped workload also carries a gather index that groups
  tokens of one cluster together (a semantic permutation of the kind permuted
  block-sparse attention uses: InstaGen, Abstract).

Random streams: one numpy PCG64 stream seeded with ``[seed]`` draws the
cluster seed points and the cluster relabelling; each (b, h) draws its
centroids and noise from its own stream seeded with ``[seed, 1, b, h]``, so any
head can be made alone; clustered values draw nu_c from ``[seed, 2, b, h]``,
clustered key spreads draw u_c from ``[seed, 3, b, h]``.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Iterable, Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "generate",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "cluster_ids",
    "as_float32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer shape plus the generator's knobs."""

    name: str
    B: int
    H: int
    grid: tuple  # (T, Hs, W)
    d: int
    dtype: str  # "fp32" or "bf16"
    block_q: int
    block_k: int
    k_exact: int
    m_sample: int
    clusters: int
    temperature: float
    permute: bool = False
    noise_std: float = 0.5
    centroid_std: float = 2.0
    seed: int = 0
    select_seed: int = 0
    value_mode: str = "noise"  # "noise" or "clustered"
    key_spread: str = "uniform"  # "uniform" or "clustered"

    @property
    def N(self) -> int:
        T, Hs, W = self.grid
        return T * Hs * W

    @property
    def N_pad(self) -> int:
        step = max(self.block_q, self.block_k)
        return -(-self.N // step) * step

    @property
    def n_qblocks(self) -> int:
        return self.N_pad // self.block_q

    @property
    def n_units(self) -> int:
        return self.N_pad // self.block_k

    @property
    def n_valid_units(self) -> int:
        return -(-self.N // self.block_k)

    @property
    def list_len(self) -> int:
        return self.k_exact + self.m_sample

    @property
    def sm_scale(self) -> float:
        return 1.0 / self.temperature

    @property
    def density(self) -> float:
        """Fraction of valid key units each query block computes."""
        return self.list_len / self.n_valid_units

    def executed_flops(self) -> float:
        """QK^T plus PV multiply-adds over every issued query row and listed key."""
        return 4.0 * self.d * self.B * self.H * self.n_qblocks * self.block_q * self.list_len * self.block_k

    def dense_flops(self) -> float:
        """Dense-equivalent work on the N valid tokens."""
        return 4.0 * self.N * self.N * self.d * self.B * self.H

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Small case the fp64 oracle finishes in seconds.
    "tiny": Workload("tiny", B=1, H=1, grid=(4, 16, 16), d=64, dtype="fp32",
                     block_q=64, block_k=64, k_exact=2, m_sample=2,
                     clusters=8, temperature=1.0, noise_std=0.5),
    # Wan2.1-T2V-1.3B-shaped layer, 25% density.
    "wan13b": Workload("wan13b", B=1, H=12, grid=(21, 30, 52), d=128, dtype="bf16",
                       block_q=128, block_k=128, k_exact=16, m_sample=48,
                       clusters=64, temperature=1.0),
    # Wan2.1-T2V-14B at 480p, ~10% density (temperature swept 0.5 / 1 / 2).
    "wan14b_480p": Workload("wan14b_480p", B=1, H=40, grid=(21, 30, 52), d=128, dtype="bf16",
                            block_q=128, block_k=128, k_exact=8, m_sample=18,
                            clusters=64, temperature=1.0),
    # Wan2.1-T2V-14B at 720p, ~10% density: the headline layer.
    "wan14b_720p": Workload("wan14b_720p", B=1, H=40, grid=(21, 45, 80), d=128, dtype="bf16",
                            block_q=128, block_k=128, k_exact=20, m_sample=40,
                            clusters=128, temperature=1.0),
    # HunyuanVideo-13B-shaped layer: 32-key units, 4 per 128-key tile, permuted tokens.
    "hunyuan": Workload("hunyuan", B=1, H=24, grid=(33, 45, 80), d=128, dtype="bf16",
                        block_q=128, block_k=32, k_exact=96, m_sample=200,
                        clusters=128, temperature=1.0, permute=True),
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns the uint16 bit patterns.

    The 32-bit sum cannot wrap: the largest finite pattern plus 0x8000 stays below 2^32.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cluster_ids(w: Workload) -> np.ndarray:
    """Cluster id of every valid token (int64[N]), nearest seed point in the unit box."""
    rng = np.random.default_rng([w.seed])
    pts = rng.random((w.clusters, 3))
    T, Hs, W = w.grid
    t = (np.arange(T) + 0.5) / T
    y = (np.arange(Hs) + 0.5) / Hs
    x = (np.arange(W) + 0.5) / W
    coords = np.stack(np.meshgrid(t, y, x, indexing="ij"), axis=-1).reshape(-1, 3)
    out = np.empty(coords.shape[0], dtype=np.int64)
    step = 8192
    for s in range(0, coords.shape[0], step):
        c = coords[s:s + step]
        d2 = ((c[:, None, :] - pts[None, :, :]) ** 2).sum(-1)
        out[s:s + step] = np.argmin(d2, axis=1)  # first minimum: lower id on ties
    return out


def _permutation(w: Workload, cid: np.ndarray) -> np.ndarray:
    rng = np.random.default_rng([w.seed])
    rng.random((w.clusters, 3))  # the seed points come first in this stream
    relabel = rng.permutation(w.clusters)
    perm = np.arange(w.N_pad, dtype=np.int32)
    perm[: w.N] = np.argsort(relabel[cid], kind="stable").astype(np.int32)
    return perm


def generate(w: Workload, heads: Optional[Iterable[int]] = None) -> dict:
    """Make Q, K, V (and the gather index) for workload ``w``.

    Returns a dict with ``q``, ``k``, ``v`` of shape [B, len(heads), N_pad, d]
    (float32 for fp32 workloads, uint16 bf16 bit patterns for bf16 ones),
    ``perm`` (int32[N_pad] or None) and ``heads`` (the head ids made).
    Rows N..N_pad-1 are zero.
    """
    heads = list(range(w.H)) if heads is None else list(heads)
    cid = cluster_ids(w)
    N, Np, d = w.N, w.N_pad, w.d
    shape = (w.B, len(heads), Np, d)
    bf16 = w.dtype == "bf16"
    store = np.uint16 if bf16 else np.float32
    q = np.zeros(shape, dtype=store)
    k = np.zeros(shape, dtype=store)
    v = np.zeros(shape, dtype=store)
    inv_sqrt_d = np.float32(1.0 / math.sqrt(d))

    def one_head(job):
        b, hi, h = job
        rng = np.random.default_rng([w.seed, 1, b, h])
        mu = rng.standard_normal((w.clusters, d), dtype=np.float32) * np.float32(w.centroid_std)
        base = mu[cid]
        if w.key_spread == "clustered":
            u = np.random.default_rng([w.seed, 3, b, h]).uniform(0.0, 3.0, w.clusters)
            k_std = (np.float32(w.noise_std) * np.exp2(u).astype(np.float32))[cid][:, None]
        elif w.key_spread == "uniform":
            k_std = np.float32(w.noise_std)
        else:
            raise ValueError(f"unknown key_spread {w.key_spread!r}")
        out = []
        for which in ("q", "k", "v"):  # Q, K share the centroid; V is pure noise
            x = rng.standard_normal((N, d), dtype=np.float32)
            if which != "v":
                x *= k_std if which == "k" else np.float32(w.noise_std)
                x += base
                x *= inv_sqrt_d
            out.append(x)
        if w.value_mode == "clustered":
            nu = np.random.default_rng([w.seed, 2, b, h]).standard_normal((w.clusters, d), dtype=np.float32)
            out[2] *= np.float32(w.noise_std)
            out[2] += nu[cid]
        elif w.value_mode != "noise":
            raise ValueError(f"unknown value_mode {w.value_mode!r}")
        for dst, x in zip((q, k, v), out):
            dst[b, hi, :N] = bf16_bits_from_f32(x) if bf16 else x

    jobs = [(b, hi, h) for b in range(w.B) for hi, h in enumerate(heads)]
    workers = max(1, min(8, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one_head, jobs))
    perm = _permutation(w, cid) if w.permute else None
    return {"q": q, "k": k, "v": v, "perm": perm, "heads": heads}


def as_float32(x: np.ndarray) -> np.ndarray:
    """fp32 view of a generated tensor (bf16 bit patterns are widened exactly)."""
    if x.dtype == np.uint16:
        return f32_from_bf16_bits(x)
    return np.asarray(x, dtype=np.float32)
