"""Seeded workload generator: determinism, shapes, padding, bf16 rounding, permutation."""

import numpy as np
import pytest
import torch

from block_sparse_attention_27_amd.inputs import (WORKLOADS, generate, bf16_bits_from_f32,
                                                  f32_from_bf16_bits, cluster_ids, as_float32)


def test_same_seed_same_bytes_and_head_subsets():
    w = WORKLOADS["tiny"]
    a, b = generate(w), generate(w)
    for key in ("q", "k", "v"):
        assert a[key].tobytes() == b[key].tobytes()
    w2 = WORKLOADS["wan13b"].replace(grid=(2, 8, 8), H=3)
    full = generate(w2)
    one = generate(w2, heads=[2])
    assert np.array_equal(full["q"][:, 2:3], one["q"])


def test_shapes_padding_and_dtypes():
    w = WORKLOADS["hunyuan"].replace(H=2, grid=(3, 9, 10))  # N = 270 -> N_pad = 384
    g = generate(w)
    assert w.N == 270 and w.N_pad == 384 and g["q"].shape == (1, 2, 384, 128)
    assert g["q"].dtype == np.uint16 and np.all(g["k"][..., 270:, :] == 0)
    perm = g["perm"]
    assert sorted(perm[:270].tolist()) == list(range(270))
    assert np.array_equal(perm[270:], np.arange(270, 384))
    cid = cluster_ids(w)[perm[:270]]
    # the gather groups each cluster into one contiguous run
    runs = 1 + int(np.count_nonzero(np.diff(cid)))
    assert runs == len(np.unique(cid))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -2.0 ** -130, 65504.0, 3.0e38], np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(f32_from_bf16_bits(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_headline_shape_numbers():
    w = WORKLOADS["wan14b_720p"]
    assert (w.N, w.N_pad, w.n_qblocks, w.n_units) == (75600, 75648, 591, 591)
    assert abs(w.executed_flops() - 1.190e13) / 1.190e13 < 1e-3
    h = WORKLOADS["hunyuan"]
    assert (h.N_pad, h.n_units, h.n_valid_units, h.list_len * h.block_k) == (118912, 3716, 3713, 296 * 32)


def test_clustered_values_follow_clusters_and_leave_q_k_alone():
    w = WORKLOADS["tiny"].replace(grid=(2, 8, 8), clusters=4)
    a, b = generate(w), generate(w.replace(value_mode="clustered"))
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["k"], b["k"])
    assert np.array_equal(b["v"], generate(w.replace(value_mode="clustered"))["v"])
    cid = cluster_ids(w)
    v = as_float32(b["v"])[0, 0, : w.N].astype(np.float64)
    # the within-cluster spread is the value noise (std 0.5); the cluster means differ by ~N(0, 2)
    within = np.mean([v[cid == c].std(axis=0).mean() for c in np.unique(cid) if (cid == c).sum() > 8])
    assert 0.35 < within < 0.65
    with pytest.raises(ValueError):
        generate(w.replace(value_mode="other"))


def test_clustered_key_spread_changes_only_the_key_noise():
    w = WORKLOADS["tiny"].replace(grid=(2, 8, 8), clusters=4)
    a, b = generate(w), generate(w.replace(key_spread="clustered"))
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["v"], b["v"])
    assert np.array_equal(b["k"], generate(w.replace(key_spread="clustered"))["k"])
    cid = cluster_ids(w)
    ka, kb = (as_float32(x["k"])[0, 0, : w.N].astype(np.float64) * np.sqrt(w.d) for x in (a, b))
    # the same centroids and the same unit normals: the deviations differ by one factor per cluster
    stds = []
    for c in np.unique(cid):
        rows = cid == c
        if rows.sum() < 8:
            continue
        dev_a = ka[rows] - ka[rows].mean(axis=0)
        dev_b = kb[rows] - kb[rows].mean(axis=0)
        ratio = np.linalg.norm(dev_b) / np.linalg.norm(dev_a)
        assert 0.9 < ratio < 8.5, ratio  # 2^u with u in [0, 3], up to the rounding of the noise draw
        stds.append(ratio)
    assert max(stds) / min(stds) > 1.5  # the spreads really differ between clusters
    with pytest.raises(ValueError):
        generate(w.replace(key_spread="other"))
