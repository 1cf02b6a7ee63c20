"""bsa_mfma_ceiling, the sustained-MFMA-rate probe the bench reads bsa_attend's
rate against: its output is the product its fragments define (so the
matrix-core work it is timed on is really done), and it reaches a rate above
bsa_attend's and below the published peak."""

import numpy as np
import pytest
import torch

import block_sparse_attention_27_amd as bsa
from gpu_util import print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bsa.load_library()


def _expected(iters: int) -> np.ndarray:
    """Per lane: 8 iters sum_r C[i_r][l % 32] for the 32x16 A and 16x32 B the lanes' fragments form."""
    lanes = np.arange(64)
    e = np.arange(8)
    c1, c2 = torch.tensor(0.001, dtype=torch.float32), torch.tensor(0.002, dtype=torch.float32)
    a = (c1 * torch.from_numpy((lanes[:, None] + e[None, :]).astype(np.float32))).to(torch.bfloat16)
    b = (c2 * torch.from_numpy((lanes[:, None] - e[None, :]).astype(np.float32))).to(torch.bfloat16)
    a, b = a.double().numpy(), b.double().numpy()
    A = np.empty((32, 16))
    B = np.empty((16, 32))
    for k in range(16):
        A[:, k] = a[np.arange(32) + 32 * (k // 8), k % 8]
        B[k, :] = b[np.arange(32) + 32 * (k // 8), k % 8]
    C = A @ B
    out = np.empty(64)
    for l in lanes:
        rows = [8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)]
        out[l] = 8 * iters * C[rows, l % 32].sum()
    return out


def test_output_is_the_fragment_product():
    print_case("bsa_mfma_ceiling: 3 rounds, 2 workgroups, against the product of its fragments")
    iters, n_wg = 3, 2
    out = torch.full((n_wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    bsa.bsa_mfma_ceiling(out, iters, n_wg)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(n_wg * 4, 64)
    ref = _expected(iters)
    assert np.allclose(got, ref[None, :], rtol=1e-5, atol=1e-6 * np.abs(ref).max()), np.abs(got - ref).max()


def _lowbias32(x: np.ndarray) -> np.ndarray:
    """Wellons' lowbias32 integer hash on uint32 arrays (arithmetic mod 2^32)."""
    x = x.astype(np.uint64)
    m = np.uint64(0xFFFFFFFF)
    x ^= x >> np.uint64(16)
    x = (x * np.uint64(0x7FEB352D)) & m
    x ^= x >> np.uint64(15)
    x = (x * np.uint64(0x846CA68B)) & m
    x ^= x >> np.uint64(16)
    return x


def _expected_random(iters: int, n_wg: int) -> np.ndarray:
    """Per thread: the sum of its accumulators for the hashed fragments of bsa_mfma_ceiling_random."""
    n = np.arange(n_wg * 256, dtype=np.uint64)
    lane = (n % np.uint64(64))
    f = np.arange(4, dtype=np.uint64)[None, :, None]
    e = np.arange(8, dtype=np.uint64)[None, None, :]
    base = (n * np.uint64(64))[:, None, None]

    def val(x):
        v = (_lowbias32(x) >> np.uint64(8)).astype(np.float64) * (4.0 / 16777216.0) - 2.0
        return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()

    a = val(base + np.uint64(8) * f + e)                                        # [thread, f, e]
    b = val(base + np.uint64(32) + np.uint64(8) * f + e + lane[:, None, None])  # [thread, f, e]
    out = np.empty(n_wg * 256)
    for wv in range(n_wg * 4):
        t = np.arange(64) + 64 * wv
        A = np.empty((4, 32, 16))
        B = np.empty((4, 16, 32))
        for k in range(16):
            A[:, :, k] = a[t[np.arange(32) + 32 * (k // 8)], :, k % 8].T
            B[:, k, :] = b[t[np.arange(32) + 32 * (k // 8)], :, k % 8].T
        T = np.zeros((32, 32))
        for c in range(8):
            for u in range(4):
                T += A[(c + u) % 4] @ B[(c // 2 + 3 * u) % 4]
        T *= iters // 4
        for l in range(64):
            rows = [8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)]
            out[t[l]] = T[rows, l % 32].sum()
    return out


def test_random_operand_output_is_the_fragment_product():
    print_case("bsa_mfma_ceiling_random: 8 rounds, 2 workgroups, against the products of its hashed fragments")
    iters, n_wg = 8, 2
    out = torch.full((n_wg * 256,), float("nan"), dtype=torch.float32, device="cuda")
    bsa.bsa_mfma_ceiling_random(out, iters, n_wg)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = _expected_random(iters, n_wg)
    # fp32 accumulation of 16 x 16 x 8 x 8 products of magnitude <= 4: a few ulps of the partial sums
    assert np.allclose(got, ref, rtol=1e-4, atol=1e-4 * np.abs(ref).max()), np.abs(got - ref).max()


def test_rate_is_between_attention_and_peak():
    import bench
    print_case("bsa_mfma_ceiling: sustained rate, 512 workgroups, ~10 ms launches")
    r = bench.mfma_ceiling(bsa, torch, iters=40000, n_wg=512, reps=3)
    print_case(f"  {r['tflops']} TFLOP/s ({r['frac_of_peak'] * 100:.1f}% of {bench.PEAK_BF16_TFLOPS:.0f})")
    # at least what the attention kernel sustains, at most the published peak
    assert 1000.0 < r["tflops"] <= bench.PEAK_BF16_TFLOPS
    rr = bench.mfma_ceiling(bsa, torch, iters=40000, n_wg=512, reps=3, random=True)
    print_case(f"  random operands: {rr['tflops']} TFLOP/s ({rr['frac_of_peak'] * 100:.1f}%)")
    assert 1000.0 < rr["tflops"] <= bench.PEAK_BF16_TFLOPS
