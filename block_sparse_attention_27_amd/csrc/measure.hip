// Measurement aid: the sustained rate of the bf16 matrix cores.
//
// The published bf16 peak assumes the top clock. Under a long matrix load the
// chip runs well below it (at or near its socket power limit), so the rate a
// kernel can reach is set by what else it spends energy on. This kernel spends
// it on nothing else: every wave keeps 8 independent v_mfma_f32_32x32x16_bf16
// chains on register operands (no memory traffic, no other vector work in the
// loop), in workgroups of 4 waves, two per CU as in the attention kernel. Its
// rate is the ceiling a matrix-bound kernel meets on the same chip and clock
// policy.
//
// The energy of a matrix product depends on its data: operands that stay the
// same from one product to the next toggle few bits. So the probe runs in two
// forms: constant operands (one A and one B fragment for every round) and
// random operands (four A and four B fragments of hashed values in [-2, 2),
// taken in a rotation that changes both operands from one MFMA to the next),
// whose rate is the ceiling for products over real data such as attention's.
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_CHAINS = 8;

// Lane l (of 64) holds the A fragment a_e = bf16(0.001 (l + e)) and the B
// fragment b_e = bf16(0.002 (l - e)), e = 0..7, and after `iters` rounds writes
// the sum of its 8 x 16 accumulators: 8 iters sum_r C[row_r][l % 32] with
// C = A B for the 32x16 A and 16x32 B those fragments form.
__global__ __launch_bounds__(PROBE_THREADS, 2) void mfma_ceiling_kernel(float* out, int iters) {
  const int lane = threadIdx.x % 64;
  probe_bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * static_cast<float>(lane + e));
    b[e] = static_cast<__bf16>(0.002f * static_cast<float>(lane - e));
  }
  probe_f32x16 acc[PROBE_CHAINS];
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = probe_f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[static_cast<size_t>(blockIdx.x) * PROBE_THREADS + threadIdx.x] = s;
}

// A value in [-2, 2) from a 32-bit counter: Wellons' lowbias32 integer hash
// (xorshift-multiply, constants 0x7feb352d and 0x846ca68b), top 24 bits as a
// fraction.
__device__ __forceinline__ float probe_value(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return static_cast<float>(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

// Random operands: thread t of workgroup g (n = 256 g + t, lane l = t % 64)
// holds A fragments a_f[e] = bf16(v(64 n + 8 f + e)) and B fragments
// b_f[e] = bf16(v(64 n + 32 + 8 f + e + l)), f = 0..3, e = 0..7. Round
// 4 j + u (u = 0..3) multiplies into chain c the fragments a_((c + u) mod 4)
// and b_((c / 2 + 3 u) mod 4), so consecutive MFMAs of a wave never repeat
// an operand pair. iters is a multiple of 4; the output is the sum of the
// lane's accumulators, as in the constant form.
__global__ __launch_bounds__(PROBE_THREADS, 2) void mfma_ceiling_random_kernel(float* out, int iters) {
  const int lane = threadIdx.x % 64;
  const uint32_t base = (blockIdx.x * PROBE_THREADS + threadIdx.x) * 64u;
  probe_bf16x8 a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[f][e] = static_cast<__bf16>(probe_value(base + 8 * f + e));
      b[f][e] = static_cast<__bf16>(probe_value(base + 32 + 8 * f + e + lane));
    }
  probe_f32x16 acc[PROBE_CHAINS];
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = probe_f32x16{};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < PROBE_CHAINS; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(c + u) & 3], b[((c >> 1) + 3 * u) & 3], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < PROBE_CHAINS; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[static_cast<size_t>(blockIdx.x) * PROBE_THREADS + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_ceiling(float* out, int iters, int n_wg, bool random_operands, hipStream_t s) {
  if (random_operands) {
    hipLaunchKernelGGL(mfma_ceiling_random_kernel, dim3(n_wg), dim3(PROBE_THREADS), 0, s, out, iters);
  } else {
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(n_wg), dim3(PROBE_THREADS), 0, s, out, iters);
  }
  return hipGetLastError();
}

}  // namespace bsa
