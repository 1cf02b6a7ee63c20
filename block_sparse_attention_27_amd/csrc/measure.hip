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

}  // namespace

hipError_t launch_mfma_ceiling(float* out, int iters, int n_wg, hipStream_t s) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(n_wg), dim3(PROBE_THREADS), 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace bsa
