// Row gather into the permuted token order: x_perm[b][h][r] = x[b][h][perm[r]].
// Permuted block-sparse attention (InstaGen, Abstract) works on a sequence
// whose tokens are reordered so that similar ones sit together; done once per
// layer for K and V, the reorder lets the sparse pass stage every key unit as
// one contiguous run of rows, where gathering inside the pass would fetch each
// row separately on every one of its many reuses.
//
// A plain copy bound by HBM bandwidth: each thread moves PERMUTE_UNROLL
// 16-byte chunks (all loads first, then all stores), a wave covers whole rows
// of consecutive output positions, so the stores are contiguous and every
// load reads a contiguous part of one source row.
#include "bsa_internal.hpp"

namespace bsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int PERMUTE_THREADS = 256;
constexpr int PERMUTE_UNROLL = 4;
constexpr int CHUNKS_PER_WG = PERMUTE_THREADS * PERMUTE_UNROLL;

struct PermuteArgs {
  const char* x;
  const int32_t* perm;
  char* y;
  int N, N_pad;
  int wg_per_head;  // workgroups per (b, h): ceil(N_pad * CPR / CHUNKS_PER_WG)
};

template <int CPR>  // 16-byte chunks per row
__global__ __launch_bounds__(PERMUTE_THREADS) void permute_rows_kernel(PermuteArgs a) {
  constexpr int RB = 16 * CPR;  // bytes per row
  const int bh = blockIdx.x / a.wg_per_head;
  const int c0 = (blockIdx.x % a.wg_per_head) * CHUNKS_PER_WG + threadIdx.x;
  const size_t head = static_cast<size_t>(bh) * a.N_pad * RB;
  const int n_chunks = a.N_pad * CPR;
  u32x4 v[PERMUTE_UNROLL];
#pragma unroll
  for (int u = 0; u < PERMUTE_UNROLL; ++u) {
    const int c = c0 + u * PERMUTE_THREADS;
    const int r = c / CPR, col = c % CPR;
    int g = -1;  // rows past N and chunks past the head: zeros
    if (c < n_chunks && r < a.N) g = a.perm[r];
    const bool ok = static_cast<unsigned>(g) < static_cast<unsigned>(a.N_pad);
    v[u] = ok ? *reinterpret_cast<const u32x4*>(a.x + head + static_cast<size_t>(g) * RB + 16 * col)
              : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < PERMUTE_UNROLL; ++u) {
    const int c = c0 + u * PERMUTE_THREADS;
    if (c < n_chunks) *reinterpret_cast<u32x4*>(a.y + head + static_cast<size_t>(c) * 16) = v[u];
  }
}

}  // namespace

hipError_t launch_permute_rows(const Geometry& g, const void* x, const int32_t* perm, void* x_perm, hipStream_t s) {
  PermuteArgs a;
  a.x = static_cast<const char*>(x);
  a.perm = perm;
  a.y = static_cast<char*>(x_perm);
  a.N = g.N;
  a.N_pad = g.N_pad;
  const int cpr = g.d * (g.bf16 ? 2 : 4) / 16;
  a.wg_per_head = static_cast<int>((static_cast<int64_t>(g.N_pad) * cpr + CHUNKS_PER_WG - 1) / CHUNKS_PER_WG);
  const dim3 grid(static_cast<unsigned>(g.B) * g.H * a.wg_per_head);
  switch (cpr) {
    case 8: hipLaunchKernelGGL((permute_rows_kernel<8>), grid, dim3(PERMUTE_THREADS), 0, s, a); break;
    case 16: hipLaunchKernelGGL((permute_rows_kernel<16>), grid, dim3(PERMUTE_THREADS), 0, s, a); break;
    default: hipLaunchKernelGGL((permute_rows_kernel<32>), grid, dim3(PERMUTE_THREADS), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace bsa
