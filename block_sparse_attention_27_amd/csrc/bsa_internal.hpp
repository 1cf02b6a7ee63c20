// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// Geometry derived from a validated bsa_problem.
struct Geometry {
  int B, H, N, N_pad, d, block_q, block_k;
  int nQB, nKU, n_valid_units, L;
  bool bf16;
  bool out_fp32;  // bf16 inputs with an fp32 output
  bool kv_permuted;  // K and V rows arrive in permuted order (only Q and out go through perm)
  float sm_scale;
  uint64_t seed;
};

// ---- scoring ----
// keys_only: key-unit means only (q and q_mean unused); k_var != nullptr: also
// the per-dimension population variance of every key unit
hipError_t launch_block_means(const Geometry& g, const void* q, const void* k, const int32_t* perm,
                              float* q_mean, float* k_mean, float* k_var, bool keys_only, hipStream_t s);
// groups in {1, 2, 4, 8}: q_rep holds `groups` representatives per query block,
// q_size their row counts (nullptr with groups == 1: weight 1); k_var != nullptr
// (groups == 1): statistics-aware logits s <q, k> + (s^2/2) <q^2, var>
hipError_t launch_scores(const Geometry& g, int groups, const float* q_rep, const int32_t* q_size,
                         const float* k_mean, const float* k_var, float* S, hipStream_t s);
// k-means of every query block's valid rows: `groups` centroids and row counts
hipError_t launch_block_clusters(const Geometry& g, int groups, int iters, const void* q,
                                 const int32_t* perm, float* q_cent, int32_t* q_size, hipStream_t s);

// ---- permutation ----
// x_perm[b][h][r] = x[b][h][perm[r]] for r < N (a zero row for an entry
// outside [0, N_pad)); rows N .. N_pad-1 of x_perm are zero
hipError_t launch_permute_rows(const Geometry& g, const void* x, const int32_t* perm, void* x_perm, hipStream_t s);
hipError_t launch_mfma_ceiling(float* out, int iters, int n_wg, bool random_operands, hipStream_t s);

// ---- selection ----
hipError_t launch_select(const Geometry& g, int k_exact, int m_sample, const float* S, int32_t* idx,
                         float* w, hipStream_t s);

// ---- attention ----
// idx/w == nullptr selects the dense variant (every valid key, weight 1).
hipError_t launch_attend_bf16_d128(const Geometry& g, const void* q, const void* k, const void* v,
                                   const int32_t* perm, const int32_t* idx, const float* w, void* out,
                                   float* lse, bool out_fp32, hipStream_t s);
hipError_t launch_attend_bf16_d64(const Geometry& g, const void* q, const void* k, const void* v,
                                  const int32_t* perm, const int32_t* idx, const float* w, void* out,
                                  float* lse, bool out_fp32, hipStream_t s);
hipError_t launch_attend_bf16(const Geometry& g, const void* q, const void* k, const void* v,
                              const int32_t* perm, const int32_t* idx, const float* w, void* out,
                              float* lse, hipStream_t s);
hipError_t launch_attend_fp32(const Geometry& g, const void* q, const void* k, const void* v,
                              const int32_t* perm, const int32_t* idx, const float* w, void* out,
                              float* lse, hipStream_t s);

// Maps a hardware workgroup id onto a logical one so that each of the 8 XCDs
// (which take workgroups round-robin) receives one contiguous logical range:
// neighbouring query blocks of one head then share an XCD's L2.
__device__ __forceinline__ int xcd_remap(int g, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = g % 8;
  return x * per + (x < rem ? x : rem) + g / 8;
}

}  // namespace bsa
