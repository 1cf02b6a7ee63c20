// C ABI of libbsa.so: argument validation and dispatch. Every check runs on
// the host before any HIP call, so a rejected call launches nothing and needs
// no GPU.
#include "../../include/bsa.h"
#include "bsa_internal.hpp"

#include <math.h>

namespace {

constexpr int kMaxSelectUnits = 4096;  // |valid units| * 2^20 must fit the 2^32 fixed point
constexpr int kMaxClusterIters = 16;   // Lloyd iterations accepted by bsa_score_ibcs

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by all calls; fills the geometry.
bsa_status check_problem(const bsa_problem* p, bsa::Geometry* g) {
  if (p == nullptr) return BSA_ERR_INVALID_ARG;
  if (p->kv_permuted != 0 && p->kv_permuted != 1) return BSA_ERR_INVALID_ARG;
  if (p->B < 1 || p->H < 1 || p->N < 1 || p->N_pad < p->N) return BSA_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return BSA_ERR_INVALID_ARG;
  if (p->block_q != 64 && p->block_q != 128) return BSA_ERR_INVALID_ARG;
  if (p->block_k != 32 && p->block_k != 64 && p->block_k != 128) return BSA_ERR_INVALID_ARG;
  if (p->N_pad % p->block_q != 0 || p->N_pad % p->block_k != 0) return BSA_ERR_INVALID_ARG;
  if (p->dtype != BSA_BF16 && p->dtype != BSA_FP32) return BSA_ERR_INVALID_ARG;
  if (p->out_fp32 != 0 && p->out_fp32 != 1) return BSA_ERR_INVALID_ARG;
  if (!(p->sm_scale > 0.f) || !isfinite(p->sm_scale)) return BSA_ERR_INVALID_ARG;
  // index arithmetic inside the kernels: rows of one (b, h) and workgroup ids in int32
  if (p->N_pad > (1 << 28)) return BSA_ERR_INVALID_ARG;
  const int64_t nQB = p->N_pad / p->block_q;
  if (static_cast<int64_t>(p->B) * p->H * nQB > 0x7FFFFFFFll) return BSA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(p->B) * p->H * (nQB + p->N_pad / p->block_k) > 0x7FFFFFFFll) return BSA_ERR_INVALID_ARG;
  g->B = p->B;
  g->H = p->H;
  g->N = p->N;
  g->N_pad = p->N_pad;
  g->d = p->d;
  g->block_q = p->block_q;
  g->block_k = p->block_k;
  g->nQB = static_cast<int>(nQB);
  g->nKU = p->N_pad / p->block_k;
  g->n_valid_units = (p->N + p->block_k - 1) / p->block_k;
  g->L = 0;
  g->bf16 = p->dtype == BSA_BF16;
  g->out_fp32 = p->out_fp32 == 1;
  g->kv_permuted = p->kv_permuted == 1;
  g->sm_scale = p->sm_scale;
  g->seed = p->seed;
  return BSA_OK;
}

// Budget checks for the calls that take a list: 1 <= k + m <= valid units.
bsa_status check_budget(const bsa_problem* p, bsa::Geometry* g) {
  if (p->k_exact < 0 || p->m_sample < 0) return BSA_ERR_INVALID_ARG;
  const int64_t L = static_cast<int64_t>(p->k_exact) + p->m_sample;
  if (L < 1 || L > g->n_valid_units) return BSA_ERR_INVALID_ARG;
  g->L = static_cast<int>(L);
  return BSA_OK;
}

// Calls that take a permutation: kv_permuted = 1 describes K and V gathered
// by one, so it needs one.
bool perm_ok(const bsa::Geometry& g, const int32_t* perm) {
  if (perm && !aligned(perm, 4)) return false;
  return perm != nullptr || !g.kv_permuted;
}

bsa_status from_hip(hipError_t e) { return e == hipSuccess ? BSA_OK : BSA_ERR_HIP; }

// The scoring kernels read one head's key means through a buffer resource
// whose byte count (nKU * d * 4) is a 32-bit record count.
bool score_units_ok(const bsa::Geometry& g) { return static_cast<int64_t>(g.nKU) * g.d * 4 <= 0x7FFFFFFFll; }

}  // namespace

namespace bsa {

hipError_t launch_attend_bf16(const Geometry& g, const void* q, const void* k, const void* v,
                              const int32_t* perm, const int32_t* idx, const float* w, void* out,
                              float* lse, hipStream_t s) {
  return g.d == 128 ? launch_attend_bf16_d128(g, q, k, v, perm, idx, w, out, lse, g.out_fp32, s)
                    : launch_attend_bf16_d64(g, q, k, v, perm, idx, w, out, lse, g.out_fp32, s);
}

}  // namespace bsa

extern "C" {

int32_t bsa_abi_version(void) { return BSA_ABI_VERSION; }

const char* bsa_status_string(int32_t status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported shape";
    case BSA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

bsa_status bsa_score(const bsa_problem* p, const void* q, const void* k, const int32_t* perm,
                     float* S, float* q_mean, float* k_mean, hipStream_t stream) {
  bsa::Geometry g;
  bsa_status st = check_problem(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !S || !q_mean || !k_mean) return BSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(S, 4) || !aligned(q_mean, 16) || !aligned(k_mean, 16))
    return BSA_ERR_INVALID_ARG;
  if (!perm_ok(g, perm)) return BSA_ERR_INVALID_ARG;
  if (!score_units_ok(g)) return BSA_ERR_UNSUPPORTED;
  st = from_hip(bsa::launch_block_means(g, q, k, perm, q_mean, k_mean, nullptr, false, stream));
  if (st != BSA_OK) return st;
  return from_hip(bsa::launch_scores(g, 1, q_mean, nullptr, k_mean, nullptr, S, stream));
}

bsa_status bsa_score_stats(const bsa_problem* p, const void* q, const void* k, const int32_t* perm, float* S,
                           float* q_mean, float* k_mean, float* k_var, hipStream_t stream) {
  bsa::Geometry g;
  bsa_status st = check_problem(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !S || !q_mean || !k_mean || !k_var) return BSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(S, 4) || !aligned(q_mean, 16) || !aligned(k_mean, 16) ||
      !aligned(k_var, 16))
    return BSA_ERR_INVALID_ARG;
  if (!perm_ok(g, perm)) return BSA_ERR_INVALID_ARG;
  if (!score_units_ok(g)) return BSA_ERR_UNSUPPORTED;
  st = from_hip(bsa::launch_block_means(g, q, k, perm, q_mean, k_mean, k_var, false, stream));
  if (st != BSA_OK) return st;
  return from_hip(bsa::launch_scores(g, 1, q_mean, nullptr, k_mean, k_var, S, stream));
}

bsa_status bsa_score_ibcs(const bsa_problem* p, int32_t groups, int32_t iters, const void* q, const void* k,
                          const int32_t* perm, float* S, float* q_cent, int32_t* q_size, float* k_mean,
                          hipStream_t stream) {
  bsa::Geometry g;
  bsa_status st = check_problem(p, &g);
  if (st != BSA_OK) return st;
  if (groups != 1 && groups != 2 && groups != 4 && groups != 8) return BSA_ERR_INVALID_ARG;
  if (iters < 1 || iters > kMaxClusterIters) return BSA_ERR_INVALID_ARG;
  if (!q || !k || !S || !q_cent || !q_size || !k_mean) return BSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(S, 4) || !aligned(q_cent, 16) || !aligned(q_size, 4) ||
      !aligned(k_mean, 16))
    return BSA_ERR_INVALID_ARG;
  if (!perm_ok(g, perm)) return BSA_ERR_INVALID_ARG;
  if (!score_units_ok(g)) return BSA_ERR_UNSUPPORTED;
  st = from_hip(bsa::launch_block_means(g, q, k, perm, nullptr, k_mean, nullptr, true, stream));
  if (st != BSA_OK) return st;
  st = from_hip(bsa::launch_block_clusters(g, groups, iters, q, perm, q_cent, q_size, stream));
  if (st != BSA_OK) return st;
  return from_hip(bsa::launch_scores(g, groups, q_cent, q_size, k_mean, nullptr, S, stream));
}

bsa_status bsa_permute_rows(const bsa_problem* p, const void* x, const int32_t* perm, void* x_perm,
                            hipStream_t stream) {
  bsa::Geometry g;
  bsa_status st = check_problem(p, &g);
  if (st != BSA_OK) return st;
  if (!x || !perm || !x_perm) return BSA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(x_perm, 16) || !aligned(perm, 4)) return BSA_ERR_INVALID_ARG;
  const int64_t row_bytes = static_cast<int64_t>(g.d) * (g.bf16 ? 2 : 4);
  const int64_t bytes = static_cast<int64_t>(g.B) * g.H * g.N_pad * row_bytes;
  const uintptr_t xs = reinterpret_cast<uintptr_t>(x), ys = reinterpret_cast<uintptr_t>(x_perm);
  if (xs < ys + static_cast<uintptr_t>(bytes) && ys < xs + static_cast<uintptr_t>(bytes)) return BSA_ERR_INVALID_ARG;
  // the kernel indexes the 16-byte chunks of one (b, h) in int32, and the grid
  // (1024 chunks per 256-thread workgroup) must stay within 2^32 work-items
  const int64_t chunks = static_cast<int64_t>(g.N_pad) * (row_bytes / 16);
  if (chunks > 0x7FFFFFFFll - 1024) return BSA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(g.B) * g.H * ((chunks + 1023) / 1024) * 256 > 0xFFFFFFFFll) return BSA_ERR_UNSUPPORTED;
  return from_hip(bsa::launch_permute_rows(g, x, perm, x_perm, stream));
}

bsa_status bsa_select(const bsa_problem* p, const float* S, int32_t* idx, float* w, hipStream_t stream) {
  bsa::Geometry g;
  bsa_status st = check_problem(p, &g);
  if (st != BSA_OK) return st;
  st = check_budget(p, &g);
  if (st != BSA_OK) return st;
  if (!S || !idx || !w) return BSA_ERR_INVALID_ARG;
  if (!aligned(S, 4) || !aligned(idx, 4) || !aligned(w, 4)) return BSA_ERR_INVALID_ARG;
  if (g.n_valid_units > kMaxSelectUnits) return BSA_ERR_UNSUPPORTED;
  return from_hip(bsa::launch_select(g, p->k_exact, p->m_sample, S, idx, w, stream));
}

bsa_status bsa_attend(const bsa_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* perm, const int32_t* idx, const float* w, void* out, float* lse,
                      hipStream_t stream) {
  bsa::Geometry g;
  bsa_status st = check_problem(p, &g);
  if (st != BSA_OK) return st;
  st = check_budget(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !idx || !w || !out) return BSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(idx, 4) ||
      !aligned(w, 4) || (lse && !aligned(lse, 4)) || !perm_ok(g, perm))
    return BSA_ERR_INVALID_ARG;
  if (g.bf16) return from_hip(bsa::launch_attend_bf16(g, q, k, v, perm, idx, w, out, lse, stream));
  return from_hip(bsa::launch_attend_fp32(g, q, k, v, perm, idx, w, out, lse, stream));
}

bsa_status bsa_attend_dense(const bsa_problem* p, const void* q, const void* k, const void* v,
                            const int32_t* perm, void* out, float* lse, hipStream_t stream) {
  bsa::Geometry g;
  bsa_status st = check_problem(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !out) return BSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)) || !perm_ok(g, perm))
    return BSA_ERR_INVALID_ARG;
  if (g.bf16) return from_hip(bsa::launch_attend_bf16(g, q, k, v, perm, nullptr, nullptr, out, lse, stream));
  return from_hip(bsa::launch_attend_fp32(g, q, k, v, perm, nullptr, nullptr, out, lse, stream));
}

bsa_status bsa_mfma_ceiling(float* out, int32_t iters, int32_t n_wg, hipStream_t stream) {
  if (!out || !aligned(out, 4) || iters < 1 || n_wg < 1) return BSA_ERR_INVALID_ARG;
  return from_hip(bsa::launch_mfma_ceiling(out, iters, n_wg, false, stream));
}

bsa_status bsa_mfma_ceiling_random(float* out, int32_t iters, int32_t n_wg, hipStream_t stream) {
  if (!out || !aligned(out, 4) || iters < 4 || iters % 4 != 0 || n_wg < 1 || n_wg > (1 << 18))
    return BSA_ERR_INVALID_ARG;
  return from_hip(bsa::launch_mfma_ceiling(out, iters, n_wg, true, stream));
}

}  // extern "C"
