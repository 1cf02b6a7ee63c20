// Weighted block-sparse attention (and dense attention) in fp32 on the vector
// ALUs: the exact-precision variant for fp32 Q/K/V.
//
// Same mathematics as the bf16 MFMA kernel (AB-Attention, Abstract and
// transcript: weights applied as pre-softmax shifts, one pass estimating
// dense attention): for each query row, over the listed units and their valid
// keys, an online softmax in base 2 whose exponent carries log2(w_j).
//
// One workgroup per (b, h, query block), one thread per query row holding q
// and its output accumulator in registers. Keys are streamed through LDS in
// segments of up to 32 rows; every thread reads the same K/V row at a time
// (an LDS broadcast).
#include "bsa_internal.hpp"

#include <math.h>

namespace bsa {
namespace {

constexpr int SEG = 32;

struct Fp32Args {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* perm;
  const int32_t* idx;
  const float* w;
  float* out;
  float* lse;
  int N, N_pad, nQB, nKU, L, block_k, n_wg;
  int kv_gather;  // 1: key rows go through perm as well (the sparse pass on K and V in token order)
  float c;        // sm_scale * log2(e)
};

template <bool PERM>
__device__ __forceinline__ int row_of(const Fp32Args& a, int r, bool& ok) {
  if constexpr (PERM) {
    if (!ok) return 0;
    const int g = a.perm[r];
    ok = static_cast<unsigned>(g) < static_cast<unsigned>(a.N_pad);
    return ok ? g : 0;
  } else {
    return r;
  }
}

template <int D, int BQ, bool DENSE, bool PERM>
__global__ __launch_bounds__(BQ) void attend_fp32_kernel(Fp32Args a) {
  __shared__ float ks[SEG][D];
  __shared__ float vs[SEG][D];
  const int tid = threadIdx.x;
  const int logical = xcd_remap(blockIdx.x, a.n_wg);
  const int bh = logical / a.nQB, qi = logical % a.nQB;
  const size_t off = static_cast<size_t>(bh) * a.N_pad * D;
  const float* kb = a.k + off;
  const float* vb = a.v + off;

  const int qrow = qi * BQ + tid;
  bool qok = qrow < a.N;
  const int qg = row_of<PERM>(a, qrow, qok);
  float qv[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = qok ? a.q[off + static_cast<size_t>(qg) * D + c] : 0.f;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int n_entries = DENSE ? (a.N + SEG - 1) / SEG : a.L * (a.block_k / SEG);
  for (int e = 0; e < n_entries; ++e) {
    int base, cnt;
    float lw = 0.f;
    if constexpr (DENSE) {
      base = e * SEG;
      cnt = min(SEG, a.N - base);
    } else {
      const int per = a.block_k / SEG;
      const int ent = e / per, sub = e % per;
      const int j = a.idx[static_cast<size_t>(logical) * a.L + ent];
      const float wv = a.w[static_cast<size_t>(logical) * a.L + ent];
      const bool ok = j >= 0 && j < a.nKU && wv > 0.f && wv < INFINITY;
      base = ok ? j * a.block_k + sub * SEG : 0;
      cnt = ok ? max(0, min(SEG, a.N - base)) : 0;
      lw = ok ? log2f(wv) : 0.f;
    }
    __syncthreads();
    for (int x = tid; x < SEG * D; x += BQ) {
      const int r = x / D, col = x % D;
      bool ok = r < cnt;
      const int g = a.kv_gather ? row_of<PERM>(a, base + r, ok) : base + r;
      ks[r][col] = ok ? kb[static_cast<size_t>(g) * D + col] : 0.f;
      vs[r][col] = ok ? vb[static_cast<size_t>(g) * D + col] : 0.f;
    }
    __syncthreads();
    if (cnt == 0) continue;
    float x[SEG];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < SEG; ++r) {
      float s = 0.f;
#pragma unroll
      for (int col = 0; col < D; ++col) s = fmaf(qv[col], ks[r][col], s);
      x[r] = r < cnt ? fmaf(s, a.c, lw) : -INFINITY;  // shifted logit x + log2(w)
      mx = fmaxf(mx, x[r]);
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int col = 0; col < D; ++col) acc[col] *= alpha;
    m = m_new;
#pragma unroll
    for (int r = 0; r < SEG; ++r) {
      const float p = exp2f(x[r] - m);
      l += p;
#pragma unroll
      for (int col = 0; col < D; ++col) acc[col] = fmaf(p, vs[r][col], acc[col]);
    }
  }

  if (qrow < a.N) {
    bool ok = true;
    const int orow = row_of<PERM>(a, qrow, ok);
    if (ok) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float* op = a.out + off + static_cast<size_t>(orow) * D;
#pragma unroll
      for (int col = 0; col < D; ++col) op[col] = acc[col] * inv;
      if (a.lse != nullptr) {
        a.lse[static_cast<size_t>(bh) * a.N_pad + orow] =
            l > 0.f ? (m + log2f(l)) * 0.69314718055994531f : -INFINITY;
      }
    }
  } else {
    float* op = a.out + off + static_cast<size_t>(qrow) * D;
#pragma unroll
    for (int col = 0; col < D; ++col) op[col] = 0.f;
    if (a.lse != nullptr) a.lse[static_cast<size_t>(bh) * a.N_pad + qrow] = -INFINITY;
  }
}

template <int D, int BQ>
hipError_t dispatch(const Fp32Args& a, bool dense, bool perm, hipStream_t s) {
  if (dense) {
    if (perm) hipLaunchKernelGGL((attend_fp32_kernel<D, BQ, true, true>), dim3(a.n_wg), dim3(BQ), 0, s, a);
    else hipLaunchKernelGGL((attend_fp32_kernel<D, BQ, true, false>), dim3(a.n_wg), dim3(BQ), 0, s, a);
  } else {
    if (perm) hipLaunchKernelGGL((attend_fp32_kernel<D, BQ, false, true>), dim3(a.n_wg), dim3(BQ), 0, s, a);
    else hipLaunchKernelGGL((attend_fp32_kernel<D, BQ, false, false>), dim3(a.n_wg), dim3(BQ), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_fp32(const Geometry& g, const void* q, const void* k, const void* v,
                              const int32_t* perm, const int32_t* idx, const float* w, void* out,
                              float* lse, hipStream_t s) {
  Fp32Args a;
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.perm = perm;
  a.idx = idx;
  a.w = w;
  a.out = static_cast<float*>(out);
  a.lse = lse;
  a.N = g.N;
  a.N_pad = g.N_pad;
  a.nQB = g.nQB;
  a.nKU = g.nKU;
  a.L = g.L;
  a.block_k = g.block_k;
  a.n_wg = g.B * g.H * g.nQB;
  a.c = g.sm_scale * 1.4426950408889634f;
  const bool dense = idx == nullptr, p = perm != nullptr;
  // dense attention takes every valid key, in whatever order: no key gather
  a.kv_gather = p && !dense && !g.kv_permuted;
  if (g.d == 128) return g.block_q == 128 ? dispatch<128, 128>(a, dense, p, s) : dispatch<128, 64>(a, dense, p, s);
  return g.block_q == 128 ? dispatch<64, 128>(a, dense, p, s) : dispatch<64, 64>(a, dense, p, s);
}

}  // namespace bsa
