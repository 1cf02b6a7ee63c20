// Weighted block-sparse flash attention (and its dense special case) on bf16
// MFMA for gfx950: launch and dispatch over the kernel variants
// (attend_bf16_w32.hpp). Instantiated per head dimension in
// attend_bf16_d128.hip and attend_bf16_d64.hip.
#pragma once

#include "attend_bf16_w32.hpp"

namespace bsa {
namespace attend_bf16_impl {

template <int D, int BQ, int BK, bool DENSE, bool PERM, bool OUT32>
hipError_t launch_one(const AttendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attend_w32_kernel<D, BQ, BK, DENSE, PERM, OUT32>), dim3(a.n_wg), dim3(BQ * 4), 0, s, a);
  return hipGetLastError();
}

template <int D, int BQ, bool DENSE, bool PERM, bool OUT32>
hipError_t dispatch_bk(const AttendArgs& a, int bk, hipStream_t s) {
  if constexpr (DENSE) {
    return launch_one<D, BQ, 128, true, PERM, OUT32>(a, s);
  } else {
    switch (bk) {
      case 32: return launch_one<D, BQ, 32, false, PERM, OUT32>(a, s);
      case 64: return launch_one<D, BQ, 64, false, PERM, OUT32>(a, s);
      default: return launch_one<D, BQ, 128, false, PERM, OUT32>(a, s);
    }
  }
}

template <int D, int BQ, bool OUT32>
hipError_t dispatch_mode(const AttendArgs& a, int bk, bool dense, bool perm, hipStream_t s) {
  if (dense) return perm ? dispatch_bk<D, BQ, true, true, OUT32>(a, bk, s) : dispatch_bk<D, BQ, true, false, OUT32>(a, bk, s);
  return perm ? dispatch_bk<D, BQ, false, true, OUT32>(a, bk, s) : dispatch_bk<D, BQ, false, false, OUT32>(a, bk, s);
}

// Launch for one head dimension D (one translation unit per D).
template <int D>
hipError_t launch_d(const Geometry& g, const void* q, const void* k, const void* v, const int32_t* perm,
                    const int32_t* idx, const float* w, void* out, float* lse, bool out_fp32, hipStream_t s) {
  const bool dense = idx == nullptr;
  AttendArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.perm = perm;
  a.idx = idx;
  a.w = w;
  a.out = out;
  a.lse = lse;
  a.H = g.H;
  a.N = g.N;
  a.N_pad = g.N_pad;
  a.nQB = g.nQB;
  a.nKU = g.nKU;
  a.L = dense ? 0 : g.L;
  a.qchunk = (g.nQB + 7) / 8;
  a.n_wg = 8 * a.qchunk * g.B * g.H;
  a.c = g.sm_scale * 1.4426950408889634f;
  const bool p = perm != nullptr;
  if (out_fp32) {
    return g.block_q == 128 ? dispatch_mode<D, 128, true>(a, g.block_k, dense, p, s)
                            : dispatch_mode<D, 64, true>(a, g.block_k, dense, p, s);
  }
  return g.block_q == 128 ? dispatch_mode<D, 128, false>(a, g.block_k, dense, p, s)
                          : dispatch_mode<D, 64, false>(a, g.block_k, dense, p, s);
}

}  // namespace attend_bf16_impl
}  // namespace bsa
