// bf16 MFMA attention kernels for head dimension 128 (kernel template in attend_bf16.hpp).
#include "attend_bf16.hpp"

namespace bsa {

hipError_t launch_attend_bf16_d128(const Geometry& g, const void* q, const void* k, const void* v,
                                   const int32_t* perm, const int32_t* idx, const float* w, void* out,
                                   float* lse, bool out_fp32, hipStream_t s) {
  return attend_bf16_impl::launch_d<128>(g, q, k, v, perm, idx, w, out, lse, out_fp32, s);
}

}  // namespace bsa
