// attn_bwd_doc.hip - packed-document launches of the backward kernels
// (attn_bwd_kernels.h).  A translation unit of its own so that these
// instantiations, which carry the work-ranked document schedule, take the
// compiler's default scheduling strategy rather than the iterative ILP one
// of the causal kernels.
#include "attn_bwd_kernels.h"

namespace attn {

hipError_t launch_bwd_dkdv_doc(const Args &a) {
  switch (a.dtype) {
    case 1: return a.out16 ? launch_dkdv_d<bf16, bf16, true>(a) : launch_dkdv_d<bf16, float, true>(a);
    case 2: return a.out16 ? launch_dkdv_d<f16, f16, true>(a) : launch_dkdv_d<f16, float, true>(a);
    default: return launch_dkdv_d<float, float, true>(a);
  }
}

hipError_t launch_bwd_dq_doc(const Args &a, bool fuse_delta) {
  if (fuse_delta) {
    switch (a.dtype) {
      case 1: return a.out16 ? launch_dq_d<bf16, bf16, true, true>(a) : launch_dq_d<bf16, float, true, true>(a);
      case 2: return a.out16 ? launch_dq_d<f16, f16, true, true>(a) : launch_dq_d<f16, float, true, true>(a);
      default: return hipErrorInvalidValue;  // Delta fusion follows the 16-bit preprocess layout
    }
  }
  switch (a.dtype) {
    case 1: return a.out16 ? launch_dq_d<bf16, bf16, true, false>(a) : launch_dq_d<bf16, float, true, false>(a);
    case 2: return a.out16 ? launch_dq_d<f16, f16, true, false>(a) : launch_dq_d<f16, float, true, false>(a);
    default: return launch_dq_d<float, float, true, false>(a);
  }
}

hipError_t launch_bwd_dkdv_parts_doc(const Args &a, int P, float *wk, float *wv, int64_t n) {
  const bool bf = a.dtype == 1;
  if (a.D == 128)
    return bf ? launch_dkdv_pair<bf16, float, 128, true>(a, P, wk, wv, n)
              : launch_dkdv_pair<f16, float, 128, true>(a, P, wk, wv, n);
  if (a.D == 64)
    return bf ? launch_dkdv_split<bf16, float, 64, true, 1>(a, P, wk, wv, n)
              : launch_dkdv_split<f16, float, 64, true, 1>(a, P, wk, wv, n);
  return bf ? launch_dkdv_split<bf16, float, 32, true, 1>(a, P, wk, wv, n)
            : launch_dkdv_split<f16, float, 32, true, 1>(a, P, wk, wv, n);
}

}  // namespace attn
