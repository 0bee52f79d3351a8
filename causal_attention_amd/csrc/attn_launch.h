// attn_launch.h - internal launcher interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Validated arguments of one call (the C ABI fills this after checking them).
struct Args {
  const void *q, *k, *v, *dO;
  const float *o_in, *lse_in, *delta_in;
  float *o, *lse, *dq, *dk, *dv, *delta;
  int B, H, S, D;
  int H_kv;                 // key/value heads (H for plain multi-head attention)
  float scale;
  bool doc;                 // packed-document mask
  const int32_t *cu_seqlens;
  int n_seqs, max_seqlen;
  bool bf16;                // input dtype: bf16 (true) or fp32 (false)
  hipStream_t stream;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const Args &a);
hipError_t launch_bwd_preprocess(const Args &a);
hipError_t launch_bwd_dkdv(const Args &a);
hipError_t launch_bwd_dq(const Args &a);
// bf16 only: dQ that also computes Delta from O and dO (written to a.delta)
hipError_t launch_bwd_dq_delta(const Args &a);

}  // namespace attn
