// attn_launch.h - internal launcher interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
// Element strides of one [B, H, S, D] tensor whose D elements are
// contiguous: batch, head and row (sequence position).  The contiguous layout
// is {H*S*D, S*D, D}.
struct Layout {
  int64_t sb, sh;
  int ss;
};
}  // namespace attn

namespace attn {

// Validated arguments of one call (the C ABI fills this after checking them).
struct Args {
  const void *q, *k, *v, *dO;
  const void *o_in;          // O as the backward reads it (output dtype)
  const float *lse_in, *delta_in;
  void *o, *dq, *dk, *dv;    // outputs: fp32, or the 16-bit input dtype when out16
  float *lse, *delta;
  int B, H, S, D;
  int H_kv;                 // key/value heads (H for plain multi-head attention)
  float scale;
  bool doc;                 // packed-document mask
  const int32_t *cu_seqlens;
  int n_seqs, max_seqlen;
  int dtype;                // input dtype: ATTN_DTYPE_F32, _BF16 or _F16 (attn_api.h)
  bool half() const { return dtype != 0; }  // 16-bit inputs
  bool out16;               // O, dQ, dK, dV in the input dtype (16-bit inputs only)
  const float *rope;        // RoPE table [rope_npos][D/2][2] (cos, sin), or NULL: dQ and dK
  int rope_npos;            // epilogues turn the gradients back by the row's angles
  // element strides of each [B, H(_kv), S, D] tensor (contiguous unless the caller gives others)
  Layout lq, lk, lv, lo, ldo, ldq, ldk, ldv;
  hipStream_t stream;
  // the contiguous layout for every tensor (k, v, dk, dv with H_kv heads)
  void contiguous() {
    const Layout qs{(int64_t)H * S * D, (int64_t)S * D, D};
    const Layout ks{(int64_t)H_kv * S * D, (int64_t)S * D, D};
    lq = lo = ldo = ldq = qs;
    lk = lv = ldk = ldv = ks;
  }
};

// Decode step against a key/value cache (attn_decode).
struct DecodeArgs {
  const void *q, *k_cache, *v_cache;
  const int32_t *cache_lens;
  float *o, *lse;
  float *o_part, *lse_part;  // chunk partials (workspace), unused with one chunk
  int B, H, H_kv, S_max, D, max_len;
  float scale;
  int dtype;
  hipStream_t stream;
};
hipError_t launch_decode(const DecodeArgs &a);
size_t decode_workspace_bytes(int B, int H, int H_kv, int D, int max_len);
// The same with the partials in the library's static per-device scratch
// (a.o_part, a.lse_part ignored); the caller has checked the size against
// decode_scratch_bytes().
hipError_t launch_decode_noalloc(DecodeArgs a);
size_t decode_scratch_bytes();

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const Args &a);
hipError_t launch_bwd_preprocess(const Args &a);
hipError_t launch_bwd_dkdv(const Args &a);
// Grouped heads with a workspace: the number of parts the dK/dV step splits
// each group into (0: the parts path does not apply), the workspace it needs,
// and the step itself (launch_bwd_dkdv where no parts apply).
int dkdv_parts(const Args &a);
size_t dkdv_workspace_bytes(const Args &a);
hipError_t launch_bwd_dkdv_parts(const Args &a, float *ws);
hipError_t launch_bwd_dq(const Args &a);
// Small causal grids at D = 64 (16-bit inputs, H_kv == H): whether the
// one-launch backward applies, and the backward itself (Delta, dK/dV, dQ).
bool bwd_small_applies(const Args &a);
hipError_t launch_bwd_small(const Args &a);
// Packed-document launches (attn_bwd_doc.hip): launch_bwd_dkdv,
// launch_bwd_dq / launch_bwd_dq_delta (fuse_delta) and the parts step of
// launch_bwd_dkdv_parts (P parts into wk, wv, n elements each), for a.doc.
hipError_t launch_bwd_dkdv_doc(const Args &a);
hipError_t launch_bwd_dq_doc(const Args &a, bool fuse_delta);
hipError_t launch_bwd_dkdv_parts_doc(const Args &a, int P, float *wk, float *wv, int64_t n);
// 16-bit inputs only: dQ that also computes Delta from O and dO (written to a.delta)
hipError_t launch_bwd_dq_delta(const Args &a);
// RoPE: the cos/sin table, and the rotation of a.q, a.k into q_rot, k_rot (table a.rope)
hipError_t launch_rope_table(float *tab, int n_pos, int D, double base, hipStream_t stream);
hipError_t launch_rope(const Args &a, void *q_rot, void *k_rot);
// Clock probe (attn_clock_probe): shader cycles and real-time ticks over `ticks`.
hipError_t launch_clock_probe(unsigned long long *out, unsigned long long ticks, hipStream_t stream);

}  // namespace attn
