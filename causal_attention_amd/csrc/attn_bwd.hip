// attn_bwd.hip - backward entry points: Delta preprocess, dK/dV, dQ (the
// kernels are in attn_bwd_kernels.h).  Causal launches are instantiated here;
// packed-document launches come from attn_bwd_doc.hip.
#include "attn_bwd_kernels.h"

namespace attn {

template <typename T, typename OT>
static hipError_t launch_dkdv_dt(const Args &a) {
  return a.doc ? launch_bwd_dkdv_doc(a) : launch_dkdv_d<T, OT, false>(a);
}

template <typename T, typename OT, bool FUSE_DELTA>
static hipError_t launch_dq_dt(const Args &a) {
  return a.doc ? launch_bwd_dq_doc(a, FUSE_DELTA) : launch_dq_d<T, OT, false, FUSE_DELTA>(a);
}

hipError_t launch_bwd_preprocess(const Args &a) {
  switch (a.dtype) {
    case 1: return a.out16 ? launch_pre_dt<bf16, bf16>(a) : launch_pre_dt<bf16, float>(a);
    case 2: return a.out16 ? launch_pre_dt<f16, f16>(a) : launch_pre_dt<f16, float>(a);
    default: return launch_pre_dt<float, float>(a);
  }
}

hipError_t launch_bwd_dkdv(const Args &a) {
  switch (a.dtype) {
    case 1: return a.out16 ? launch_dkdv_dt<bf16, bf16>(a) : launch_dkdv_dt<bf16, float>(a);
    case 2: return a.out16 ? launch_dkdv_dt<f16, f16>(a) : launch_dkdv_dt<f16, float>(a);
    default: return launch_dkdv_dt<float, float>(a);
  }
}

// Grouped heads with a workspace (attn_bwd_gqa_ws).  At D = 128 the wave
// pairs chain a K/V head's whole group of query heads through each key
// block, and with few K/V heads their grid is small: fewer than 1024 64-key
// units leave the step waiting on the first key blocks' chains.  The parts
// path gives each (key block, K/V head) P workgroups, part p running G/P of
// the group's heads and writing its dK, dV to the workspace; then
// attn_bwd_sum_parts_kernel adds the P sets in part order (deterministic).
// At D <= 64 the one-wave kernel (128 keys per workgroup) takes the parts
// where G >= 8: the in-workgroup splits serve smaller groups better (the
// parts' partial sums cost as much HBM traffic as G / P more K/V heads).
// P is the smallest divisor of G that brings the grid to 1024 units, else G.
// 16-bit inputs (any output type, strides, RoPE: the parts are fp32 and
// contiguous, dK turned back by RoPE in each part, which is linear); 0 where
// it does not apply.
int dkdv_parts(const Args &a) {
  if (!a.half()) return 0;
  const int G = a.H / a.H_kv;
  if (a.D == 128 ? G % 2 != 0 : G < 8) return 0;
  const int bn = a.D == 128 ? 64 : 128;  // keys per workgroup
  const int64_t units = a.doc ? (int64_t)a.n_seqs * a.H_kv * ((a.max_seqlen + bn - 1) / bn)
                              : (int64_t)a.B * a.H_kv * ((a.S + bn - 1) / bn);
  if (units >= 1024) return 0;
  for (int p = 2; p < G; ++p)
    if (G % p == 0 && units * p >= 1024) return p;
  return G;
}

size_t dkdv_workspace_bytes(const Args &a) {
  const int P = dkdv_parts(a);
  return P == 0 ? 0 : (size_t)P * 2 * a.B * a.H_kv * a.S * a.D * sizeof(float);
}

// out = ws[0] + ws[1] + ... + ws[P-1], in that order, four elements per
// thread: over the n4 float4s of dK (parts 0 .. P-1 of the workspace, each a
// contiguous [B, H_kv, S, D] set) and then of dV (parts P .. 2P-1), stored in
// the output type through the outputs' layouts.
template <typename OT, int D>
__global__ __launch_bounds__(256) void attn_bwd_sum_parts_kernel(const f32x4 *__restrict__ ws, OT *__restrict__ dk,
                                                                  OT *__restrict__ dv, int P, int64_t n4, int S,
                                                                  int Hkv, Layout ldk, Layout ldv) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n4) return;
  const bool second = i >= n4;
  const int64_t j = second ? i - n4 : i;
  const f32x4 *src = ws + (second ? (int64_t)P * n4 : 0) + j;
  f32x4 acc = src[0];
  for (int p = 1; p < P; ++p) acc += src[(int64_t)p * n4];
  const int64_t r = j / (D / 4);  // row of the [B, H_kv, S, D] tensor
  const int col = (int)(j - r * (D / 4)) * 4;
  const int s = (int)(r % S);
  const int bh = (int)(r / S);
  const Layout &l = second ? ldv : ldk;
  const GBuf g((second ? dv : dk) + panel_off(l, bh / Hkv, bh % Hkv), panel_bytes(l, S, D, sizeof(OT)));
  store_out4<OT>(g, acc, (uint32_t)s * (uint32_t)l.ss + (uint32_t)col);
}

template <typename OT, int D>
static hipError_t launch_sum_parts(const Args &a, const float *ws, int P, int64_t n) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL((attn_bwd_sum_parts_kernel<OT, D>), dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0,
                     a.stream, reinterpret_cast<const f32x4 *>(ws), static_cast<OT *>(a.dk), static_cast<OT *>(a.dv),
                     P, n4, a.S, a.H_kv, a.ldk, a.ldv);
  return hipGetLastError();
}

template <typename OT>
static hipError_t launch_sum_parts_d(const Args &a, const float *ws, int P, int64_t n) {
  switch (a.D) {
    case 32: return launch_sum_parts<OT, 32>(a, ws, P, n);
    case 64: return launch_sum_parts<OT, 64>(a, ws, P, n);
    default: return launch_sum_parts<OT, 128>(a, ws, P, n);
  }
}

hipError_t launch_bwd_dkdv_parts(const Args &a, float *ws) {
  const int P = dkdv_parts(a);
  if (P == 0) return launch_bwd_dkdv(a);
  const int64_t n = (int64_t)a.B * a.H_kv * a.S * a.D;  // elements of dK (and of dV)
  float *wk = ws, *wv = ws + P * n;
  hipError_t e;
  const bool bf = a.dtype == 1;
  if (a.doc)
    e = launch_bwd_dkdv_parts_doc(a, P, wk, wv, n);
  else if (a.D == 128)
    e = bf ? launch_dkdv_pair<bf16, float, 128, false>(a, P, wk, wv, n)
           : launch_dkdv_pair<f16, float, 128, false>(a, P, wk, wv, n);
  else if (a.D == 64)
    e = bf ? launch_dkdv_split<bf16, float, 64, false, 1>(a, P, wk, wv, n)
           : launch_dkdv_split<f16, float, 64, false, 1>(a, P, wk, wv, n);
  else
    e = bf ? launch_dkdv_split<bf16, float, 32, false, 1>(a, P, wk, wv, n)
           : launch_dkdv_split<f16, float, 32, false, 1>(a, P, wk, wv, n);
  if (e != hipSuccess) return e;
  if (!a.out16) return launch_sum_parts_d<float>(a, ws, P, n);
  return bf ? launch_sum_parts_d<bf16>(a, ws, P, n) : launch_sum_parts_d<f16>(a, ws, P, n);
}

// Small causal grids (attn_bwd_small_kernel): the grids of fewer than 768
// workgroups on which dQ takes its 64-key tiles (launch_dq_t).
bool bwd_small_applies(const Args &a) {
  return a.half() && a.D == 64 && !a.doc && a.H_kv == a.H && (int64_t)a.B * a.H * ((a.S + 127) / 128) < 768;
}

template <typename T, typename OT>
static hipError_t launch_bwd_small_t(const Args &a) {
  const int ntiles = (a.S + 127) / 128;  // 128 keys per dK/dV workgroup, 128 queries per dQ workgroup
  const int n = a.B * a.H * ntiles;
  hipLaunchKernelGGL((attn_bwd_small_kernel<T, OT>), dim3(2 * n), dim3(256), 0, a.stream, static_cast<const T *>(a.q),
                     static_cast<const T *>(a.k), static_cast<const T *>(a.v), static_cast<const T *>(a.dO),
                     a.lse_in, a.delta_in, static_cast<OT *>(a.dq), static_cast<OT *>(a.dk), static_cast<OT *>(a.dv),
                     a.S, a.scale * kLog2e, a.scale, ntiles, a.H, a.rope, a.rope_npos, a.lq, a.lk, a.lv, a.ldo,
                     a.ldq, a.ldk, a.ldv, n);
  return hipGetLastError();
}

// Delta by the preprocess kernel, then attn_bwd_small_kernel.
hipError_t launch_bwd_small(const Args &a) {
  hipError_t e = launch_bwd_preprocess(a);
  if (e != hipSuccess) return e;
  if (a.dtype == 1) return a.out16 ? launch_bwd_small_t<bf16, bf16>(a) : launch_bwd_small_t<bf16, float>(a);
  return a.out16 ? launch_bwd_small_t<f16, f16>(a) : launch_bwd_small_t<f16, float>(a);
}

hipError_t launch_bwd_dq(const Args &a) {
  switch (a.dtype) {
    case 1: return a.out16 ? launch_dq_dt<bf16, bf16, false>(a) : launch_dq_dt<bf16, float, false>(a);
    case 2: return a.out16 ? launch_dq_dt<f16, f16, false>(a) : launch_dq_dt<f16, float, false>(a);
    default: return launch_dq_dt<float, float, false>(a);
  }
}

hipError_t launch_bwd_dq_delta(const Args &a) {
  switch (a.dtype) {
    case 1: return a.out16 ? launch_dq_dt<bf16, bf16, true>(a) : launch_dq_dt<bf16, float, true>(a);
    case 2: return a.out16 ? launch_dq_dt<f16, f16, true>(a) : launch_dq_dt<f16, float, true>(a);
    default: return hipErrorInvalidValue;  // Delta fusion follows the 16-bit preprocess layout
  }
}

}  // namespace attn
