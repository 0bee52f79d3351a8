// attn_api.hip - the C ABI (include/attn_api.h): argument checks and launches.
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, then enqueues the kernels on the caller's stream and returns.
// Nothing here allocates, frees, copies or synchronises.
#include <cmath>
#include <cstdint>

#include "attn_api.h"
#include "attn_launch.h"

namespace attn {

// One wave: shader-clock cycles (s_memtime) and 100 MHz real-time ticks
// (s_memrealtime) over at least `ticks` real-time ticks, sleeping between
// reads; at most 2^24 reads, so it always ends.
__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long *out, unsigned long long ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r = r0;
  for (int it = 0; it < (1 << 24) && r - r0 < ticks; ++it) {
    __builtin_amdgcn_s_sleep(8);
    r = __builtin_amdgcn_s_memrealtime();
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r - r0;
  }
}

hipError_t launch_clock_probe(unsigned long long *out, unsigned long long ticks, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, ticks);
  return hipGetLastError();
}

}  // namespace attn

namespace {

constexpr int kAbiVersion = 192;  // 1.92: attn_params.workspace; 1.91: grouped-head backward with a workspace; 1.90: clock probe; grouped-query, decode, RoPE, fp16 inputs, attn_params calls (16-bit outputs,
                                  // strides), the fused dQ + Delta stage, the build identifier, decode without allocation

#ifndef ATTN_SOURCE_DIGEST
#error "build with -DATTN_SOURCE_DIGEST=... (causal_attention_amd/build.py computes it from the sources)"
#endif

int check_common(int B, int H, int S, int D, int dtype) {
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_DTYPE;
  if (D != 32 && D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (B < 1 || H < 1 || S < 1) return ATTN_ERR_SHAPE;
  const int64_t elems = (int64_t)B * H * S * D;
  if (elems >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  // one head's fp32 output must be addressable with 32-bit byte offsets
  if ((int64_t)S * D * 4 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

int check_mask(int B, int H, int S, int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen) {
  if (mask_mode == ATTN_MASK_CAUSAL) return ATTN_OK;
  if (mask_mode != ATTN_MASK_DOC_CAUSAL) return ATTN_ERR_MASK;
  if (cu_seqlens == nullptr) return ATTN_ERR_NULL;
  // empty documents are allowed, so n_seqs may exceed S
  if (B != 1 || n_seqs < 1) return ATTN_ERR_SEQLENS;
  if (max_seqlen < 1 || max_seqlen > S) return ATTN_ERR_SEQLENS;
  // a launch has one workgroup per (tile of the longest document, document,
  // head), with tiles of 64 rows at the finest (the backward's 64-key
  // workgroups)
  if ((int64_t)((max_seqlen + 63) / 64) * n_seqs * H >= ((int64_t)1 << 31)) return ATTN_ERR_SEQLENS;
  return ATTN_OK;
}

int check_heads(int H, int H_kv) {
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return ATTN_ERR_HEADS;
  return ATTN_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

// The RoPE table must cover every position: sequence indices (causal) or
// offsets inside the longest document.
int check_rope(const float *tab, int n_pos, int S, int mask_mode, int max_seqlen) {
  if (tab == nullptr) return ATTN_ERR_ROPE;
  const int need = mask_mode == ATTN_MASK_DOC_CAUSAL ? max_seqlen : S;
  if (n_pos < need) return ATTN_ERR_ROPE;
  return ATTN_OK;
}

// Outputs are fp32, or 16-bit in the (16-bit) input dtype.
int check_out(int dtype, int out_dtype) {
  if (out_dtype == ATTN_DTYPE_F32) return ATTN_OK;
  if (out_dtype == dtype && dtype != ATTN_DTYPE_F32) return ATTN_OK;
  return ATTN_ERR_DTYPE;
}

// Caller strides (attn_params.strides, NULL for the contiguous layout): each
// given row needs non-negative batch and head strides, rows at least D
// apart, and a panel (plus tile overhang) within 32-bit byte offsets.
int check_strides(const int64_t (*st)[3], int S, int D, int in_bytes, int out_bytes) {
  if (st == nullptr) return ATTN_OK;
  for (int i = 0; i < 8; ++i) {
    if (st[i][0] == 0 && st[i][1] == 0 && st[i][2] == 0) continue;
    const int esize = (i == ATTN_STRIDE_O || i >= ATTN_STRIDE_DQ) ? out_bytes : in_bytes;
    if (st[i][0] < 0 || st[i][1] < 0 || st[i][2] < D) return ATTN_ERR_STRIDE;
    if (st[i][2] >= ((int64_t)1 << 31)) return ATTN_ERR_STRIDE;
    // kernels form row offsets up to 255 rows past the end (tile overhang, read
    // as zeros by the range check): those must not wrap 32 bits either
    if (((int64_t)(S + 255) * st[i][2] + D) * esize >= ((int64_t)1 << 31)) return ATTN_ERR_STRIDE;
  }
  return ATTN_OK;
}

int elem_bytes(int dtype) { return dtype == ATTN_DTYPE_F32 ? 4 : 2; }

// Contiguous layouts for every tensor, then the caller's strides where given.
void set_layouts(attn::Args &a, const int64_t (*st)[3]) {
  a.contiguous();
  if (st == nullptr) return;
  attn::Layout *dst[8] = {&a.lq, &a.lk, &a.lv, &a.lo, &a.ldo, &a.ldq, &a.ldk, &a.ldv};
  for (int i = 0; i < 8; ++i)
    if (st[i][0] != 0 || st[i][1] != 0 || st[i][2] != 0) *dst[i] = attn::Layout{st[i][0], st[i][1], (int)st[i][2]};
}

attn::Args make_args(int B, int H, int S, int D, float scale, int mask_mode, const int32_t *cu_seqlens,
                     int n_seqs, int max_seqlen, int dtype, void *stream) {
  attn::Args a{};
  a.B = B;
  a.H = H;
  a.H_kv = H;
  a.S = S;
  a.D = D;
  a.scale = scale;
  a.doc = mask_mode == ATTN_MASK_DOC_CAUSAL;
  a.cu_seqlens = cu_seqlens;
  a.n_seqs = n_seqs;
  a.max_seqlen = max_seqlen;
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  a.contiguous();
  return a;
}

int to_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Whole forward (optionally rotating q and k first): argument checks, then
// the kernels on one stream.
int fwd_all(const void *q, const void *k, const void *v, void *o, float *lse, bool with_rope,
                   const float *rope, int rope_npos, void *q_rot, void *k_rot, int B, int H, int H_kv, int S, int D,
                   float scale, int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype,
                   int out_dtype, const int64_t (*strides)[3], void *stream) {
  int st = check_common(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if ((st = check_out(dtype, out_dtype)) != ATTN_OK) return st;
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (with_rope && (!q_rot || !k_rot)) return ATTN_ERR_NULL;
  if ((st = check_mask(B, H, S, mask_mode, cu_seqlens, n_seqs, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  if (with_rope && (st = check_rope(rope, rope_npos, S, mask_mode, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_strides(strides, S, D, elem_bytes(dtype), elem_bytes(out_dtype))) != ATTN_OK) return st;
  attn::Args a = make_args(B, H, S, D, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype, stream);
  a.H_kv = H_kv;
  a.out16 = out_dtype != ATTN_DTYPE_F32;
  set_layouts(a, strides);
  a.q = q;
  a.k = k;
  if (with_rope) {
    a.rope = rope;
    a.rope_npos = rope_npos;
    if (attn::launch_rope(a, q_rot, k_rot) != hipSuccess) return ATTN_ERR_HIP;
    a.q = q_rot;  // contiguous from here on
    a.k = k_rot;
    const attn::Layout lv = a.lv, lo = a.lo;
    a.contiguous();
    a.lv = lv;
    a.lo = lo;
  }
  a.v = v;
  a.o = o;
  a.lse = lse;
  return to_status(attn::launch_fwd(a));
}

// Delta and dQ.  16-bit inputs: the dQ kernel computes Delta on the way
// (bitwise equal to the preprocess kernel's) and writes it for dK/dV, one pass
// over O and dO fewer; fp32 inputs: the preprocess kernel, then dQ.
hipError_t dq_delta_stage(const attn::Args &a) {
  if (a.half()) return attn::launch_bwd_dq_delta(a);
  hipError_t e = attn::launch_bwd_preprocess(a);
  if (e == hipSuccess) e = attn::launch_bwd_dq(a);
  return e;
}

// Whole backward (optionally with RoPE gradients turned back in the dQ and dK
// epilogues): argument checks, then the kernels on one stream.
// with_ws: the caller passed a workspace (attn_bwd_gqa_ws), which the
// grouped-head parts path uses where it applies (attn::dkdv_parts).
int bwd_all(const void *q, const void *k, const void *v, const void *o, const void *dO, const float *lse,
                   void *dq, void *dk, void *dv, float *delta, bool with_rope, const float *rope, int rope_npos,
                   int B, int H, int H_kv, int S, int D, float scale, int mask_mode, const int32_t *cu_seqlens,
                   int n_seqs, int max_seqlen, int dtype, int out_dtype, const int64_t (*strides)[3],
                   void *stream, bool with_ws = false, void *ws = nullptr, size_t ws_bytes = 0) {
  int st = check_common(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if ((st = check_out(dtype, out_dtype)) != ATTN_OK) return st;
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv || !delta) return ATTN_ERR_NULL;
  if ((st = check_mask(B, H, S, mask_mode, cu_seqlens, n_seqs, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  if (with_rope && (st = check_rope(rope, rope_npos, S, mask_mode, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_strides(strides, S, D, elem_bytes(dtype), elem_bytes(out_dtype))) != ATTN_OK) return st;
  attn::Args a = make_args(B, H, S, D, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype, stream);
  a.H_kv = H_kv;
  a.out16 = out_dtype != ATTN_DTYPE_F32;
  set_layouts(a, strides);
  if (with_rope) {  // the kernels read the contiguous q_rot and k_rot
    a.lq = attn::Layout{(int64_t)H * S * D, (int64_t)S * D, D};
    a.lk = attn::Layout{(int64_t)H_kv * S * D, (int64_t)S * D, D};
  }
  a.rope = rope;
  a.rope_npos = rope_npos;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.o_in = o;
  a.lse_in = lse;
  a.delta = delta;
  a.delta_in = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  const size_t need = with_ws ? attn::dkdv_workspace_bytes(a) : 0;
  if (need > 0 && (ws == nullptr || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 16 != 0))
    return ATTN_ERR_WORKSPACE;
  if (need == 0 && attn::bwd_small_applies(a)) return to_status(attn::launch_bwd_small(a));
  hipError_t e = dq_delta_stage(a);
  if (e == hipSuccess) e = need > 0 ? attn::launch_bwd_dkdv_parts(a, static_cast<float *>(ws)) : attn::launch_bwd_dkdv(a);
  return to_status(e);
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return kAbiVersion; }

const char *attn_build_id(void) { return ATTN_SOURCE_DIGEST; }

int attn_clock_probe(unsigned long long *out, unsigned long long ticks, void *stream) {
  if (out == nullptr) return ATTN_ERR_NULL;
  if (ticks == 0) return ATTN_ERR_SHAPE;
  return to_status(attn::launch_clock_probe(out, ticks, static_cast<hipStream_t>(stream)));
}

const char *attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H or S out of range (each >= 1, B*H*S*D < 2^31)";
    case ATTN_ERR_HEAD_DIM: return "head dimension D must be 32, 64 or 128";
    case ATTN_ERR_DTYPE: return "unknown input dtype (ATTN_DTYPE_F32, ATTN_DTYPE_BF16 or ATTN_DTYPE_F16)";
    case ATTN_ERR_MASK: return "unknown mask mode (ATTN_MASK_CAUSAL or ATTN_MASK_DOC_CAUSAL)";
    case ATTN_ERR_SEQLENS: return "packed-document mode needs B == 1, n_seqs >= 1, 1 <= max_seqlen <= S and ceil(max_seqlen/64)*n_seqs*H < 2^31";
    case ATTN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case ATTN_ERR_UNIMPLEMENTED: return "valid request that this library does not implement";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_HEADS: return "H_kv must divide H (1 <= H_kv <= H)";
    case ATTN_ERR_WORKSPACE: return "workspace NULL, not 16-byte aligned, or smaller than its *_workspace_bytes() size";
    case ATTN_ERR_ROPE: return "RoPE table NULL or shorter than the positions (S, or max_seqlen for documents), or base not finite and > 0";
    case ATTN_ERR_STRIDE: return "strides: batch and head >= 0, sequence >= D, panel extent < 2^31 bytes";
    case ATTN_ERR_SCRATCH: return "attn_decode_noalloc: the key split needs more than ATTN_DECODE_SCRATCH_BYTES (16 MiB) of partials; use attn_decode with a workspace";
    default: return "unknown status";
  }
}

int attn_fwd_gqa(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H, int H_kv, int S,
                 int D, float scale, int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype,
                 void *stream) {
  return fwd_all(q, k, v, o, lse, false, nullptr, 0, nullptr, nullptr, B, H, H_kv, S, D, scale, mask_mode,
                 cu_seqlens, n_seqs, max_seqlen, dtype, ATTN_DTYPE_F32, nullptr, stream);
}

int attn_fwd(const void *q, const void *k, const void *v, float *o, float *lse, int B, int H, int S, int D,
             float scale, int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype,
             void *stream) {
  return attn_fwd_gqa(q, k, v, o, lse, B, H, H, S, D, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype,
                      stream);
}

int attn_bwd_preprocess(const float *o, const void *dO, float *delta, int B, int H, int S, int D, int dtype,
                        void *stream) {
  int st = check_common(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if (!o || !dO || !delta) return ATTN_ERR_NULL;
  attn::Args a = make_args(B, H, S, D, 1.f, ATTN_MASK_CAUSAL, nullptr, 0, 0, dtype, stream);
  a.o_in = o;
  a.dO = dO;
  a.delta = delta;
  return to_status(attn::launch_bwd_preprocess(a));
}

int attn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dO, const float *lse,
                  const float *delta, float *dk, float *dv, int B, int H, int S, int D, float scale, int mask_mode,
                  const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype, void *stream) {
  int st = check_common(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if (!q || !k || !v || !dO || !lse || !delta || !dk || !dv) return ATTN_ERR_NULL;
  if ((st = check_mask(B, H, S, mask_mode, cu_seqlens, n_seqs, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  attn::Args a = make_args(B, H, S, D, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype, stream);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.lse_in = lse;
  a.delta_in = delta;
  a.dk = dk;
  a.dv = dv;
  return to_status(attn::launch_bwd_dkdv(a));
}

int attn_bwd_dq(const void *q, const void *k, const void *v, const void *dO, const float *lse, const float *delta,
                float *dq, int B, int H, int S, int D, float scale, int mask_mode, const int32_t *cu_seqlens,
                int n_seqs, int max_seqlen, int dtype, void *stream) {
  int st = check_common(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if (!q || !k || !v || !dO || !lse || !delta || !dq) return ATTN_ERR_NULL;
  if ((st = check_mask(B, H, S, mask_mode, cu_seqlens, n_seqs, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  attn::Args a = make_args(B, H, S, D, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype, stream);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.lse_in = lse;
  a.delta_in = delta;
  a.dq = dq;
  return to_status(attn::launch_bwd_dq(a));
}

int attn_bwd_dq_delta(const void *q, const void *k, const void *v, const float *o, const void *dO,
                      const float *lse, float *dq, float *delta, int B, int H, int S, int D, float scale,
                      int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype,
                      void *stream) {
  int st = check_common(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !delta) return ATTN_ERR_NULL;
  if ((st = check_mask(B, H, S, mask_mode, cu_seqlens, n_seqs, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  attn::Args a = make_args(B, H, S, D, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype, stream);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dO = dO;
  a.o_in = o;
  a.lse_in = lse;
  a.delta = delta;
  a.delta_in = delta;
  a.dq = dq;
  return to_status(dq_delta_stage(a));
}

int attn_bwd_gqa(const void *q, const void *k, const void *v, const float *o, const void *dO, const float *lse,
                 float *dq, float *dk, float *dv, float *delta, int B, int H, int H_kv, int S, int D, float scale,
                 int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype, void *stream) {
  return bwd_all(q, k, v, o, dO, lse, dq, dk, dv, delta, false, nullptr, 0, B, H, H_kv, S, D, scale, mask_mode,
                 cu_seqlens, n_seqs, max_seqlen, dtype, ATTN_DTYPE_F32, nullptr, stream);
}

size_t attn_bwd_gqa_workspace_bytes(int B, int H, int H_kv, int S, int D, int mask_mode, int n_seqs,
                                     int max_seqlen, int dtype) {
  // invalid arguments need nothing here: attn_bwd_gqa_ws reports them
  static const int32_t any_cu = 0;  // check_mask only tests the pointer
  if (check_common(B, H, S, D, dtype) != ATTN_OK || check_heads(H, H_kv) != ATTN_OK) return 0;
  if (check_mask(B, H, S, mask_mode, &any_cu, n_seqs, max_seqlen) != ATTN_OK) return 0;
  attn::Args a = make_args(B, H, S, D, 1.f, mask_mode, nullptr, n_seqs, max_seqlen, dtype, nullptr);
  a.H_kv = H_kv;
  return attn::dkdv_workspace_bytes(a);
}

int attn_bwd_gqa_ws(const void *q, const void *k, const void *v, const float *o, const void *dO, const float *lse,
                    float *dq, float *dk, float *dv, float *delta, int B, int H, int H_kv, int S, int D, float scale,
                    int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_all(q, k, v, o, dO, lse, dq, dk, dv, delta, false, nullptr, 0, B, H, H_kv, S, D, scale, mask_mode,
                 cu_seqlens, n_seqs, max_seqlen, dtype, ATTN_DTYPE_F32, nullptr, stream, true, workspace,
                 workspace_bytes);
}

int attn_bwd(const void *q, const void *k, const void *v, const float *o, const void *dO, const float *lse,
             float *dq, float *dk, float *dv, float *delta, int B, int H, int S, int D, float scale, int mask_mode,
             const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype, void *stream) {
  return attn_bwd_gqa(q, k, v, o, dO, lse, dq, dk, dv, delta, B, H, H, S, D, scale, mask_mode, cu_seqlens, n_seqs,
                      max_seqlen, dtype, stream);
}

int attn_rope_table(float *tab, int n_pos, int D, float base, void *stream) {
  if (D != 32 && D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (n_pos < 1 || (int64_t)n_pos * D >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  if (tab == nullptr) return ATTN_ERR_NULL;
  if (!std::isfinite(base) || !(base > 0.f)) return ATTN_ERR_ROPE;
  return to_status(attn::launch_rope_table(tab, n_pos, D, (double)base, static_cast<hipStream_t>(stream)));
}

int attn_rope(const void *q, const void *k, void *q_rot, void *k_rot, const float *tab, int n_pos, int B, int H,
              int H_kv, int S, int D, int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype,
              void *stream) {
  int st = check_common(B, H, S, D, dtype);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (!q || !k || !q_rot || !k_rot) return ATTN_ERR_NULL;
  if ((st = check_mask(B, H, S, mask_mode, cu_seqlens, n_seqs, max_seqlen)) != ATTN_OK) return st;
  if ((st = check_rope(tab, n_pos, S, mask_mode, max_seqlen)) != ATTN_OK) return st;
  attn::Args a = make_args(B, H, S, D, 1.f, mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype, stream);
  a.H_kv = H_kv;
  a.contiguous();
  a.q = q;
  a.k = k;
  a.rope = tab;
  a.rope_npos = n_pos;
  return to_status(attn::launch_rope(a, q_rot, k_rot));
}

int attn_fwd_rope(const void *q, const void *k, const void *v, void *q_rot, void *k_rot, float *o, float *lse,
                  const float *tab, int n_pos, int B, int H, int H_kv, int S, int D, float scale, int mask_mode,
                  const int32_t *cu_seqlens, int n_seqs, int max_seqlen, int dtype, void *stream) {
  return fwd_all(q, k, v, o, lse, true, tab, n_pos, q_rot, k_rot, B, H, H_kv, S, D, scale, mask_mode, cu_seqlens,
                 n_seqs, max_seqlen, dtype, ATTN_DTYPE_F32, nullptr, stream);
}

int attn_bwd_rope(const void *q_rot, const void *k_rot, const void *v, const float *o, const void *dO,
                  const float *lse, float *dq, float *dk, float *dv, float *delta, const float *tab, int n_pos, int B,
                  int H, int H_kv, int S, int D, float scale, int mask_mode, const int32_t *cu_seqlens, int n_seqs,
                  int max_seqlen, int dtype, void *stream) {
  return bwd_all(q_rot, k_rot, v, o, dO, lse, dq, dk, dv, delta, true, tab, n_pos, B, H, H_kv, S, D, scale,
                 mask_mode, cu_seqlens, n_seqs, max_seqlen, dtype, ATTN_DTYPE_F32, nullptr, stream);
}

int attn_fwd_ex(const attn_params *p, void *stream) {
  if (p == nullptr) return ATTN_ERR_NULL;
  const int H_kv = p->H_kv == 0 ? p->H : p->H_kv;
  const bool rope = p->rope_table != nullptr;
  return fwd_all(p->q, p->k, p->v, p->o, p->lse, rope, p->rope_table, p->rope_npos, p->q_rot, p->k_rot, p->B, p->H,
                 H_kv, p->S, p->D, p->scale, p->mask_mode, p->cu_seqlens, p->n_seqs, p->max_seqlen, p->dtype,
                 p->out_dtype, p->strides, stream);
}

int attn_bwd_ex(const attn_params *p, void *stream) {
  if (p == nullptr) return ATTN_ERR_NULL;
  const int H_kv = p->H_kv == 0 ? p->H : p->H_kv;
  const bool rope = p->rope_table != nullptr;
  // a workspace, when given, lets grouped heads split their dK/dV step (as attn_bwd_gqa_ws)
  return bwd_all(rope ? p->q_rot : p->q, rope ? p->k_rot : p->k, p->v, p->o, p->dO, p->lse, p->dq, p->dk, p->dv,
                 p->delta, rope, p->rope_table, p->rope_npos, p->B, p->H, H_kv, p->S, p->D, p->scale, p->mask_mode,
                 p->cu_seqlens, p->n_seqs, p->max_seqlen, p->dtype, p->out_dtype, p->strides, stream,
                 p->workspace != nullptr, p->workspace, p->workspace_bytes);
}

size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int D, int max_len) {
  if (B < 1 || H < 1 || H_kv < 1 || max_len < 1) return 0;
  return attn::decode_workspace_bytes(B, H, H_kv, D, max_len);
}

}  // extern "C"

namespace {

// Checks shared by the decode entry points; fills `a` on success.
int decode_args(const void *q, const void *k_cache, const void *v_cache, const int32_t *cache_lens, float *o,
                float *lse, int B, int H, int H_kv, int S_max, int D, float scale, int max_len, int dtype,
                void *stream, attn::DecodeArgs &a) {
  int st = check_common(B, H, S_max, D, dtype);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, H_kv)) != ATTN_OK) return st;
  if (H / H_kv > 32) return ATTN_ERR_UNIMPLEMENTED;  // one wave holds a group's queries
  if ((int64_t)B * H_kv * S_max * D >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
  if (max_len < 1 || max_len > S_max) return ATTN_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !cache_lens || !o) return ATTN_ERR_NULL;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  a = attn::DecodeArgs{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_lens = cache_lens;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.H_kv = H_kv;
  a.S_max = S_max;
  a.D = D;
  a.max_len = max_len;
  a.scale = scale;
  a.dtype = dtype;
  a.stream = static_cast<hipStream_t>(stream);
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *cache_lens, float *o,
                float *lse, void *workspace, size_t workspace_bytes, int B, int H, int H_kv, int S_max, int D,
                float scale, int max_len, int dtype, void *stream) {
  attn::DecodeArgs a;
  const int st = decode_args(q, k_cache, v_cache, cache_lens, o, lse, B, H, H_kv, S_max, D, scale, max_len, dtype,
                             stream, a);
  if (st != ATTN_OK) return st;
  const size_t need = attn::decode_workspace_bytes(B, H, H_kv, D, max_len);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  a.o_part = static_cast<float *>(workspace);
  a.lse_part = need > 0 ? static_cast<float *>(workspace) + (need / sizeof(float)) / (D + 1) * D : nullptr;
  return to_status(attn::launch_decode(a));
}

int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int32_t *cache_lens,
                        float *o, float *lse, int B, int H, int H_kv, int S_max, int D, float scale, int max_len,
                        int dtype, void *stream) {
  attn::DecodeArgs a;
  const int st = decode_args(q, k_cache, v_cache, cache_lens, o, lse, B, H, H_kv, S_max, D, scale, max_len, dtype,
                             stream, a);
  if (st != ATTN_OK) return st;
  if (attn::decode_workspace_bytes(B, H, H_kv, D, max_len) > attn::decode_scratch_bytes()) return ATTN_ERR_SCRATCH;
  return to_status(attn::launch_decode_noalloc(a));
}

}  // extern "C"
