// attn_rope.hip - rotary position embedding (RoPE) of queries and keys.
//
// RoFormer's rotation (Su et al. 2021, which ARK cites; ARK's model applies it
// from precomputed sine/cosine tables, Forge's attention takes it with
// grouped-query heads): pair i = (x_2i, x_2i+1) of a row at position p turns
// by the angle p * theta_i, theta_i = base^(-2i/D).  Positions count from 0
// at the start of each sequence, or of each document in packed mode.
//
//  * attn_rope_table_kernel fills the table tab[p][i] = (cos, sin)(p theta_i),
//    fp32 [n_pos][D/2][2], from angles computed in double precision.
//  * attn_rope_kernel rotates every row of q and k once, into q_rot and k_rot
//    in the input dtype (fp32 arithmetic, one rounding).  It is a streaming,
//    HBM-bound pass: attention tiles reach LDS by direct global->LDS copies
//    that cannot transform data, and each key tile is read by many query
//    workgroups, so rotating once beats rotating on every load; q_rot and
//    k_rot are what the backward reads.  A thread owns 8 consecutive elements
//    (4 pairs) of one position in four heads: its 32 bytes of table are read
//    once for the four 16-byte (16-bit inputs) loads.
//  * The backward turns dQ and dK back in the epilogues of the dQ and dK/dV
//    kernels (attn_bwd.hip), where every lane holds both elements of its pairs.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

__global__ __launch_bounds__(256) void attn_rope_table_kernel(float *__restrict__ tab, int n_pos, int half,
                                                              double base) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n_pos * half) return;
  const int p = (int)(idx / half);
  const int i = (int)(idx % half);
  const double theta = pow(base, -(double)i / (double)half);  // base^(-2i/D)
  double s, c;
  sincos((double)p * theta, &s, &c);
  tab[2 * idx] = (float)c;
  tab[2 * idx + 1] = (float)s;
}

// Eight elements of a row as fp32, and back (round to nearest even).
template <typename T> struct Row8 {
  __device__ __forceinline__ static void load(const T *p, float (&x)[8]) {
    const typename Elem<T>::frag v = *reinterpret_cast<const typename Elem<T>::frag *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  }
  __device__ __forceinline__ static void store(T *p, const float (&x)[8]) {
    typename Elem<T>::frag v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (T)x[i];
    *reinterpret_cast<typename Elem<T>::frag *>(p) = v;
  }
};
template <> struct Row8<float> {
  __device__ __forceinline__ static void load(const float *p, float (&x)[8]) {
    const f32x4 a = reinterpret_cast<const f32x4 *>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4 *>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
  __device__ __forceinline__ static void store(float *p, const float (&x)[8]) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = x[i];
      b[i] = x[4 + i];
    }
    reinterpret_cast<f32x4 *>(p)[0] = a;
    reinterpret_cast<f32x4 *>(p)[1] = b;
  }
};

// Grid (flat): position block fastest, then batch entry, then group of HPT heads.  A thread owns one
// 8-element chunk of one position and rotates it in HPT heads (query heads
// 0 .. H-1, then key heads H .. H+H_kv-1): the chunk's table values are read
// once and the HPT loads are in flight together.  q_rot and k_rot are
// contiguous; with contiguous q and k they may be q and k themselves (each
// thread reads its elements before writing them), so no restrict.
template <typename T, int D, bool DOC, int HPT>
__global__ __launch_bounds__(256) void attn_rope_kernel(const T *q, const T *k, T *qr, T *kr,
                                                        const float *__restrict__ tab, int n_pos, int H, int Hkv,
                                                        int B, int S, int nsb, const int32_t *__restrict__ cu,
                                                        int n_seqs, Layout lq, Layout lk) {
  constexpr int CPR = D / 8;  // 8-element chunks per row
  const int pb = blockIdx.x % nsb;
  const int b = (blockIdx.x / nsb) % B;
  const int h0 = (int)(blockIdx.x / nsb / B) * HPT;
  const int idx = pb * 256 + threadIdx.x;
  if (idx >= S * CPR) return;
  const int s = idx / CPR;
  const int ch = idx % CPR;
  int pos = s;
  if constexpr (DOC) {  // the document holding s: cu[lo] <= s < cu[hi]
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (cu[mid] <= s)
        lo = mid;
      else
        hi = mid;
    }
    pos = min(s - cu[lo], n_pos - 1);  // a document past max_seqlen breaks the call's contract:
  }                                    // keep its reads inside the table
  const f32x4 *t4 = reinterpret_cast<const f32x4 *>(tab + (size_t)pos * D + ch * 8);
  const f32x4 cs0 = t4[0], cs1 = t4[1];  // (cos, sin) of this chunk's four pairs

  auto src = [&](int h) -> const T * {  // this chunk of head h's row s (q and k may be strided views)
    return h < H ? q + panel_off(lq, b, h) + (size_t)s * lq.ss + ch * 8
                 : k + panel_off(lk, b, h - H) + (size_t)s * lk.ss + ch * 8;
  };
  auto dst = [&](int h) -> T * {  // q_rot and k_rot are contiguous
    return h < H ? qr + ((size_t)(b * H + h) * S + s) * D + ch * 8 : kr + ((size_t)(b * Hkv + h - H) * S + s) * D + ch * 8;
  };
  float x[HPT][8];
#pragma unroll
  for (int j = 0; j < HPT; ++j)
    if (h0 + j < H + Hkv) Row8<T>::load(src(h0 + j), x[j]);
#pragma unroll
  for (int j = 0; j < HPT; ++j) {
    if (h0 + j >= H + Hkv) break;
    float y[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float c = p < 2 ? cs0[2 * p] : cs1[2 * p - 4];
      const float sn = p < 2 ? cs0[2 * p + 1] : cs1[2 * p - 3];
      y[2 * p] = x[j][2 * p] * c - x[j][2 * p + 1] * sn;
      y[2 * p + 1] = x[j][2 * p] * sn + x[j][2 * p + 1] * c;
    }
    Row8<T>::store(dst(h0 + j), y);
  }
}

hipError_t launch_rope_table(float *tab, int n_pos, int D, double base, hipStream_t stream) {
  const int half = D / 2;
  const int64_t n = (int64_t)n_pos * half;
  hipLaunchKernelGGL(attn_rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, tab, n_pos,
                     half, base);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_rope_t(const Args &a, void *q_rot, void *k_rot) {
  constexpr int HPT = 4;
  const int nsb = (a.S * (D / 8) + 255) / 256;
  const dim3 grid((unsigned)nsb * a.B * ((a.H + a.H_kv + HPT - 1) / HPT));
  const T *q = static_cast<const T *>(a.q);
  const T *k = static_cast<const T *>(a.k);
  T *qr = static_cast<T *>(q_rot);
  T *kr = static_cast<T *>(k_rot);
  if (a.doc)
    hipLaunchKernelGGL((attn_rope_kernel<T, D, true, HPT>), grid, dim3(256), 0, a.stream, q, k, qr, kr, a.rope,
                       a.rope_npos, a.H, a.H_kv, a.B, a.S, nsb, a.cu_seqlens, a.n_seqs, a.lq, a.lk);
  else
    hipLaunchKernelGGL((attn_rope_kernel<T, D, false, HPT>), grid, dim3(256), 0, a.stream, q, k, qr, kr, a.rope,
                       a.rope_npos, a.H, a.H_kv, a.B, a.S, nsb, a.cu_seqlens, a.n_seqs, a.lq, a.lk);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_rope_dt(const Args &a, void *q_rot, void *k_rot) {
  switch (a.D) {
    case 32: return launch_rope_t<T, 32>(a, q_rot, k_rot);
    case 64: return launch_rope_t<T, 64>(a, q_rot, k_rot);
    default: return launch_rope_t<T, 128>(a, q_rot, k_rot);
  }
}

hipError_t launch_rope(const Args &a, void *q_rot, void *k_rot) {
  switch (a.dtype) {
    case 1: return launch_rope_dt<bf16>(a, q_rot, k_rot);
    case 2: return launch_rope_dt<f16>(a, q_rot, k_rot);
    default: return launch_rope_dt<float>(a, q_rot, k_rot);
  }
}

}  // namespace attn
