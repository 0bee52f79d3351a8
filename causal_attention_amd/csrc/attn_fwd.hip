// attn_fwd.hip - forward kernel: O = softmax(scale * Q K^T + mask) V and the row LSE.
//
// Flash-attention forward (Forge, "What this is": fused forward written after
// FlashAttention-2, "Acknowledgements"): one workgroup owns BM query rows of
// one head and streams the key/value tiles up to its causal diagonal (keys of
// its document only, in packed mode), keeping per row a running maximum m,
// a running sum l and the unnormalised output; after the last tile
// O = acc / l and LSE = m + ln l.  Scores never leave registers.
//
// gfx950 mapping.  Each wave computes S^T = K Q^T for its 32*QB queries, so a
// lane owns one query (column) and holds that query's scores against 16 keys
// per 32-key block in its own registers: the row maximum and sum are in-lane
// except for one exchange between the two wave halves, and P^T is already
// the B operand of O^T += V^T P^T (the "accum" slot order, attn_device.h).
// K is staged row-major and V transposed in LDS; the next tile's global
// loads are in flight while the current tile is computed.  Softmax runs in
// base 2 with scale * log2(e) folded into one multiply.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

template <typename T, int D, int QB, int BN, bool DOC>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                       const T *__restrict__ v, float *__restrict__ o,
                                                       float *__restrict__ lse, int S, float c2,
                                                       const int32_t *__restrict__ cu, int ntiles) {
  constexpr int NW = 4;
  constexpr int NT = NW * kWaveSize;
  constexpr int BM = NW * 32 * QB;  // query rows per workgroup
  constexpr int KB = D / 16;        // k-blocks over the head dimension
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int NB = BN / 32;       // 32-key blocks per tile
  constexpr int PB = BN / 16;       // k-blocks over the keys of a tile
  using E = Elem<T>;
  using frag = typename E::frag;
  using G = TileGeom<T, BN, D>;
  using Loader = TileLoader<T, BN, D, NT>;

  __shared__ __attribute__((aligned(16))) T sK[G::kSizeRM];
  __shared__ __attribute__((aligned(16))) T sVt[G::kSizeTR];

  const RowTile t = DOC ? doc_tile(cu, blockIdx.x, gridDim.x, blockIdx.y, blockIdx.z, BM, true)
                        : causal_tile(blockIdx.x, gridDim.x, ntiles, BM, S, true);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  const size_t base = (size_t)t.head * S * D;
  // Resources end at the last valid row (queries) or key of the segment.
  const GBuf gq(q + base, (uint32_t)(t.r_end * D * sizeof(T)));
  const GBuf gk(k + base, (uint32_t)(t.seg_end * D * sizeof(T)));
  const GBuf gv(v + base, (uint32_t)(t.seg_end * D * sizeof(T)));

  const int w0 = t.r_start + wave * 32 * QB;  // first query of this wave
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32 * QB, t.r_end) - 1;

  frag qf[QB][KB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[qb][kb] = global_frag<T, D>(gq, w0 + 32 * qb + c, 16 * kb + 8 * hh);

  f32x16 oacc[QB][DB];
  float m[QB], l[QB];  // running max (scaled, base 2) and this lane-half's partial sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  }

  const int kv_lo = t.seg_start;
  const int kv_hi = min(t.r_end, t.seg_end);  // one past the last key any row here can see
  const int ntile = (kv_hi - kv_lo + BN - 1) / BN;

  Loader lk, lv;
  lk.load(gk, kv_lo, tid);
  lv.load(gv, kv_lo, tid);

  // One key tile for this wave.  MASK selects the diagonal / segment-end
  // variant; interior tiles take the branch-free path.
  auto tile = [&]<bool MASK>(int k0) {
    // S^T = K Q^T : rows are keys, columns (lanes) are queries.
    f32x16 sacc[QB][NB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[qb][nb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const frag a = lds_frag<T>(sK + (nb * 32 + c) * G::kLdRM + 16 * kb + 8 * hh);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) E::mma(sacc[qb][nb], a, qf[qb][kb]);
      }
    }

    // Online softmax in base 2: the maximum is taken on raw scores and the
    // scale folded into one multiply-add before each exp2.
    frag pf[QB][PB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = w0 + 32 * qb + c;
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (MASK) {
            const int key = k0 + 32 * nb + 8 * (r / 4) + 4 * hh + (r % 4);
            sacc[qb][nb][r] = (key > qi || key >= t.seg_end) ? -INFINITY : sacc[qb][nb][r];
          }
          mx = fmaxf(mx, sacc[qb][nb][r]);
        }
      }
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = fmaxf(m[qb], mx * c2);
      const float alpha = fast_exp2(m[qb] - mnew);
      m[qb] = mnew;
      float psum = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(sacc[qb][nb][r], c2, -mnew));
          sacc[qb][nb][r] = p;
          psum += p;
        }
      }
      l[qb] = l[qb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
#pragma unroll
      for (int j = 0; j < PB; ++j) pf[qb][j] = E::pack(sacc[qb][j / 2], j % 2);
    }

    // O^T += V^T P^T : rows are head dims, columns (lanes) are queries.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const frag a = lds_frag<T>(sVt + (db * 32 + c) * G::kLdTR + 16 * j + 8 * hh);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) E::mma(oacc[qb][db], a, pf[qb][j]);
      }
    }
  };

  for (int it = 0; it < ntile; ++it) {
    const int k0 = kv_lo + it * BN;
    __syncthreads();  // every wave is done with the previous tile
    lk.store_rm(sK, tid);
    lv.store_tr(sVt, tid);
    __syncthreads();
    if (it + 1 < ntile) {
      lk.load(gk, k0 + BN, tid);
      lv.load(gv, k0 + BN, tid);
    }
    if (!wave_active || k0 > wave_last) continue;  // tile entirely above this wave's diagonal
    if ((k0 + BN - 1 > w0) || (k0 + BN > t.seg_end))
      tile.template operator()<true>(k0);
    else
      tile.template operator()<false>(k0);
  }

  if (!wave_active) return;
  const GBuf go(o + base, (uint32_t)(t.r_end * D * sizeof(float)));
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = w0 + 32 * qb + c;
    const float lt = l[qb] + swap_halves(l[qb]);
    const float inv = 1.0f / lt;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 val;
#pragma unroll
        for (int i = 0; i < 4; ++i) val[i] = oacc[qb][db][4 * g + i] * inv;
        go.store16(val, (uint32_t)(qi * D + db * 32 + 8 * g + 4 * hh) * sizeof(float));
      }
    }
    if (lse != nullptr && hh == 0 && qi < t.r_end) lse[(size_t)t.head * S + qi] = (m[qb] + __log2f(lt)) * kLn2;
  }
}

// Tile shape per (dtype, D): queries per wave (32 * QB) and keys per tile (BN).
template <typename T, int D> struct FwdCfg {
  static constexpr int QB = 1;
  static constexpr int BN = 64;
};

template <typename T, int D, bool DOC>
static hipError_t launch_fwd_t(const Args &a) {
  constexpr int QB = FwdCfg<T, D>::QB;
  constexpr int BN = FwdCfg<T, D>::BN;
  constexpr int BM = 4 * 32 * QB;
  const float c2 = a.scale * kLog2e;
  dim3 block(256);
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BM - 1) / BM;
    grid = dim3(ntiles, a.n_seqs, a.H);
  } else {
    ntiles = (a.S + BM - 1) / BM;
    grid = dim3(ntiles * a.B * a.H);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, QB, BN, DOC>), grid, block, 0, a.stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     a.o, a.lse, a.S, c2, a.cu_seqlens, ntiles);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_fwd_d(const Args &a) {
  return a.doc ? launch_fwd_t<T, D, true>(a) : launch_fwd_t<T, D, false>(a);
}

template <typename T>
static hipError_t launch_fwd_dt(const Args &a) {
  switch (a.D) {
    case 32: return launch_fwd_d<T, 32>(a);
    case 64: return launch_fwd_d<T, 64>(a);
    default: return launch_fwd_d<T, 128>(a);
  }
}

hipError_t launch_fwd(const Args &a) { return a.bf16 ? launch_fwd_dt<bf16>(a) : launch_fwd_dt<float>(a); }

}  // namespace attn
