// attn_bwd.hip - backward kernels: Delta preprocess, dK/dV, dQ.
//
// The backward recomputes each probability tile from the stored row LSE
// instead of storing P (FlashAttention-2, which Forge's attention follows,
// "Acknowledgements"): P_ij = exp(S_ij - LSE_i).  With Delta_i = sum_d dO_id O_id,
// dS = P o (dO V^T - Delta), dV = P^T dO, dK = scale * dS^T Q, dQ = scale * dS K.
// Forge found its fused dK/dV backward limited by register spills and split
// it (Forge, finding 3, "Register pressure, not bandwidth, owns attention
// backward"); here dK/dV and dQ are separate kernels so neither needs
// atomics or a second pass over its outputs, and every output element has
// exactly one writer (results are bitwise reproducible run to run).
//
// gfx950 mapping, as in the forward: every contraction is 32x32x16 matrix-core
// steps with the reduction index of the second product held in the lane's
// own registers ("accum" order, attn_device.h), so P and dS feed the next
// product without leaving registers.
//   dK/dV: a lane owns one key.  S and dP are computed as [query][key]
//          blocks (Q and dO row fragments from LDS against K and V held in
//          registers), then dV^T += dO^T P and dK^T += Q^T dS with Q and dO
//          read from the same LDS tiles through the transposing load.
//   dQ:    a lane owns one query.  S^T and dP^T are [key][query] blocks (K
//          and V rows from LDS against Q and dO in registers), then
//          dQ^T += K^T dS^T with K read transposed from the same tile.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

// ---------------------------------------------------------------------------
// Delta_i = sum_d dO_id * O_id.  Memory bound: each group of D/VEC lanes reads
// one row of dO (input dtype) and O (fp32) with 16-byte loads and reduces
// across the group.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_bwd_preprocess_kernel(const float *__restrict__ o,
                                                                  const T *__restrict__ dO,
                                                                  float *__restrict__ delta, int rows) {
  constexpr int VEC = 16 / sizeof(T);  // dO elements per 16-byte load
  constexpr int LPR = D / VEC;         // lanes per row
  constexpr int RPB = 256 / LPR;       // rows per block per step
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  for (int row0 = blockIdx.x * RPB; row0 < rows; row0 += gridDim.x * RPB) {
    const int row = row0 + tid / LPR;
    float acc = 0.f;
    if (row < rows) {
      const T *dp = dO + (size_t)row * D + sub * VEC;
      const float *op = o + (size_t)row * D + sub * VEC;
      if constexpr (sizeof(T) == 2) {
        const bf16x8 g = *reinterpret_cast<const bf16x8 *>(dp);
        const f32x4 o0 = *reinterpret_cast<const f32x4 *>(op);
        const f32x4 o1 = *reinterpret_cast<const f32x4 *>(op + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += (float)g[i] * o0[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += (float)g[4 + i] * o1[i];
      } else {
        const f32x4 g = *reinterpret_cast<const f32x4 *>(dp);
        const f32x4 o0 = *reinterpret_cast<const f32x4 *>(op);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += g[i] * o0[i];
      }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off /= 2) acc += __shfl_xor(acc, off, kWaveSize);
    if (row < rows && sub == 0) delta[row] = acc;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  A workgroup owns BN = 4 * 32 * KBW keys of one head and loops over
// query tiles of BMQ rows from its first key to the end of the sequence (or
// document).
template <typename T, int D, int KBW, int BMQ, bool DOC>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, float *__restrict__ dk,
    float *__restrict__ dv, int S, float c2, float scale, const int32_t *__restrict__ cu, int ntiles) {
  constexpr int NW = 4;
  constexpr int NT = NW * kWaveSize;
  constexpr int BN = NW * 32 * KBW;  // keys per workgroup
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = BMQ / 32;       // 32-query blocks per tile
  constexpr int PB = BMQ / 16;       // k-blocks over the queries of a tile
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int LD = RowStride<T, D>::kPadded;  // read both as rows and transposed
  using Loader = TileLoader<T, BMQ, D, NT>;

  __shared__ __attribute__((aligned(16))) T sQ[BMQ * LD];
  __shared__ __attribute__((aligned(16))) T sdO[BMQ * LD];
  __shared__ __attribute__((aligned(16))) float sL[BMQ];  // LSE * log2(e); +inf past the end
  __shared__ __attribute__((aligned(16))) float sD[BMQ];  // Delta; 0 past the end

  const RowTile t = DOC ? doc_tile(cu, blockIdx.x, gridDim.x, blockIdx.y, blockIdx.z, BN, false)
                        : causal_tile(blockIdx.x, gridDim.x, ntiles, BN, S, false);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  const size_t base = (size_t)t.head * S * D;
  const size_t rbase = (size_t)t.head * S;
  const GBuf gq(q + base, (uint32_t)(t.seg_end * D * sizeof(T)));
  const GBuf gdo(dO + base, (uint32_t)(t.seg_end * D * sizeof(T)));
  const GBuf gk(k + base, (uint32_t)(t.r_end * D * sizeof(T)));
  const GBuf gv(v + base, (uint32_t)(t.r_end * D * sizeof(T)));
  const GBuf glse(lse + rbase, (uint32_t)(t.seg_end * sizeof(float)));
  const GBuf gdel(delta + rbase, (uint32_t)(t.seg_end * sizeof(float)));

  const int w0 = t.r_start + wave * 32 * KBW;  // first key of this wave
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32 * KBW, t.r_end) - 1;

  frag kf[KBW][KB], vf[KBW][KB];
#pragma unroll
  for (int kw = 0; kw < KBW; ++kw)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      kf[kw][kb] = global_frag<T, D>(gk, w0 + 32 * kw + c, 16 * kb + 8 * hh);
      vf[kw][kb] = global_frag<T, D>(gv, w0 + 32 * kw + c, 16 * kb + 8 * hh);
    }

  f32x16 dkacc[KBW][DB], dvacc[KBW][DB];
#pragma unroll
  for (int kw = 0; kw < KBW; ++kw)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      dkacc[kw][db] = f32x16{};
      dvacc[kw][db] = f32x16{};
    }

  const int q_lo = t.r_start;  // the first query that sees any of these keys
  const int q_hi = t.seg_end;
  const int ntile = (q_hi - q_lo + BMQ - 1) / BMQ;

  // Per-row statistics of the next query tile: LSE (to base 2) and Delta.
  float lval = 0.f, dval = 0.f;
  // Every thread loads (rows past the end read 0); threads tid < BMQ publish.
  auto load_stats = [&](int q0) {
    const int row = q0 + tid % BMQ;
    const float lv = glse.load4((uint32_t)row * 4);
    dval = gdel.load4((uint32_t)row * 4);
    lval = row < q_hi ? lv * kLog2e : INFINITY;
  };

  Loader lq, ldo;
  lq.load(gq, q_lo, tid);
  ldo.load(gdo, q_lo, tid);
  load_stats(q_lo);

  const TrRead<T, LD> trq(sQ, lane);
  const TrRead<T, LD> trdo(sdO, lane);

  auto tile = [&]<bool MASK>(int q0) {
    // S and dP as [query][key] blocks: lane c owns key w0 + 32*kw + c.
    f32x16 sacc[QB][KBW], pacc[QB][KBW];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kw = 0; kw < KBW; ++kw) {
        sacc[qb][kw] = f32x16{};
        pacc[qb][kw] = f32x16{};
      }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const frag aq = lds_frag<T>(sQ + (qb * 32 + c) * LD + 16 * kb + 8 * hh);
        const frag ad = lds_frag<T>(sdO + (qb * 32 + c) * LD + 16 * kb + 8 * hh);
#pragma unroll
        for (int kw = 0; kw < KBW; ++kw) {
          E::mma(sacc[qb][kw], aq, kf[kw][kb]);
          E::mma(pacc[qb][kw], ad, vf[kw][kb]);
        }
      }
    }

    // P = exp2(S * c2 - LSE2), dS = P (dP - Delta); packed as B operands whose
    // slots run over queries.
    frag pf[KBW][PB], sf[KBW][PB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4 lq4[4], dq4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        lq4[g] = *reinterpret_cast<const f32x4 *>(sL + qb * 32 + 8 * g + 4 * hh);
        dq4[g] = *reinterpret_cast<const f32x4 *>(sD + qb * 32 + 8 * g + 4 * hh);
      }
#pragma unroll
      for (int kw = 0; kw < KBW; ++kw) {
        const int key = w0 + 32 * kw + c;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(sacc[qb][kw][r], c2, -lq4[r / 4][r % 4]));
          if constexpr (MASK) {
            const int qi = q0 + qb * 32 + 8 * (r / 4) + 4 * hh + (r % 4);
            p = qi < key ? 0.f : p;
          }
          sacc[qb][kw][r] = p;
          pacc[qb][kw][r] = p * (pacc[qb][kw][r] - dq4[r / 4][r % 4]);
        }
        pf[kw][2 * qb] = E::pack(sacc[qb][kw], 0);
        pf[kw][2 * qb + 1] = E::pack(sacc[qb][kw], 1);
        sf[kw][2 * qb] = E::pack(pacc[qb][kw], 0);
        sf[kw][2 * qb + 1] = E::pack(pacc[qb][kw], 1);
      }
    }

    // dV^T += dO^T P,  dK^T += Q^T dS : rows are head dims, lanes are keys.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const frag ad = trdo(16 * j, 32 * db);
        const frag aq = trq(16 * j, 32 * db);
#pragma unroll
        for (int kw = 0; kw < KBW; ++kw) {
          E::mma(dvacc[kw][db], ad, pf[kw][j]);
          E::mma(dkacc[kw][db], aq, sf[kw][j]);
        }
      }
    }
  };

  for (int it = 0; it < ntile; ++it) {
    const int q0 = q_lo + it * BMQ;
    __syncthreads();
    lq.template store<LD>(sQ, tid);
    ldo.template store<LD>(sdO, tid);
    if (tid < BMQ) {
      sL[tid] = lval;
      sD[tid] = dval;
    }
    __syncthreads();
    if (it + 1 < ntile) {
      lq.load(gq, q0 + BMQ, tid);
      ldo.load(gdo, q0 + BMQ, tid);
      load_stats(q0 + BMQ);
    }
    if (!wave_active || q0 + BMQ - 1 < w0) continue;  // every query precedes every key here
    if (q0 < wave_last)
      tile.template operator()<true>(q0);
    else
      tile.template operator()<false>(q0);
  }

  if (!wave_active) return;
  const GBuf gdk(dk + base, (uint32_t)(t.r_end * D * sizeof(float)));
  const GBuf gdv(dv + base, (uint32_t)(t.r_end * D * sizeof(float)));
#pragma unroll
  for (int kw = 0; kw < KBW; ++kw) {
    const int key = w0 + 32 * kw + c;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a4, b4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a4[i] = dkacc[kw][db][4 * g + i] * scale;
          b4[i] = dvacc[kw][db][4 * g + i];
        }
        const uint32_t off = (uint32_t)(key * D + db * 32 + 8 * g + 4 * hh) * sizeof(float);
        gdk.store16(a4, off);
        gdv.store16(b4, off);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ.  A workgroup owns BM = 4 * 32 * QB queries of one head and loops over
// key tiles of BN rows up to its causal diagonal.
template <typename T, int D, int QB, int BN, bool DOC>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, float *__restrict__ dq, int S, float c2,
    float scale, const int32_t *__restrict__ cu, int ntiles) {
  constexpr int NW = 4;
  constexpr int NT = NW * kWaveSize;
  constexpr int BM = NW * 32 * QB;
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int NB = BN / 32;
  constexpr int PB = BN / 16;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int LD = RowStride<T, D>::kPadded;
  using Loader = TileLoader<T, BN, D, NT>;

  __shared__ __attribute__((aligned(16))) T sK[BN * LD];
  __shared__ __attribute__((aligned(16))) T sV[BN * LD];

  const RowTile t = DOC ? doc_tile(cu, blockIdx.x, gridDim.x, blockIdx.y, blockIdx.z, BM, true)
                        : causal_tile(blockIdx.x, gridDim.x, ntiles, BM, S, true);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  const size_t base = (size_t)t.head * S * D;
  const size_t rbase = (size_t)t.head * S;
  const GBuf gq(q + base, (uint32_t)(t.r_end * D * sizeof(T)));
  const GBuf gdo(dO + base, (uint32_t)(t.r_end * D * sizeof(T)));
  const GBuf gk(k + base, (uint32_t)(t.seg_end * D * sizeof(T)));
  const GBuf gv(v + base, (uint32_t)(t.seg_end * D * sizeof(T)));
  const GBuf glse(lse + rbase, (uint32_t)(t.r_end * sizeof(float)));
  const GBuf gdel(delta + rbase, (uint32_t)(t.r_end * sizeof(float)));

  const int w0 = t.r_start + wave * 32 * QB;
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32 * QB, t.r_end) - 1;

  frag qf[QB][KB], df[QB][KB];
  float l2[QB], dl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = w0 + 32 * qb + c;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qf[qb][kb] = global_frag<T, D>(gq, row, 16 * kb + 8 * hh);
      df[qb][kb] = global_frag<T, D>(gdo, row, 16 * kb + 8 * hh);
    }
    const float lv = glse.load4((uint32_t)row * 4);
    dl[qb] = gdel.load4((uint32_t)row * 4);
    l2[qb] = row < t.r_end ? lv * kLog2e : INFINITY;
  }

  f32x16 dqacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) dqacc[qb][db] = f32x16{};

  const int kv_lo = t.seg_start;
  const int kv_hi = min(t.r_end, t.seg_end);
  const int ntile = (kv_hi - kv_lo + BN - 1) / BN;

  Loader lk, lv;
  lk.load(gk, kv_lo, tid);
  lv.load(gv, kv_lo, tid);

  const TrRead<T, LD> trk(sK, lane);

  auto tile = [&]<bool MASK>(int k0) {
    // S^T = K Q^T and dP^T = V dO^T : rows are keys, lanes are queries.
    f32x16 sacc[QB][NB], pacc[QB][NB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sacc[qb][nb] = f32x16{};
        pacc[qb][nb] = f32x16{};
      }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const frag ak = lds_frag<T>(sK + (nb * 32 + c) * LD + 16 * kb + 8 * hh);
        const frag av = lds_frag<T>(sV + (nb * 32 + c) * LD + 16 * kb + 8 * hh);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          E::mma(sacc[qb][nb], ak, qf[qb][kb]);
          E::mma(pacc[qb][nb], av, df[qb][kb]);
        }
      }
    }

    frag sf[QB][PB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = w0 + 32 * qb + c;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(sacc[qb][nb][r], c2, -l2[qb]));
          if constexpr (MASK) {
            const int key = k0 + 32 * nb + 8 * (r / 4) + 4 * hh + (r % 4);
            p = (key > qi || key >= t.seg_end) ? 0.f : p;
          }
          pacc[qb][nb][r] = p * (pacc[qb][nb][r] - dl[qb]);
        }
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) sf[qb][j] = E::pack(pacc[qb][j / 2], j % 2);
    }

    // dQ^T += K^T dS^T : rows are head dims, lanes are queries.
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const frag a = trk(16 * j, 32 * db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) E::mma(dqacc[qb][db], a, sf[qb][j]);
      }
    }
  };

  for (int it = 0; it < ntile; ++it) {
    const int k0 = kv_lo + it * BN;
    __syncthreads();
    lk.template store<LD>(sK, tid);
    lv.template store<LD>(sV, tid);
    __syncthreads();
    if (it + 1 < ntile) {
      lk.load(gk, k0 + BN, tid);
      lv.load(gv, k0 + BN, tid);
    }
    if (!wave_active || k0 > wave_last) continue;
    if ((k0 + BN - 1 > w0) || (k0 + BN > t.seg_end))
      tile.template operator()<true>(k0);
    else
      tile.template operator()<false>(k0);
  }

  if (!wave_active) return;
  const GBuf gdq(dq + base, (uint32_t)(t.r_end * D * sizeof(float)));
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = w0 + 32 * qb + c;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a4;
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = dqacc[qb][db][4 * g + i] * scale;
        gdq.store16(a4, (uint32_t)(qi * D + db * 32 + 8 * g + 4 * hh) * sizeof(float));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.

#ifndef ATTN_DKDV_KBW
#define ATTN_DKDV_KBW 1
#endif
#ifndef ATTN_DKDV_BMQ
#define ATTN_DKDV_BMQ 64
#endif
#ifndef ATTN_DQ_QB
#define ATTN_DQ_QB 1
#endif
#ifndef ATTN_DQ_BN
#define ATTN_DQ_BN 64
#endif
template <typename T, int D> struct BwdCfg {
  static constexpr int KBW = (D == 128 || sizeof(T) == 4) ? 1 : ATTN_DKDV_KBW;  // key blocks per wave (dK/dV)
  static constexpr int BMQ = (D == 128 || sizeof(T) == 4) ? 32 : ATTN_DKDV_BMQ;  // query tile (dK/dV)
  static constexpr int QB = ATTN_DQ_QB;                                         // query blocks per wave (dQ)
  static constexpr int BN = ATTN_DQ_BN;                                         // key tile (dQ)
};

template <typename T, int D>
static hipError_t launch_pre_t(const Args &a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int RPB = 256 / (D / VEC);
  const int rows = a.B * a.H * a.S;
  const int blocks = min((rows + RPB - 1) / RPB, 65536);
  hipLaunchKernelGGL((attn_bwd_preprocess_kernel<T, D>), dim3(blocks), dim3(256), 0, a.stream, a.o_in,
                     static_cast<const T *>(a.dO), a.delta, rows);
  return hipGetLastError();
}

template <typename T, int D, bool DOC>
static hipError_t launch_dkdv_t(const Args &a) {
  constexpr int KBW = BwdCfg<T, D>::KBW;
  constexpr int BMQ = BwdCfg<T, D>::BMQ;
  constexpr int BN = 4 * 32 * KBW;
  const float c2 = a.scale * kLog2e;
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BN - 1) / BN;
    grid = dim3(ntiles, a.n_seqs, a.H);
  } else {
    ntiles = (a.S + BN - 1) / BN;
    grid = dim3(ntiles * a.B * a.H);
  }
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, KBW, BMQ, DOC>), grid, dim3(256), 0, a.stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<const T *>(a.dO), a.lse_in, a.delta_in, a.dk, a.dv, a.S, c2, a.scale,
                     a.cu_seqlens, ntiles);
  return hipGetLastError();
}

template <typename T, int D, bool DOC>
static hipError_t launch_dq_t(const Args &a) {
  constexpr int QB = BwdCfg<T, D>::QB;
  constexpr int BN = BwdCfg<T, D>::BN;
  constexpr int BM = 4 * 32 * QB;
  const float c2 = a.scale * kLog2e;
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BM - 1) / BM;
    grid = dim3(ntiles, a.n_seqs, a.H);
  } else {
    ntiles = (a.S + BM - 1) / BM;
    grid = dim3(ntiles * a.B * a.H);
  }
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, QB, BN, DOC>), grid, dim3(256), 0, a.stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<const T *>(a.dO), a.lse_in, a.delta_in, a.dq, a.S, c2, a.scale, a.cu_seqlens,
                     ntiles);
  return hipGetLastError();
}

#define ATTN_DISPATCH_D(FN, T, ...)                     \
  switch (a.D) {                                        \
    case 32: return FN<T, 32 __VA_OPT__(, ) __VA_ARGS__>(a);  \
    case 64: return FN<T, 64 __VA_OPT__(, ) __VA_ARGS__>(a);  \
    default: return FN<T, 128 __VA_OPT__(, ) __VA_ARGS__>(a); \
  }

template <typename T>
static hipError_t launch_pre_dt(const Args &a) { ATTN_DISPATCH_D(launch_pre_t, T) }
template <typename T, bool DOC>
static hipError_t launch_dkdv_dt(const Args &a) { ATTN_DISPATCH_D(launch_dkdv_t, T, DOC) }
template <typename T, bool DOC>
static hipError_t launch_dq_dt(const Args &a) { ATTN_DISPATCH_D(launch_dq_t, T, DOC) }

hipError_t launch_bwd_preprocess(const Args &a) {
  return a.bf16 ? launch_pre_dt<bf16>(a) : launch_pre_dt<float>(a);
}

hipError_t launch_bwd_dkdv(const Args &a) {
  if (a.bf16) return a.doc ? launch_dkdv_dt<bf16, true>(a) : launch_dkdv_dt<bf16, false>(a);
  return a.doc ? launch_dkdv_dt<float, true>(a) : launch_dkdv_dt<float, false>(a);
}

hipError_t launch_bwd_dq(const Args &a) {
  if (a.bf16) return a.doc ? launch_dq_dt<bf16, true>(a) : launch_dq_dt<bf16, false>(a);
  return a.doc ? launch_dq_dt<float, true>(a) : launch_dq_dt<float, false>(a);
}

}  // namespace attn
