// attn_fwd.hip - forward kernel: O = softmax(scale * Q K^T + mask) V and the row LSE.
//
// Flash-attention forward (Forge, "What this is": fused forward written after
// FlashAttention-2, "Acknowledgements"): one workgroup owns BM query rows of
// one head and streams key/value tiles up to its causal diagonal (keys of its
// document only, in packed mode), keeping per row a reference maximum m, a
// running sum l and the unnormalised output; after the last tile O = acc / l
// and LSE = m + ln l.  Scores never leave registers.
//
// gfx950 mapping.
//  * Each wave computes S^T = K Q^T for its 32*QB queries, so a lane owns one
//    query and holds that query's scores in its own registers; P^T is then
//    already the B operand of O^T += V^T P^T ("accum" slot order,
//    attn_device.h).  K is read from LDS as (swizzled) row fragments; V is
//    stored row-major and read through the transposing LDS load.
//  * Software pipeline per wave: while the softmax of tile j runs on the
//    vector ALUs, the matrix cores compute the scores of tile j+1 and the
//    P V product of tile j-1.
//  * K and V tiles arrive by direct global->LDS copies into 3-slot rings,
//    requested two iterations before use, with one barrier per tile.
//  * No per-tile maximum: p = exp2(s * c2 - m) uses the reference maximum m
//    of earlier tiles (c2 = scale * log2 e).  The first tile, and any tile
//    whose exponentials could overflow (a row sum above 2^64 or not finite,
//    voted across the wave), take the exact path: true row maximum, rescale
//    of the running output and sum (an out-of-range tile's scores are
//    recomputed from its key tile, still in LDS, so the exponentials can
//    overwrite the scores in place).
//  * P is rounded to the input type (round to nearest even) for the P V
//    product; the row sum adds the fp32 values.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

constexpr float kRescaleLimit = 1.8446744e19f;  // 2^64: larger row sums take the exact path

template <typename T, int D, int NW, int QB, int BN, bool DOC>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                       const T *__restrict__ v, float *__restrict__ o,
                                                       float *__restrict__ lse, int S, float c2,
                                                       const int32_t *__restrict__ cu, int ntiles) {
  constexpr int NT = NW * kWaveSize;
  constexpr int BM = NW * 32 * QB;  // query rows per workgroup
  constexpr int KB = D / 16;        // k-blocks over the head dimension
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int NB = BN / 32;       // 32-key blocks per tile
  constexpr int PB = BN / 16;       // k-blocks over the keys of a tile
  constexpr int NS = 3;             // LDS ring slots for K and for V
  using E = Elem<T>;
  using frag = typename E::frag;
  using KTile = DmaTile<T, BN, D, NT, true>;   // read as row fragments: swizzled
  using VTile = DmaTile<T, BN, D, NT, false>;  // read through the transposing load
  constexpr int IPW = KTile::kPerWave;         // copy instructions per wave per tile
  static_assert(VTile::kPerWave == IPW, "K and V tiles have the same shape");

  __shared__ __attribute__((aligned(1024))) T sK[NS][BN * D];
  __shared__ __attribute__((aligned(1024))) T sV[NS][BN * D];

  const RowTile t = DOC ? doc_tile(cu, blockIdx.x, gridDim.x, blockIdx.y, blockIdx.z, BM, true)
                        : causal_tile(blockIdx.x, gridDim.x, ntiles, BM, S, true);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  const size_t base = (size_t)t.head * S * D;
  const GBuf gq(q + base, (uint32_t)(t.r_end * D * sizeof(T)));
  const GBuf gk(k + base, (uint32_t)(t.seg_end * D * sizeof(T)));
  const GBuf gv(v + base, (uint32_t)(t.seg_end * D * sizeof(T)));

  const int w0 = t.r_start + wave * 32 * QB;  // first query of this wave
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32 * QB, t.r_end) - 1;
  const int kv_lo = t.seg_start;
  const int kv_hi = min(t.r_end, t.seg_end);  // one past the last key any row here can see
  const int ntile = (kv_hi - kv_lo + BN - 1) / BN;
  const int jw = wave_active ? (wave_last - kv_lo) / BN + 1 : 0;  // tiles this wave needs

  // Tiles past the end are still requested (they arrive as zeros into slots
  // nobody reads), so every iteration issues the same number of copies and
  // one fixed wait count covers the tiles an iteration needs.
  auto issue_k = [&](int tile) { KTile::issue(gk, sK[tile % NS], kv_lo + tile * BN, wave, lane); };
  auto issue_v = [&](int tile) { VTile::issue(gv, sV[tile % NS], kv_lo + tile * BN, wave, lane); };
  issue_k(0);
  issue_k(1);
  issue_k(2);
  issue_v(0);

  frag qf[QB][KB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[qb][kb] = global_frag<T, D>(gq, w0 + 32 * qb + c, 16 * kb + 8 * hh);

  f32x16 oacc[QB][DB];
  float m[QB], l[QB];  // reference max (scaled, base 2) and this lane-half's partial sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  }

  // S^T of the key tile in ring slot `b`.
  auto scores = [&](int b, f32x16 (&sacc)[QB][NB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[qb][nb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const frag a = swz_frag<T, D, KTile::kSW>(sK[b], nb * 32 + c, (16 * kb + 8 * hh) / KTile::kVec);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) E::mma(sacc[qb][nb], a, qf[qb][kb]);
      }
    }
  };

  // O^T += V^T P^T for the value tile in ring slot `b`.
  auto pv = [&](int b, const frag (&pf)[QB][PB]) {
    const TrRead<T, D> vr(sV[b], lane);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const frag a = vr(16 * j, 32 * db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) E::mma(oacc[qb][db], a, pf[qb][j]);
      }
    }
  };

  auto apply_mask = [&](f32x16 (&sacc)[QB][NB], int k0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qi = w0 + 32 * qb + c;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * nb + 8 * (r / 4) + 4 * hh + (r % 4);
          sacc[qb][nb][r] = (key > qi || key >= t.seg_end) ? -INFINITY : sacc[qb][nb][r];
        }
    }
  };

  // Exponentials against the reference max, in place, then rounded and
  // summed.  True when every row of the wave stayed in range.
  auto softmax_fast = [&](f32x16 (&sacc)[QB][NB], frag (&pf)[QB][PB], float (&psum)[QB]) {
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][nb][r] = fast_exp2(__builtin_fmaf(sacc[qb][nb][r], c2, -m[qb]));
      psum[qb] = 0.f;
#pragma unroll
      for (int j = 0; j < PB; ++j) pf[qb][j] = E::pack_sum(sacc[qb][j / 2], j % 2, psum[qb]);
      bad = bad || !(psum[qb] <= kRescaleLimit);
    }
    return __builtin_amdgcn_ballot_w64(bad) == 0;
  };

  // Exact path: true row maximum, rescale of the running output and sum.
  // Works in place on raw scores.
  auto softmax_exact = [&](f32x16 (&sacc)[QB][NB], frag (&pf)[QB][PB], float (&psum)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][nb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = fmaxf(m[qb], mx * c2);
      const float alpha = fast_exp2(m[qb] - mnew);
      m[qb] = mnew;
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][nb][r] = fast_exp2(__builtin_fmaf(sacc[qb][nb][r], c2, -mnew));
      psum[qb] = 0.f;
#pragma unroll
      for (int j = 0; j < PB; ++j) pf[qb][j] = E::pack_sum(sacc[qb][j / 2], j % 2, psum[qb]);
    }
  };

  auto needs_mask = [&](int k0) { return (k0 + BN - 1 > w0) || (k0 + BN > t.seg_end); };

  // Prologue: scores of tile 0 (this wave's copies of K0 done, then everyone's).
  wait_vmcnt<3 * IPW>();
  wg_barrier();
  f32x16 snext[QB][NB];
  if (jw > 0) {
    scores(0, snext);
    if (needs_mask(kv_lo)) apply_mask(snext, kv_lo);
  }

  frag pprev[QB][PB];
  bool have_prev = false;
  for (int j = 0; j < ntile; ++j) {
    const int k0 = kv_lo + j * BN;
    // K(j+1) and V(j-1) were requested two iterations ago: wait for this
    // wave's copies, then for everyone's.  The barrier also retires every
    // read of K(j) and V(j-2), whose slots the next copies overwrite.
    wait_vmcnt<2 * IPW>();
    wg_barrier();
    issue_k(j + 3);
    issue_v(j + 1);

    f32x16 scur[QB][NB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) scur[qb][nb] = snext[qb][nb];
    const bool cur_active = j < jw;
    const bool next_active = j + 1 < jw;
    const bool next_mask = needs_mask(k0 + BN);
    frag pcur[QB][PB];
    float psum[QB];

    // Scores of tile j again, from its key slot (rewritten only by the copy
    // issued at the next iteration), for the exact path after an
    // out-of-range fast pass.
    auto redo_exact = [&]() {
      scores(j % NS, scur);
      if (needs_mask(k0)) apply_mask(scur, k0);
      softmax_exact(scur, pcur, psum);
    };
    if (cur_active && next_active && have_prev && !next_mask) {
      // Steady state: scores of tile j+1 and P V of tile j-1 on the matrix
      // cores while the exponentials of tile j run.
      scores((j + 1) % NS, snext);
      pv((j + NS - 1) % NS, pprev);
      if (!softmax_fast(scur, pcur, psum)) redo_exact();
    } else {
      if (have_prev) pv((j + NS - 1) % NS, pprev);
      if (next_active) {
        scores((j + 1) % NS, snext);
        if (next_mask) apply_mask(snext, k0 + BN);
      }
      if (cur_active) {
        if (m[0] == -INFINITY)
          softmax_exact(scur, pcur, psum);
        else if (!softmax_fast(scur, pcur, psum))
          redo_exact();
      }
    }
    if (cur_active) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l[qb] += psum[qb];
#pragma unroll
        for (int jj = 0; jj < PB; ++jj) pprev[qb][jj] = pcur[qb][jj];
      }
    }
    have_prev = cur_active;
  }
  if (have_prev) {
    wait_vmcnt<2 * IPW>();  // V(ntile-1) was requested in the last iteration but one
    wg_barrier();
    pv((ntile - 1) % NS, pprev);
  }
  wait_vmcnt<0>();  // no copy may land in LDS after the workgroup retires

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

// Tile shape per (dtype, D): waves per workgroup (NW), queries per wave (32 * QB)
// and keys per tile (BN).  Two query blocks per wave would halve the LDS traffic
// per matrix-core step, but with two score tiles live in the pipeline they leave
// one wave per SIMD; eight waves sharing one K/V ring (two per SIMD) halve the
// copy traffic per CU but give half as many workgroups.  Both measured slower at
// context 1024 than four waves with one query block each.
template <typename T, int D> struct FwdCfg {
#ifdef ATTN_FWD_QB
  static constexpr int NW = (sizeof(T) == 2 && D == 64) ? ATTN_FWD_NW : 4;
  static constexpr int QB = ATTN_FWD_QB;
  static constexpr int BN = D == 32 ? 64 : (sizeof(T) == 4 && D == 128) ? 32 : ATTN_FWD_BN;
#else
  static constexpr int NW = 4;
  static constexpr int QB = 1;
  static constexpr int BN = (sizeof(T) == 4 && D == 128) ? 32 : 64;  // LDS: 3-slot K and V rings
#endif
};

template <typename T, int D, bool DOC>
static hipError_t launch_fwd_t(const Args &a) {
  constexpr int QB = FwdCfg<T, D>::QB;
  constexpr int BN = FwdCfg<T, D>::BN;
  constexpr int NW = FwdCfg<T, D>::NW;
  constexpr int BM = NW * 32 * QB;
  const float c2 = a.scale * kLog2e;
  dim3 block(NW * 64);
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BM - 1) / BM;
    grid = dim3(ntiles, a.n_seqs, a.H);
  } else {
    ntiles = (a.S + BM - 1) / BM;
    grid = dim3(ntiles * a.B * a.H);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, NW, QB, BN, DOC>), grid, block, 0, a.stream,
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
