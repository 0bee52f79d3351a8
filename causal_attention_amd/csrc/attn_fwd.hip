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
//  * Each wave computes S^T = K Q^T for its 32 queries, so a lane owns one
//    query and holds that query's scores in its own registers; P^T is then
//    already the B operand of O^T += V^T P^T ("accum" slot order,
//    attn_device.h).  K is read from LDS as (swizzled) row fragments; V is
//    read through the transposing LDS load from a swizzled row-major tile.
//  * No software pipeline inside a wave: at D = 64 the kernel needs about
//    122 VGPRs, so four workgroups share a CU and the hardware overlaps one
//    wave's exponentials with another wave's matrix-core work.
//  * K and V tiles arrive by direct global->LDS copies into two-slot rings,
//    requested one iteration before use, with one barrier per tile.
//  * No per-tile maximum: p = exp2(s * c2 - m) uses the reference maximum m
//    of earlier tiles (c2 = scale * log2 e).  The first tile, and any tile
//    whose exponentials could overflow (a row sum above 2^64 or not finite,
//    voted across the wave), take the exact path: true row maximum, rescale
//    of the running output and sum (an out-of-range tile's scores are
//    recomputed from its key tile, still in LDS, so the exponentials can
//    overwrite the scores in place).
//  * P is rounded to the input type (round to nearest even) for the P V
//    product.  O is divided by the sum of the rounded weights (a one-key row
//    then gives that key's value exactly, whatever the shift), LSE takes the
//    sum of the fp32 weights.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

constexpr float kRescaleLimit = 1.8446744e19f;  // 2^64: larger row sums take the exact path
// Packed documents take the work-ranked schedule (attn_device.h, doc_tile):
// measured on MI355X (B1 H16, 8,192 tokens in documents of 32-1024,
// same-process A/B) forward 47.2 -> 43.5 us median per call.
constexpr bool kRankDocsFwd = true;

template <typename T, typename OT, int D, int NW, int BN, int MINB, bool DOC>
__global__ __launch_bounds__(NW * 64, MINB) void attn_fwd_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                                 const T *__restrict__ v, OT *__restrict__ o,
                                                                 float *__restrict__ lse, int S, float c2,
                                                                 const int32_t *__restrict__ cu, int ntiles, int n_seqs, int H, int G,
                                                                 Layout lq, Layout lk, Layout lv, Layout lo) {
  constexpr int NT = NW * kWaveSize;
  constexpr int BM = NW * 32;  // query rows per workgroup
  constexpr int KB = D / 16;   // k-blocks over the head dimension
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int NB = BN / 32;  // 32-key blocks per tile
  constexpr int PB = BN / 16;  // k-blocks over the keys of a tile
  using E = Elem<T>;
  using frag = typename E::frag;
  using KTile = DmaTile<T, BN, D, NT, true>;   // read as row fragments: swizzled
  using VTile = DmaTile<T, BN, D, NT, true>;   // read through the transposing load: swizzled too

  // Two ring slots for K and for V, each its own LDS object: the slot an
  // access touches is known at compile time (the loop is unrolled by two),
  // so reading one slot never waits for the copy in flight into the other.
  __shared__ __attribute__((aligned(1024))) T sK0[BN * D];
  __shared__ __attribute__((aligned(1024))) T sK1[BN * D];
  __shared__ __attribute__((aligned(1024))) T sV0[BN * D];
  __shared__ __attribute__((aligned(1024))) T sV1[BN * D];

  const RowTile t = DOC ? doc_tile(cu, blockIdx.x, gridDim.x, ntiles, n_seqs, BM, S, true, kRankDocsFwd)
                        : causal_tile(blockIdx.x, gridDim.x, ntiles, BM, S, true);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  const int bi = t.head / H;  // batch entry
  const int hq = t.head % H;  // query head, and its key/value head hq / G
  const GBuf gq(q + panel_off(lq, bi, hq), panel_bytes(lq, t.r_end, D, sizeof(T)));
  const GBuf gk(k + panel_off(lk, bi, hq / G), panel_bytes(lk, t.seg_end, D, sizeof(T)));
  const GBuf gv(v + panel_off(lv, bi, hq / G), panel_bytes(lv, t.seg_end, D, sizeof(T)));

  const int w0 = t.r_start + wave * 32;  // first query of this wave
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32, t.r_end) - 1;
  const int kv_lo = t.seg_start;
  const int kv_hi = min(t.r_end, t.seg_end);  // one past the last key any row here can see
  const int ntile = (kv_hi - kv_lo + BN - 1) / BN;
  const int jw = wave_active ? (wave_last - kv_lo) / BN + 1 : 0;  // tiles this wave needs

  auto kslot = [&]<int P>() { return lds_cast(P == 0 ? sK0 : sK1); };
  auto vslot = [&]<int P>() { return lds_cast(P == 0 ? sV0 : sV1); };
  uint32_t koff[KTile::kPerWave], voff[VTile::kPerWave];
  KTile::lane_offsets(koff, wave, lane, lk.ss);
  VTile::lane_offsets(voff, wave, lane, lv.ss);
  auto issue = [&]<int P>(int tile) {
    const int r0 = kv_lo + tile * BN;
    KTile::issue_at(gk, kslot.template operator()<P>(), KTile::row0_bytes(r0, lk.ss), koff, wave);
    VTile::issue_at(gv, vslot.template operator()<P>(), VTile::row0_bytes(r0, lv.ss), voff, wave);
  };
  issue.template operator()<0>(0);

  frag qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) qf[kb] = global_frag_rs<T>(gq, w0 + c, 16 * kb + 8 * hh, lq.ss);

  f32x16 oacc[DB];
  float m = -INFINITY;  // reference max (scaled, base 2)
  float l = 0.f;        // this lane-half's partial row sum (for LSE)
  float lr = 0.f;       // ... of the rounded weights (16-bit inputs; divides O)
  constexpr bool kRounded = sizeof(T) == 2;
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};

  const RowFrag<T, D> rf0(lane);  // row fragments of the K tiles
  const TrSwz<T, D> trv0(lane);   // transposed reads of the V tiles

  // S^T = K Q^T for the key tile in `ks`.
  auto scores = [&](const lds_t<T> *ks, f32x16 (&sacc)[NB]) {
    const RowFrag<T, D> rf = rf0.pinned();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sacc[nb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const frag a = rf(ks, nb, kb);
        E::mma(sacc[nb], a, qf[kb]);
      }
  };

  // O^T += V^T P^T for the value tile in `vs` (transposed reads of the
  // swizzled tile: free of LDS bank conflicts, like the backward's).
  auto pv = [&](const lds_t<T> *vs, const frag (&pf)[PB]) {
    const TrSwz<T, D> tr = trv0.pinned();
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < PB; ++j) E::mma(oacc[db], tr(vs, 16 * j, db), pf[j]);
  };

  auto apply_mask = [&](f32x16 (&sacc)[NB], int k0) {
    // key k0 + off > query qi, off = 32 nb + 8 (r / 4) + 4 hh + r % 4: one
    // per-lane limit, compared with compile-time offsets.  key > qi also
    // covers keys past the sequence or document end: every stored row has
    // qi < r_end <= seg_end (those keys read as zeros).
    const int lim = (w0 + c) - k0 - 4 * hh;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[nb][r] = (32 * nb + 8 * (r / 4) + (r % 4)) > lim ? -INFINITY : sacc[nb][r];
      }
  };

  // Exponentials against the reference max, in place, then rounded and
  // summed.  True when every row of the wave stayed in range.
  auto softmax_fast = [&](f32x16 (&sacc)[NB], frag (&pf)[PB], float &psum, float &rsum) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[nb][r] = fast_exp2(__builtin_fmaf(sacc[nb][r], c2, -m));
    psum = 0.f;
    rsum = 0.f;
#pragma unroll
    for (int j = 0; j < PB; ++j) pf[j] = E::pack_sums(sacc[j / 2], j % 2, psum, rsum);
    return __builtin_amdgcn_ballot_w64(!(psum <= kRescaleLimit)) == 0;
  };

  // Exact path: true row maximum, rescale of the running output and sum.
  auto softmax_exact = [&](f32x16 (&sacc)[NB], frag (&pf)[PB], float &psum, float &rsum) {
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float mnew = fmaxf(m, mx * c2);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    l *= alpha;
    lr *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[nb][r] = fast_exp2(__builtin_fmaf(sacc[nb][r], c2, -mnew));
    psum = 0.f;
    rsum = 0.f;
#pragma unroll
    for (int j = 0; j < PB; ++j) pf[j] = E::pack_sums(sacc[j / 2], j % 2, psum, rsum);
  };

  // One key tile in ring slot P: wait for its copies (issued one iteration
  // ago; this wave's own, then everyone's), request the next tile into the
  // other slot (the barrier also retires every read of that slot), then
  // scores, softmax and P V.
  auto step = [&]<int P>(int j) {
    wait_vmcnt<0>();
    wg_barrier();
    if (j + 1 < ntile) issue.template operator()<1 - P>(j + 1);
    if (j >= jw) return;
    sched_hint<true>();
    const int k0 = kv_lo + j * BN;
    const bool masked = (k0 + BN - 1 > w0) || (k0 + BN > t.seg_end);
    const lds_t<T> *ks = kslot.template operator()<P>();
    f32x16 sacc[NB];
    frag pf[PB];
    float psum, rsum;
    mma_priority_hi();
    scores(ks, sacc);
    mma_priority_lo();
    if (masked) apply_mask(sacc, k0);
    if (m == -INFINITY) {
      softmax_exact(sacc, pf, psum, rsum);
    } else if (!softmax_fast(sacc, pf, psum, rsum)) {
      // a row sum left the safe range: recompute the scores from the key
      // tile (still in its slot) and take the exact path
      scores(ks, sacc);
      if (masked) apply_mask(sacc, k0);
      softmax_exact(sacc, pf, psum, rsum);
    }
    l += psum;
    if constexpr (kRounded) lr += rsum;
    mma_priority_hi();
    pv(vslot.template operator()<P>(), pf);
    mma_priority_lo();
  };

  for (int j = 0; j < ntile; j += 2) {
    step.template operator()<0>(j);
    if (j + 1 < ntile) step.template operator()<1>(j + 1);
  }

  // Every wave is past its last read of the ring slots: each wave stores its
  // rows through one slot (store_block_rows).
  static_assert(NW == 4 && BN * D * sizeof(T) >= 4096, "one 4 KB slot per wave");
  wg_barrier();
  if (!wave_active) return;
  const GBuf go(o + panel_off(lo, bi, hq), panel_bytes(lo, t.r_end, D, sizeof(OT)));
  const int qi = w0 + c;
  const float lt = l + swap_halves(l);
  const float lrt = kRounded ? lr + swap_halves(lr) : lt;
  const float inv = 1.0f / lrt;
  lds_t<f32x4> *scr = (lds_t<f32x4> *)(wave == 0 ? kslot.template operator()<0>()
                                       : wave == 1 ? kslot.template operator()<1>()
                                       : wave == 2 ? vslot.template operator()<0>()
                                                   : vslot.template operator()<1>());
#pragma unroll
  for (int db = 0; db < DB; ++db) store_block_rows<OT>(oacc[db] * inv, scr, go, w0, lo.ss, db * 32, lane);
  if (lse != nullptr && hh == 0 && qi < t.r_end) lse[(size_t)t.head * S + qi] = (m + __log2f(lt)) * kLn2;
}

// Tile shape per (dtype, D): waves per workgroup (NW, 32 queries each), keys
// per tile (BN) and the minimum number of workgroups per CU the register
// allocation must allow (MINB).
template <typename T, int D> struct FwdCfg {
  static constexpr int NW = 4;
  static constexpr int BN = (sizeof(T) == 4 && D == 128) ? 32 : 64;
  static constexpr int MINB = 1;
};

template <typename T, typename OT, int D, bool DOC>
static hipError_t launch_fwd_t(const Args &a) {
  constexpr int BN = FwdCfg<T, D>::BN;
  constexpr int NW = FwdCfg<T, D>::NW;
  constexpr int MINB = FwdCfg<T, D>::MINB;
  constexpr int BM = NW * 32;
  const float c2 = a.scale * kLog2e;
  dim3 block(NW * 64);
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BM - 1) / BM;
    grid = dim3(a.H * doc_blocks_per_unit(a.n_seqs, ntiles, a.S, BM, kRankDocsFwd));
  } else {
    ntiles = (a.S + BM - 1) / BM;
    grid = dim3(ntiles * a.B * a.H);
  }
  hipLaunchKernelGGL((attn_fwd_kernel<T, OT, D, NW, BN, MINB, DOC>), grid, block, 0, a.stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<OT *>(a.o), a.lse, a.S, c2, a.cu_seqlens, ntiles, a.n_seqs, a.H, a.H / a.H_kv,
                     a.lq, a.lk, a.lv, a.lo);
  return hipGetLastError();
}

template <typename T, typename OT, int D>
static hipError_t launch_fwd_d(const Args &a) {
  return a.doc ? launch_fwd_t<T, OT, D, true>(a) : launch_fwd_t<T, OT, D, false>(a);
}

template <typename T, typename OT>
static hipError_t launch_fwd_dt(const Args &a) {
  switch (a.D) {
    case 32: return launch_fwd_d<T, OT, 32>(a);
    case 64: return launch_fwd_d<T, OT, 64>(a);
    default: return launch_fwd_d<T, OT, 128>(a);
  }
}

hipError_t launch_fwd(const Args &a) {
  switch (a.dtype) {
    case 1: return a.out16 ? launch_fwd_dt<bf16, bf16>(a) : launch_fwd_dt<bf16, float>(a);
    case 2: return a.out16 ? launch_fwd_dt<f16, f16>(a) : launch_fwd_dt<f16, float>(a);
    default: return launch_fwd_dt<float, float>(a);
  }
}

}  // namespace attn
