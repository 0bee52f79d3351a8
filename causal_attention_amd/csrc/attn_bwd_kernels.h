// attn_bwd_kernels.h - backward kernels: Delta preprocess, dK/dV, dQ, and
// their launch templates.  attn_bwd.hip instantiates them for causal masks,
// attn_bwd_doc.hip for packed documents.
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
#pragma once
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

// Packed documents: the work-ranked schedule (attn_device.h, doc_tile) for
// dK/dV's key tiles.  dQ keeps the per-document grid: measured on MI355X
// (B1 H16, 8,192 tokens in documents of 32-1024, same-process A/B, backward
// median) the ranked dK/dV took 85.2 -> 83.2 us; ranking dQ as well made it
// 88.5 with 64-key dQ tiles and gained nothing with 32-key ones.
constexpr bool kRankDocsDq = false;
constexpr bool kRankDocsDkdv = true;

// ---------------------------------------------------------------------------
// Delta_i = sum_d dO_id * O_id.  Memory bound: each group of D/VEC lanes reads
// one row of dO (input dtype) and O (fp32) with 16-byte loads and reduces
// across the group.
template <typename T, typename OT, int D>
__global__ __launch_bounds__(256) void attn_bwd_preprocess_kernel(const OT *__restrict__ o,
                                                                  const T *__restrict__ dO,
                                                                  float *__restrict__ delta, int rows, int S, int H,
                                                                  Layout lo, Layout ldo) {
  constexpr int VEC = 16 / sizeof(T);  // dO elements per 16-byte load
  constexpr int LPR = D / VEC;         // lanes per row
  constexpr int RPB = 256 / LPR;       // rows per block per step
  const int tid = threadIdx.x;
  const int sub = tid % LPR;
  for (int row0 = blockIdx.x * RPB; row0 < rows; row0 += gridDim.x * RPB) {
    const int row = row0 + tid / LPR;
    float acc = 0.f;
    if (row < rows) {
      const int bh = row / S;  // row of Delta [B, H, S] -> (batch, head, position)
      const int s = row - bh * S;
      const T *dp = dO + panel_off(ldo, bh / H, bh % H) + (size_t)s * ldo.ss + sub * VEC;
      const OT *op = o + panel_off(lo, bh / H, bh % H) + (size_t)s * lo.ss + sub * VEC;
      if constexpr (sizeof(T) == 2) {
        const typename Elem<T>::frag g = *reinterpret_cast<const typename Elem<T>::frag *>(dp);
        float ov[8];
        if constexpr (sizeof(OT) == 4) {
          const f32x4 o0 = *reinterpret_cast<const f32x4 *>(op);
          const f32x4 o1 = *reinterpret_cast<const f32x4 *>(op + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ov[i] = o0[i];
            ov[4 + i] = o1[i];
          }
        } else {
          const typename Vec8Of<OT>::type h = *reinterpret_cast<const typename Vec8Of<OT>::type *>(op);
#pragma unroll
          for (int i = 0; i < 8; ++i) ov[i] = (float)h[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += (float)g[i] * ov[i];
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
// dK, dV.  A workgroup owns BN = 128 keys of one head (32 per wave) and loops
// over query tiles of BMQ rows from its first key to the end of the sequence
// (or document).  Q and dO tiles, with their LSE and Delta, arrive by direct
// global->LDS copies into two ring slots (separate LDS objects, loop unrolled
// by two) one iteration ahead; Q and dO are read both as row fragments and,
// through the transposing load, as Q^T and dO^T.
//
// SPLIT = 2 or 4 (grouped heads, G a multiple of SPLIT): the workgroup owns
// 128 / SPLIT keys, and each key group of 32 has SPLIT waves, each running
// the query-tile loop over G / SPLIT of the query heads with a ring of its
// own; at the end the other waves hand their partial dK, dV to the first
// through LDS, which adds them (in the order of their parts, a fixed order)
// and stores.  SPLIT times the workgroups of SPLIT = 1 for the same keys, so
// grouped heads fill more wave slots and each wave's chain of query tiles is
// SPLIT times shorter.
template <typename T, typename OT, int D, int BMQ, bool DOC, int SPLIT>
__device__ __forceinline__ void bwd_dkdv_body(
    int bid, int nblocks, const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dO, const float *__restrict__ lse, const float *__restrict__ delta, OT *__restrict__ dk,
    OT *__restrict__ dv, int S, float c2, float scale, const int32_t *__restrict__ cu, int ntiles, int n_seqs,
    int H, int G, int P, int64_t part_stride, const float *__restrict__ rope, int rope_npos, Layout lq, Layout lk,
    Layout lv, Layout ldo, Layout ldk, Layout ldv) {
  constexpr int NW = 4;
  constexpr int NT = NW * kWaveSize;
  constexpr int NWH = NW / SPLIT;  // waves per part: one per 32-key group
  constexpr int BN = NWH * 32;     // keys per workgroup
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = BMQ / 32;  // 32-query blocks per tile
  using E = Elem<T>;
  using frag = typename E::frag;
  using QTile = DmaTile<T, BMQ, D, NT / SPLIT, true>;  // copied by the part's waves
  static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4, "one, two or four parts");
  static_assert(SPLIT == 1 || DB * 16 * kWaveSize * 4 <= SPLIT * BMQ * D * (int)sizeof(T),
                "a wave's partial dK (or dV) fits one ring slot");
  static_assert(SPLIT != 4 || 2 * DB * 16 * kWaveSize * 4 <= SPLIT * BMQ * D * (int)sizeof(T),
                "a wave's partial dK and dV fit one ring slot");
  constexpr int VROWS = BMQ < 64 ? 64 : BMQ;  // rows of LSE / Delta per slot
  constexpr int NVEC = 2 * (VROWS / 64);      // 64-row loads of LSE and Delta per tile
  static_assert(BMQ <= 64 || BMQ % 64 == 0, "LSE / Delta loads move 64 rows at a time");
  constexpr int NPW = (NVEC + NWH - 1) / NWH;  // of them per wave

  __shared__ __attribute__((aligned(1024))) T sQ0[SPLIT * BMQ * D];  // [half][row][col]
  __shared__ __attribute__((aligned(1024))) T sQ1[SPLIT * BMQ * D];
  __shared__ __attribute__((aligned(1024))) T sO0[SPLIT * BMQ * D];  // dO
  __shared__ __attribute__((aligned(1024))) T sO1[SPLIT * BMQ * D];
  __shared__ __attribute__((aligned(256))) float sL0[SPLIT * VROWS];  // LSE (natural log)
  __shared__ __attribute__((aligned(256))) float sL1[SPLIT * VROWS];
  __shared__ __attribute__((aligned(256))) float sD0[SPLIT * VROWS];  // Delta
  __shared__ __attribute__((aligned(256))) float sD1[SPLIT * VROWS];

  const RowTile t = DOC ? doc_tile(cu, bid, nblocks, ntiles, n_seqs, BN, S, false, kRankDocsDkdv)
                        : causal_tile(bid, nblocks, ntiles, BN, S, false);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int half = wave % SPLIT;  // which part of the query heads
  const int kg = wave / SPLIT;    // which 32 keys; also the wave's index in its part
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  // t.head / P is a key/value head; its G query heads are hk*G .. hk*G + G - 1,
  // and dK, dV sum over all of them (the query-tile loop runs over the
  // group, or over half of it in each half).  With P > 1 workspace parts
  // (grouped heads, attn_bwd_gqa_ws) this workgroup takes part t.head % P of
  // the group, G / P heads from hq0 on, and writes its sums to part p of the
  // workspace (dk, dv + p * part_stride); attn_bwd_sum_parts_kernel adds them.
  const int Hkv = H / G;
  const int part = t.head % P;
  const int GP = G / P;
  const int bi = t.head / P / Hkv;  // batch entry
  const int hk = t.head / P % Hkv;  // key/value head
  const int hq0 = hk * G + part * GP;  // this workgroup's first query head
  const int qh0 = bi * H + hq0;     // its (batch, head) index into LSE and Delta
  const GBuf gk(k + panel_off(lk, bi, hk), panel_bytes(lk, t.r_end, D, sizeof(T)));
  const GBuf gv(v + panel_off(lv, bi, hk), panel_bytes(lv, t.r_end, D, sizeof(T)));

  const int w0 = t.r_start + kg * 32;  // first key of this wave
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32, t.r_end) - 1;
  const int key = w0 + c;
  const int q_lo = t.r_start;  // the first query that sees any of these keys
  const int ntq = (t.seg_end - q_lo + BMQ - 1) / BMQ;  // query tiles per query head
  const int GH = GP / SPLIT;                            // query heads per part
  const int ntile = GH * ntq;                           // over the part's heads
  float staged[NPW];                                    // this wave's LSE or Delta rows in flight
#pragma unroll
  for (int i = 0; i < NPW; ++i) staged[i] = 0.f;

  auto qslot = [&]<int P>() { return lds_cast(P == 0 ? sQ0 : sQ1) + half * BMQ * D; };
  auto oslot = [&]<int P>() { return lds_cast(P == 0 ? sO0 : sO1) + half * BMQ * D; };
  auto lslot = [&]<int P>() { return lds_cast(P == 0 ? sL0 : sL1) + half * VROWS; };
  auto dslot = [&]<int P>() { return lds_cast(P == 0 ? sD0 : sD1) + half * VROWS; };
  uint32_t qoff[QTile::kPerWave], dooff[QTile::kPerWave];
  QTile::lane_offsets(qoff, kg, lane, lq.ss);
  QTile::lane_offsets(dooff, kg, lane, ldo.ss);
  auto issue = [&]<int P>(int it) {
    const int g = half * GH + it / ntq;
    const int q0 = q_lo + (it % ntq) * BMQ;
    const size_t rbase = (size_t)(qh0 + g) * S;
    // Queries past the segment read as zeros (Q, dO, LSE, Delta all 0): their
    // P is 1 but dO and Q are 0, so they add nothing to dV or dK.
    const GBuf gq(q + panel_off(lq, bi, hq0 + g), panel_bytes(lq, t.seg_end, D, sizeof(T)));
    const GBuf gdo(dO + panel_off(ldo, bi, hq0 + g), panel_bytes(ldo, t.seg_end, D, sizeof(T)));
    const GBuf glse(lse + rbase, (uint32_t)(t.seg_end * sizeof(float)));
    const GBuf gdel(delta + rbase, (uint32_t)(t.seg_end * sizeof(float)));
    QTile::issue_at(gq, qslot.template operator()<P>(), QTile::row0_bytes(q0, lq.ss), qoff, kg);
    QTile::issue_at(gdo, oslot.template operator()<P>(), QTile::row0_bytes(q0, ldo.ss), dooff, kg);
    // 64-row loads of LSE, then of Delta, dealt over the part's waves into
    // registers; each wave writes its rows to the slot (as row shifts) before
    // the tile's barrier
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int v = kg + i * NWH;
      if (v < NVEC / 2)
        staged[i] = glse.load4((uint32_t)(q0 + 64 * v + lane) * 4u);
      else if (v < NVEC)
        staged[i] = gdel.load4((uint32_t)(q0 + 64 * (v - NVEC / 2) + lane) * 4u);
    }
  };
  // The staged rows enter the tile's slot as the shifts the scores need:
  // -LSE / scale and -Delta, so that each 32-query block starts its S and dP
  // accumulators from them (shift_rows) instead of adding them afterwards.
  const float rscale = 1.0f / scale;
  auto publish = [&]<int P>() {
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int v = kg + i * NWH;
      if (v < NVEC / 2)
        lslot.template operator()<P>()[64 * v + lane] = -staged[i] * rscale;
      else if (v < NVEC)
        dslot.template operator()<P>()[64 * (v - NVEC / 2) + lane] = -staged[i];
    }
  };
  issue.template operator()<0>(0);

  // K and V fragments of this wave's keys stay in registers, except for fp32
  // inputs at D = 128 (256 registers on their own), which re-read them from
  // the cache at every query tile.
  constexpr bool kKVRegs = !(sizeof(T) == 4 && D == 128);
  constexpr int KBR = kKVRegs ? KB : 1;
  frag kf[KBR], vf[KBR];
  if constexpr (kKVRegs) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      kf[kb] = global_frag_rs<T>(gk, key, 16 * kb + 8 * hh, lk.ss);
      vf[kb] = global_frag_rs<T>(gv, key, 16 * kb + 8 * hh, lv.ss);
    }
  }
  auto kfrag = [&](int kb) {
    return kKVRegs ? kf[kKVRegs ? kb : 0] : global_frag_rs<T>(gk, key, 16 * kb + 8 * hh, lk.ss);
  };
  auto vfrag = [&](int kb) {
    return kKVRegs ? vf[kKVRegs ? kb : 0] : global_frag_rs<T>(gv, key, 16 * kb + 8 * hh, lv.ss);
  };
  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkacc[db] = f32x16{};
    dvacc[db] = f32x16{};
  }

  const TrSwz<T, D> tr0(lane);    // transposed reads of the Q and dO tiles
  const RowFrag<T, D> rf0(lane);  // row fragments of the same tiles

  // One query tile: per 32-query block, S' = Q K^T - LSE/scale and
  // dP' = dO V^T - Delta as [query][key] blocks (lane c owns key w0 + c), the
  // accumulators starting from the per-query shifts: element r of a lane's
  // block is query row 8 (r / 4) + 4 hh + r % 4, so four 16-byte LDS reads of
  // the shift rows fill it.  Then P = exp2(S' c2), dS = P dP', dV^T += dO^T P
  // and dK^T += Q^T dS.
  auto shift_rows = [&](const lds_t<float> *sh, int qb) {
    f32x16 a;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 v4 = *(const lds_t<f32x4> *)(sh + qb * 32 + 8 * j + 4 * hh);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[4 * j + i] = v4[i];
    }
    return a;
  };
  // Pipelined pair of query blocks (16-bit inputs, D = 64).  Measured on
  // MI355X, backward: ctx 1024 97.8 -> 94.9 us, S = 8192 499 -> 490 us; at
  // D = 32 the second set of score accumulators costs the fourth wave per
  // SIMD (165 VGPRs) and it is 3-6 % slower.
  constexpr bool kPipe = QB % 2 == 0 && sizeof(T) == 2 && D == 64;
  auto tile = [&]<int P>(int q0, bool masked) {
    const lds_t<T> *sq = qslot.template operator()<P>();
    const lds_t<T> *so = oslot.template operator()<P>();
    const lds_t<float> *sl = lslot.template operator()<P>();
    const lds_t<float> *sd = dslot.template operator()<P>();
    const TrSwz<T, D> tr = tr0.pinned();
    const RowFrag<T, D> rf = rf0.pinned();
    sched_hint<D != 64>();
    if constexpr (kPipe) {
      // The tile's 32-query blocks in a software pipeline inside the wave
      // (below).  A block whose queries all precede this wave's keys is
      // computed with every score masked: P = dS = 0 adds exact zeros.
      auto scores = [&](int qb, f32x16 &sacc, f32x16 &pacc) {
        sacc = shift_rows(sl, qb);
        pacc = shift_rows(sd, qb);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          E::mma(sacc, rf(sq, qb, kb), kfrag(kb));
          E::mma(pacc, rf(so, qb, kb), vfrag(kb));
        }
      };
      // query q0 + 32 qb + off < key, off = 8 (r / 4) + 4 hh + r % 4: the
      // score becomes -inf, whose exp2 is exactly 0
      auto mask = [&](int qb, f32x16 &sacc) {
        const int lim = key - q0 - qb * 32 - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = (8 * (r / 4) + (r % 4)) < lim ? -INFINITY : sacc[r];
      };
      auto soft = [&](f32x16 &sacc, f32x16 &pacc, frag (&ps)[4]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(sacc[r] * c2);
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * pacc[r];
        ps[0] = E::pack(sacc, 0);
        ps[1] = E::pack(sacc, 1);
        ps[2] = E::pack(pacc, 0);
        ps[3] = E::pack(pacc, 1);
      };
      auto accum = [&](int qb, const frag (&ps)[4]) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          E::mma(dvacc[db], tr(so, 32 * qb, db), ps[0]);
          E::mma(dvacc[db], tr(so, 32 * qb + 16, db), ps[1]);
          E::mma(dkacc[db], tr(sq, 32 * qb, db), ps[2]);
          E::mma(dkacc[db], tr(sq, 32 * qb + 16, db), ps[3]);
        }
      };
      // Each step issues block b + 1's score products, block b's softmax and
      // block b - 1's dV / dK products: independent work in one basic block
      // that the compiler interleaves; the mask branch sits between steps.
      // (Measured with two blocks per tile and with four (128-query tiles):
      // within 1 % of each other.)
      f32x16 sa[2], pa[2];
      frag ps[2][4];
      scores(0, sa[0], pa[0]);
      if (masked) mask(0, sa[0]);
#pragma unroll
      for (int b = 0; b <= QB; ++b) {
        if (b >= 1) accum(b - 1, ps[(b - 1) % 2]);
        if (b + 1 < QB) scores(b + 1, sa[(b + 1) % 2], pa[(b + 1) % 2]);
        if (b < QB) {
          soft(sa[b % 2], pa[b % 2], ps[b % 2]);
          // keep block b's softmax in this step: without a use here the
          // compiler sinks it past the next branch, next to its products
#pragma unroll
          for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(ps[b % 2][i]));
        }
        if (b + 1 < QB && masked) mask(b + 1, sa[(b + 1) % 2]);
      }
      return;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // a block whose queries all precede this wave's first key adds nothing
      if (masked && q0 + qb * 32 + 31 < w0) continue;
      f32x16 sacc = shift_rows(sl, qb), pacc = shift_rows(sd, qb);
      mma_priority_hi();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        E::mma(sacc, rf(sq, qb, kb), kfrag(kb));
        E::mma(pacc, rf(so, qb, kb), vfrag(kb));
      }
      mma_priority_lo();
      // query q0 + 32 qb + off < key, off = 8 (r / 4) + 4 hh + r % 4: one
      // per-lane limit, compared with compile-time offsets
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(sacc[r] * c2);
      if (masked) {
        const int lim = key - q0 - qb * 32 - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = (8 * (r / 4) + (r % 4)) < lim ? 0.f : sacc[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * pacc[r];
      const frag p0 = E::pack(sacc, 0), p1 = E::pack(sacc, 1);
      const frag s0 = E::pack(pacc, 0), s1 = E::pack(pacc, 1);
      mma_priority_hi();
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        E::mma(dvacc[db], tr(so, 32 * qb, db), p0);
        E::mma(dvacc[db], tr(so, 32 * qb + 16, db), p1);
        E::mma(dkacc[db], tr(sq, 32 * qb, db), s0);
        E::mma(dkacc[db], tr(sq, 32 * qb + 16, db), s1);
      }
      mma_priority_lo();
    }
  };

  // Query tile `it` in ring slot P: wait for this wave's copies and staged
  // rows, write the rows to the slot, cross the barrier (everyone's copies
  // and rows are then visible), request the next tile into the other slot,
  // compute.
  auto step = [&]<int P>(int it) {
    wait_vmcnt<0>();
    publish.template operator()<P>();
    wait_vmcnt_lgkm0<0>();
    wg_barrier();
    if (it + 1 < ntile) issue.template operator()<1 - P>(it + 1);
    const int q0 = q_lo + (it % ntq) * BMQ;
    if (!wave_active || q0 + BMQ - 1 < w0) return;  // every query precedes every key here
    // One tile body with a uniform branch around the masking: two
    // instantiations would give the accumulators different registers in
    // each and cost copies where they join.
    tile.template operator()<P>(q0, q0 < wave_last);
  };
  for (int it = 0; it < ntile; it += 2) {
    step.template operator()<0>(it);
    if (it + 1 < ntile) step.template operator()<1>(it + 1);
  }

  if constexpr (SPLIT == 2) {
    // The second half's partial sums go through the ring slots (free once
    // every wave has passed this barrier), lane-major so each lane reads
    // back its own elements; the first half adds them and stores.
    wg_barrier();
    lds_t<f32x4> *pk = (lds_t<f32x4> *)lds_cast(kg == 0 ? sQ0 : sO0);
    lds_t<f32x4> *pv = (lds_t<f32x4> *)lds_cast(kg == 0 ? sQ1 : sO1);
    if (half == 1 && wave_active) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 a4, b4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a4[i] = dkacc[db][4 * g + i];
            b4[i] = dvacc[db][4 * g + i];
          }
          pk[(db * 4 + g) * kWaveSize + lane] = a4;
          pv[(db * 4 + g) * kWaveSize + lane] = b4;
        }
    }
    wg_barrier();
    if (half == 1) return;
    if (wave_active) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 a4 = pk[(db * 4 + g) * kWaveSize + lane];
          const f32x4 b4 = pv[(db * 4 + g) * kWaveSize + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dkacc[db][4 * g + i] += a4[i];
            dvacc[db][4 * g + i] += b4[i];
          }
        }
    }
  }
  if constexpr (SPLIT == 4) {
    // One key group; parts 1-3 write their partial dK, dV (lane-major) to a
    // ring slot each, part 0 adds them in part order and stores.
    static_assert(NWH == 1, "four parts of one key group");
    wg_barrier();
    auto part_buf = [&](int h) {
      return (lds_t<f32x4> *)lds_cast(h == 1 ? sQ0 : h == 2 ? sQ1 : sO0);
    };
    constexpr int kV = DB * 4 * kWaveSize;  // f32x4 offset of dV behind dK
    if (half != 0 && wave_active) {
      lds_t<f32x4> *pb = part_buf(half);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 a4, b4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a4[i] = dkacc[db][4 * g + i];
            b4[i] = dvacc[db][4 * g + i];
          }
          pb[(db * 4 + g) * kWaveSize + lane] = a4;
          pb[kV + (db * 4 + g) * kWaveSize + lane] = b4;
        }
    }
    wg_barrier();
    if (half != 0) return;
    if (wave_active) {
#pragma unroll
      for (int h = 1; h < 4; ++h) {
        const lds_t<f32x4> *pb = part_buf(h);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 a4 = pb[(db * 4 + g) * kWaveSize + lane];
            const f32x4 b4 = pb[kV + (db * 4 + g) * kWaveSize + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              dkacc[db][4 * g + i] += a4[i];
              dvacc[db][4 * g + i] += b4[i];
            }
          }
      }
    }
  }

  // Each wave stores its keys' rows through ring-slot memory of its own
  // (store_block_rows): with one part, slot kg once every wave is past its
  // last tile; with two, the slot its partner's partial sums came through;
  // with four, the slot part 1's sums came through (read back already).
  if constexpr (SPLIT == 1) wg_barrier();
  if (!wave_active) return;
  const GBuf gdk(dk + part * part_stride + panel_off(ldk, bi, hk), panel_bytes(ldk, t.r_end, D, sizeof(OT)));
  const GBuf gdv(dv + part * part_stride + panel_off(ldv, bi, hk), panel_bytes(ldv, t.r_end, D, sizeof(OT)));
  // RoPE: this key's table row (keys past the tile end are not stored)
  const float *rrow =
      rope == nullptr ? nullptr : rope + (size_t)min(min(key, t.r_end - 1) - t.seg_start, rope_npos - 1) * D;
  static_assert(SPLIT * BMQ * D * sizeof(T) >= 4096, "a 4 KB slot per wave");
  lds_t<f32x4> *scr;
  if constexpr (SPLIT == 1)
    scr = (lds_t<f32x4> *)(kg == 0 ? lds_cast(sQ0) : kg == 1 ? lds_cast(sQ1) : kg == 2 ? lds_cast(sO0) : lds_cast(sO1));
  else
    scr = (lds_t<f32x4> *)lds_cast(kg == 0 ? sQ0 : sO0);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    f32x16 a = dkacc[db] * scale;
    if (rope != nullptr) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a4;
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = a[4 * g + i];
        rope_back(a4, *reinterpret_cast<const f32x4 *>(rrow + db * 32 + 8 * g + 4 * hh));
#pragma unroll
        for (int i = 0; i < 4; ++i) a[4 * g + i] = a4[i];
      }
    }
    store_block_rows<OT>(a, scr, gdk, w0, ldk.ss, db * 32, lane);
    store_block_rows<OT>(dvacc[db], scr, gdv, w0, ldv.ss, db * 32, lane);
  }
}

template <typename T, typename OT, int D, int BMQ, int MINB, bool DOC, int SPLIT>
__global__ __launch_bounds__(256, MINB) void attn_bwd_dkdv_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, OT *__restrict__ dk,
    OT *__restrict__ dv, int S, float c2, float scale, const int32_t *__restrict__ cu, int ntiles, int n_seqs,
    int H, int G, int P, int64_t part_stride, const float *__restrict__ rope, int rope_npos, Layout lq, Layout lk,
    Layout lv, Layout ldo, Layout ldk, Layout ldv) {
  bwd_dkdv_body<T, OT, D, BMQ, DOC, SPLIT>(blockIdx.x, gridDim.x, q, k, v, dO, lse, delta, dk, dv, S, c2, scale, cu,
                                           ntiles, n_seqs, H, G, P, part_stride, rope, rope_npos, lq, lk, lv, ldo,
                                           ldk, ldv);
}

// ---------------------------------------------------------------------------
// dK/dV by wave pairs (16-bit inputs).  A workgroup owns 64 keys; each 32-key
// group has a V-wave and a K-wave.  Per 32-query tile the V-wave computes
// S' = Q K^T - LSE/scale and P = exp2(c2 S') (masked), hands P (fp32) to its
// partner through LDS and adds P^T dO to dV; one tile later the K-wave
// computes dP' = dO V^T - Delta, dS = P dP' with the P it was handed, and
// adds dS^T Q to dK.  These are the one-wave kernel's products and
// per-element arithmetic, in the same order, split into two halves of 17
// matrix-core steps per tile; each wave keeps one accumulator and one of K,
// V in registers, so twice as many waves fit.  Query tiles pass through a
// three-slot ring: at step j the copy into slot (j+1) % 3 starts while the
// V-wave reads slot j % 3 and the K-wave slot (j-1) % 3.
//
// P > 1 parts (grouped heads, with a workspace): the workgroups of one key
// block and K/V head are P, part p running the loop over query heads
// p * G/P .. (p+1) * G/P - 1 only and writing its (scaled) dK and dV to
// dk, dv + p * part_stride; attn_bwd_sum_parts_kernel then adds the parts.
template <typename T, typename OT, int D, int MINB, bool DOC>
__global__ __launch_bounds__(256, MINB) void attn_bwd_dkdv_pair_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, OT *__restrict__ dk,
    OT *__restrict__ dv, int S, float c2, float scale, const int32_t *__restrict__ cu, int ntiles, int n_seqs,
    int H, int G, int P, int64_t part_stride, const float *__restrict__ rope, int rope_npos, Layout lq, Layout lk,
    Layout lv, Layout ldo, Layout ldk, Layout ldv) {
  static_assert(sizeof(T) == 2, "wave pairs: 16-bit inputs");
  constexpr int NW = 4;
  constexpr int NT = NW * kWaveSize;
  constexpr int BN = NW / 2 * 32;  // keys per workgroup
  constexpr int BMQ = 32;          // queries per tile
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  using E = Elem<T>;
  using frag = typename E::frag;
  using QTile = DmaTile<T, BMQ, D, NT, true>;

  __shared__ __attribute__((aligned(1024))) T sQ0[BMQ * D];
  __shared__ __attribute__((aligned(1024))) T sQ1[BMQ * D];
  __shared__ __attribute__((aligned(1024))) T sQ2[BMQ * D];
  __shared__ __attribute__((aligned(1024))) T sO0[BMQ * D];  // dO
  __shared__ __attribute__((aligned(1024))) T sO1[BMQ * D];
  __shared__ __attribute__((aligned(1024))) T sO2[BMQ * D];
  __shared__ __attribute__((aligned(256))) float sL0[64];  // LSE (natural log; 32 used)
  __shared__ __attribute__((aligned(256))) float sL1[64];
  __shared__ __attribute__((aligned(256))) float sL2[64];
  __shared__ __attribute__((aligned(256))) float sD0[64];  // Delta
  __shared__ __attribute__((aligned(256))) float sD1[64];
  __shared__ __attribute__((aligned(256))) float sD2[64];
  // P handed from V-wave to K-wave: [key group][buffer][4-slot group][lane]
  __shared__ __attribute__((aligned(256))) f32x4 sP[NW / 2 * 2 * 4 * kWaveSize];

  const RowTile t = DOC ? doc_tile(cu, blockIdx.x, gridDim.x, ntiles, n_seqs, BN, S, false, kRankDocsDkdv)
                        : causal_tile(blockIdx.x, gridDim.x, ntiles, BN, S, false);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int kg = wave / 2;             // which 32 keys
  const bool vwave = wave % 2 == 0;    // V-wave (S, P, dV) or K-wave (dP, dS, dK)
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  // t.head / P is a key/value head; its G query heads are hk * G .. hk * G +
  // G - 1 of batch entry bi, and dK, dV sum over all of them (the
  // query-tile loop runs over the group, or over part t.head % P of it).
  const int Hkv = H / G;
  const int part = t.head % P;
  const int GP = G / P;
  const int bi = t.head / P / Hkv;
  const int hk = t.head / P % Hkv;
  const int hq0 = hk * G + part * GP;
  const int qh0 = bi * H + hq0;

  const int w0 = t.r_start + kg * 32;  // first key of this wave
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32, t.r_end) - 1;
  const int key = w0 + c;
  const int q_lo = t.r_start;  // the first query that sees any of these keys
  const int ntq = (t.seg_end - q_lo + BMQ - 1) / BMQ;  // query tiles per query head
  const int ntile = GP * ntq;                           // over the group (or this part of it)

  auto qslot = [&]<int P>() { return lds_cast(P == 0 ? sQ0 : P == 1 ? sQ1 : sQ2); };
  auto oslot = [&]<int P>() { return lds_cast(P == 0 ? sO0 : P == 1 ? sO1 : sO2); };
  auto lslot = [&]<int P>() { return lds_cast(P == 0 ? sL0 : P == 1 ? sL1 : sL2); };
  auto dslot = [&]<int P>() { return lds_cast(P == 0 ? sD0 : P == 1 ? sD1 : sD2); };
  uint32_t qoff[QTile::kPerWave], dooff[QTile::kPerWave];
  QTile::lane_offsets(qoff, wave, lane, lq.ss);
  QTile::lane_offsets(dooff, wave, lane, ldo.ss);
  auto issue = [&]<int P>(int it) {
    const int g = it / ntq;
    const int q0 = q_lo + (it - g * ntq) * BMQ;
    const size_t rbase = (size_t)(qh0 + g) * S;
    // Queries past the segment read as zeros (Q, dO, LSE, Delta all 0): their
    // P is 1 but dO and Q are 0, so they add nothing to dV or dK.
    const GBuf gq(q + panel_off(lq, bi, hq0 + g), panel_bytes(lq, t.seg_end, D, sizeof(T)));
    const GBuf gdo(dO + panel_off(ldo, bi, hq0 + g), panel_bytes(ldo, t.seg_end, D, sizeof(T)));
    const GBuf glse(lse + rbase, (uint32_t)(t.seg_end * sizeof(float)));
    const GBuf gdel(delta + rbase, (uint32_t)(t.seg_end * sizeof(float)));
    QTile::issue_at(gq, qslot.template operator()<P>(), QTile::row0_bytes(q0, lq.ss), qoff, wave);
    QTile::issue_at(gdo, oslot.template operator()<P>(), QTile::row0_bytes(q0, ldo.ss), dooff, wave);
    if (wave == 0) dma_vec64(glse, lslot.template operator()<P>(), q0, lane);
    if (wave == 1) dma_vec64(gdel, dslot.template operator()<P>(), q0, lane);
  };
  issue.template operator()<0>(0);

  // K (V-wave) or V (K-wave) fragments of this wave's keys, in registers.
  const GBuf gkv = vwave ? GBuf(k + panel_off(lk, bi, hk), panel_bytes(lk, t.r_end, D, sizeof(T)))
                         : GBuf(v + panel_off(lv, bi, hk), panel_bytes(lv, t.r_end, D, sizeof(T)));
  const int kvss = vwave ? lk.ss : lv.ss;
  frag kvf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) kvf[kb] = global_frag_rs<T>(gkv, key, 16 * kb + 8 * hh, kvss);
  f32x16 acc[DB];  // dV (V-wave) or dK (K-wave)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  const TrSwz<T, D> tr0(lane);    // transposed reads of the Q and dO tiles
  const RowFrag<T, D> rf0(lane);  // row fragments of the same tiles
  const typename E::rows_frag ones = E::rows_b(hh);
  const float rscale = 1.0f / scale;
  lds_t<f32x4> *const xp = lds_cast(sP) + kg * 2 * 4 * kWaveSize;  // this key group's two buffers

  // V-wave, tile `it` in slot P: S', P (masked), P to the K-wave, dV.
  auto vtile = [&]<int P>(int it) {
    const int q0 = q_lo + (it % ntq) * BMQ;
    if (q0 + BMQ - 1 < w0) return;  // every query precedes every key here
    const lds_t<T> *sq = qslot.template operator()<P>();
    const lds_t<T> *so = oslot.template operator()<P>();
    const lds_t<float> *sl = lslot.template operator()<P>();
    const TrSwz<T, D> tr = tr0.pinned();
    const RowFrag<T, D> rf = rf0.pinned();
    f32x16 sacc = f32x16{};
    mma_priority_hi();
    E::mma_rows(sacc, E::rows_a(-sl[c] * rscale, hh), ones);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) E::mma(sacc, rf(sq, 0, kb), kvf[kb]);
    mma_priority_lo();
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(sacc[r] * c2);
    if (q0 < wave_last) {
      // query q0 + off < key, off = 8 (r / 4) + 4 hh + r % 4
      const int lim = key - q0 - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = (8 * (r / 4) + (r % 4)) < lim ? 0.f : sacc[r];
    }
    lds_t<f32x4> *xb = xp + (it & 1) * 4 * kWaveSize;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 p4;
#pragma unroll
      for (int i = 0; i < 4; ++i) p4[i] = sacc[4 * g + i];
      xb[g * kWaveSize + lane] = p4;
    }
    const frag p0 = E::pack(sacc, 0), p1 = E::pack(sacc, 1);
    mma_priority_hi();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      E::mma(acc[db], tr(so, 0, db), p0);
      E::mma(acc[db], tr(so, 16, db), p1);
    }
    mma_priority_lo();
  };

  // K-wave, tile `it` in slot P (its P written one step earlier): dP', dS, dK.
  auto ktile = [&]<int P>(int it) {
    const int q0 = q_lo + (it % ntq) * BMQ;
    if (q0 + BMQ - 1 < w0) return;
    const lds_t<T> *sq = qslot.template operator()<P>();
    const lds_t<T> *so = oslot.template operator()<P>();
    const lds_t<float> *sd = dslot.template operator()<P>();
    const TrSwz<T, D> tr = tr0.pinned();
    const RowFrag<T, D> rf = rf0.pinned();
    f32x16 pacc = f32x16{};
    mma_priority_hi();
    E::mma_rows(pacc, E::rows_a(-sd[c], hh), ones);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) E::mma(pacc, rf(so, 0, kb), kvf[kb]);
    mma_priority_lo();
    const lds_t<f32x4> *xb = xp + (it & 1) * 4 * kWaveSize;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 p4 = xb[g * kWaveSize + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) pacc[4 * g + i] = p4[i] * pacc[4 * g + i];
    }
    const frag s0 = E::pack(pacc, 0), s1 = E::pack(pacc, 1);
    mma_priority_hi();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      E::mma(acc[db], tr(sq, 0, db), s0);
      E::mma(acc[db], tr(sq, 16, db), s1);
    }
    mma_priority_lo();
  };

  // Step j (slot P = j % 3): wait for tile j's copies and this wave's LDS
  // writes, barrier, start the copy of tile j + 1, then the V-wave takes
  // tile j and the K-wave tile j - 1.  ntile + 1 steps for every wave.
  auto step = [&]<int P>(int j) {
    wait_vmcnt_lgkm0<0>();
    wg_barrier();
    if (j + 1 < ntile) issue.template operator()<(P + 1) % 3>(j + 1);
    if (!wave_active) return;
    if (vwave) {
      if (j < ntile) vtile.template operator()<P>(j);
    } else {
      if (j >= 1) ktile.template operator()<(P + 2) % 3>(j - 1);
    }
  };
  for (int j = 0; j <= ntile; j += 3) {
    step.template operator()<0>(j);
    if (j + 1 <= ntile) step.template operator()<1>(j + 1);
    if (j + 2 <= ntile) step.template operator()<2>(j + 2);
  }

  // Every wave is past its last tile: each stores its keys' rows through a
  // ring slot of its own (store_block_rows).
  static_assert(NW == 4 && BMQ * D * sizeof(T) >= 4096, "one 4 KB slot per wave");
  wg_barrier();
  if (!wave_active) return;
  OT *out = (vwave ? dv : dk) + part * part_stride;
  const Layout &lout = vwave ? ldv : ldk;
  const GBuf gout(out + panel_off(lout, bi, hk), panel_bytes(lout, t.r_end, D, sizeof(OT)));
  const float osc = vwave ? 1.0f : scale;
  // RoPE (dK only): this key's table row (keys past the tile end are not stored)
  const float *rrow = (rope == nullptr || vwave)
                          ? nullptr
                          : rope + (size_t)min(min(key, t.r_end - 1) - t.seg_start, rope_npos - 1) * D;
  lds_t<f32x4> *scr = (lds_t<f32x4> *)(wave == 0 ? lds_cast(sQ0) : wave == 1 ? lds_cast(sQ1)
                                       : wave == 2 ? lds_cast(sO0) : lds_cast(sO1));
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    f32x16 a = acc[db] * osc;
    if (rrow != nullptr) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a4;
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = a[4 * g + i];
        rope_back(a4, *reinterpret_cast<const f32x4 *>(rrow + db * 32 + 8 * g + 4 * hh));
#pragma unroll
        for (int i = 0; i < 4; ++i) a[4 * g + i] = a4[i];
      }
    }
    store_block_rows<OT>(a, scr, gout, w0, lout.ss, db * 32, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ.  A workgroup owns BM = 128 queries of one head (32 per wave) and loops
// over key tiles of BN rows up to its causal diagonal.  K and V tiles arrive
// by direct global->LDS copies into two ring slots one iteration ahead; K is
// read both as row fragments and, through the transposing load, as K^T.
template <int LPR, int M, int J, int KB>
__device__ __forceinline__ float delta_tree(const float (&part)[KB]) {
  if constexpr (M == LPR)
    return part[J];
  else
    return delta_tree<LPR, 2 * M, J, KB>(part) + delta_tree<LPR, 2 * M, J + M / 2, KB>(part);
}

// FUSE_DELTA (bf16 inputs): the kernel also computes Delta_i = sum_d dO_id O_id
// for its queries from O, in the same summation order as the preprocess
// kernel (so the result is bitwise the same), uses it, and writes it to
// `delta_out` for the dK/dV kernel that runs after it.
template <typename T, typename OT, int D, int BN, bool DOC, bool FUSE_DELTA>
__device__ __forceinline__ void bwd_dq_body(
    int bid, int nblocks, const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dO, const float *__restrict__ lse, const float *__restrict__ delta,
    const OT *__restrict__ o, float *__restrict__ delta_out, OT *__restrict__ dq, int S, float c2, float scale,
    const int32_t *__restrict__ cu, int ntiles, int n_seqs, int H, int G, const float *__restrict__ rope,
    int rope_npos, Layout lq, Layout lk, Layout lv, Layout ldo, Layout lo, Layout ldq) {
  constexpr int NW = 4;
  constexpr int NT = NW * kWaveSize;
  constexpr int BM = NW * 32;
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int NB = BN / 32;
  using E = Elem<T>;
  using frag = typename E::frag;
  using KTile = DmaTile<T, BN, D, NT, true>;

  __shared__ __attribute__((aligned(1024))) T sK0[BN * D];
  __shared__ __attribute__((aligned(1024))) T sK1[BN * D];
  __shared__ __attribute__((aligned(1024))) T sV0[BN * D];
  __shared__ __attribute__((aligned(1024))) T sV1[BN * D];

  const RowTile t = DOC ? doc_tile(cu, bid, nblocks, ntiles, n_seqs, BM, S, true, kRankDocsDq)
                        : causal_tile(bid, nblocks, ntiles, BM, S, true);
  if (!t.valid) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid % kWaveSize;
  const int hh = lane / 32;
  const int c = lane % 32;
  const int bi = t.head / H;  // batch entry
  const int hq = t.head % H;  // query head, and its key/value head hq / G
  const size_t rbase = (size_t)t.head * S;
  const GBuf gq(q + panel_off(lq, bi, hq), panel_bytes(lq, t.r_end, D, sizeof(T)));
  const GBuf gdo(dO + panel_off(ldo, bi, hq), panel_bytes(ldo, t.r_end, D, sizeof(T)));
  const GBuf gk(k + panel_off(lk, bi, hq / G), panel_bytes(lk, t.seg_end, D, sizeof(T)));
  const GBuf gv(v + panel_off(lv, bi, hq / G), panel_bytes(lv, t.seg_end, D, sizeof(T)));
  const GBuf glse(lse + rbase, (uint32_t)(t.r_end * sizeof(float)));
  const GBuf gdel(delta + rbase, (uint32_t)(t.r_end * sizeof(float)));

  const int w0 = t.r_start + wave * 32;  // first query of this wave
  const bool wave_active = w0 < t.r_end;
  const int wave_last = min(w0 + 32, t.r_end) - 1;
  const int qi = w0 + c;
  const int kv_lo = t.seg_start;
  const int kv_hi = min(t.r_end, t.seg_end);
  const int ntile = (kv_hi - kv_lo + BN - 1) / BN;
  const int jw = wave_active ? (wave_last - kv_lo) / BN + 1 : 0;  // tiles this wave needs

  auto kslot = [&]<int P>() { return lds_cast(P == 0 ? sK0 : sK1); };
  auto vslot = [&]<int P>() { return lds_cast(P == 0 ? sV0 : sV1); };
  uint32_t koff[KTile::kPerWave], voff[KTile::kPerWave];
  KTile::lane_offsets(koff, wave, lane, lk.ss);
  KTile::lane_offsets(voff, wave, lane, lv.ss);
  auto issue = [&]<int P>(int j) {
    const int r0 = kv_lo + j * BN;
    KTile::issue_at(gk, kslot.template operator()<P>(), KTile::row0_bytes(r0, lk.ss), koff, wave);
    KTile::issue_at(gv, vslot.template operator()<P>(), KTile::row0_bytes(r0, lv.ss), voff, wave);
  };
  issue.template operator()<0>(0);

  frag qf[KB], df[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    qf[kb] = global_frag_rs<T>(gq, qi, 16 * kb + 8 * hh, lq.ss);
    df[kb] = global_frag_rs<T>(gdo, qi, 16 * kb + 8 * hh, ldo.ss);
  }
  const float l2 = glse.load4((uint32_t)qi * 4) * kLog2e;
  float dl;
  if constexpr (FUSE_DELTA) {
    static_assert(sizeof(T) == 2, "fused Delta follows the 16-bit preprocess layout");
    // The preprocess kernel gives lane `sub` of a row elements 8*sub .. 8*sub+7
    // (an FMA chain from 0) and reduces the D/8 partial sums by butterfly.
    // Fragment kb of this lane is sub-block 2*kb + hh, so the lane computes
    // the butterfly's tree over its own sub-blocks and one swap across the
    // halves adds the other half's.
    const GBuf go(o + panel_off(lo, bi, hq), panel_bytes(lo, t.r_end, D, sizeof(OT)));
    float part[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float ov[8];
      load_out8<OT>(go, (uint32_t)(qi * lo.ss + 16 * kb + 8 * hh), ov);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (float)df[kb][i] * ov[i];
      part[kb] = acc;
    }
    const float mine = delta_tree<2 * KB, 2, 0, KB>(part);
    dl = mine + swap_halves(mine);
    if (hh == 0 && qi < t.r_end) delta_out[rbase + qi] = dl;
  } else {
    dl = gdel.load4((uint32_t)qi * 4);
  }
  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  const TrSwz<T, D> tr0(lane);    // transposed reads of the K tile
  const RowFrag<T, D> rf0(lane);  // row fragments of the K and V tiles

  // One key tile: per 32-key block, S^T = K Q^T and dP^T = V dO^T (lane c owns
  // query w0 + c), P, dS = P (dP - Delta), then dQ^T += K^T dS^T.
  constexpr bool kPipe = NB == 2 && sizeof(T) == 2 && D == 64;
  auto tile = [&]<int P>(int k0, bool masked) {
    const lds_t<T> *sk = kslot.template operator()<P>();
    const lds_t<T> *sv = vslot.template operator()<P>();
    const TrSwz<T, D> tr = tr0.pinned();
    const RowFrag<T, D> rf = rf0.pinned();
    const int lim = qi - k0 - 4 * hh;  // the mask's per-lane limit
    sched_hint<D != 64>();
    if constexpr (kPipe) {
      // Two 32-key blocks, software-pipelined inside the wave as in dK/dV:
      // block 1's score products issue among block 0's softmax, block 0's
      // dQ products among block 1's softmax; the mask branches sit between
      // these groups.  A masked score becomes -inf before the exponential
      // (exactly 0 after it).
      f32x16 sa0 = f32x16{}, pa0 = f32x16{}, sa1 = f32x16{}, pa1 = f32x16{};
      auto scores = [&](int nb, f32x16 &sacc, f32x16 &pacc) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          E::mma(sacc, rf(sk, nb, kb), qf[kb]);
          E::mma(pacc, rf(sv, nb, kb), df[kb]);
        }
      };
      auto mask = [&](int nb, f32x16 &sacc) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = (32 * nb + 8 * (r / 4) + (r % 4)) > lim ? -INFINITY : sacc[r];
      };
      auto soft = [&](f32x16 &sacc, f32x16 &pacc, frag (&ss)[2]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(__builtin_fmaf(sacc[r], c2, -l2));
#pragma unroll
        for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * (pacc[r] - dl);
        ss[0] = E::pack(pacc, 0);
        ss[1] = E::pack(pacc, 1);
      };
      auto accum = [&](int nb, const frag (&ss)[2]) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          E::mma(dqacc[db], tr(sk, 32 * nb, db), ss[0]);
          E::mma(dqacc[db], tr(sk, 32 * nb + 16, db), ss[1]);
        }
      };
      frag ss0[2], ss1[2];
      scores(0, sa0, pa0);
      if (masked) mask(0, sa0);
      scores(1, sa1, pa1);
      soft(sa0, pa0, ss0);
      // keep block 0's softmax in this group (see the dK/dV kernel)
#pragma unroll
      for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(ss0[i]));
      if (masked) mask(1, sa1);
      accum(0, ss0);
      soft(sa1, pa1, ss1);
      accum(1, ss1);
      return;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      mma_priority_hi();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        E::mma(sacc, rf(sk, nb, kb), qf[kb]);
        E::mma(pacc, rf(sv, nb, kb), df[kb]);
      }
      mma_priority_lo();
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = fast_exp2(__builtin_fmaf(sacc[r], c2, -l2));
      if (masked) {
        // key k0 + 32 nb + 8 (r / 4) + 4 hh + r % 4 > qi (also keys past the
        // segment end: stored rows have qi < seg_end); lim is per lane
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = (32 * nb + 8 * (r / 4) + (r % 4)) > lim ? 0.f : sacc[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = sacc[r] * (pacc[r] - dl);
      const frag s0 = E::pack(pacc, 0), s1 = E::pack(pacc, 1);
      mma_priority_hi();
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        E::mma(dqacc[db], tr(sk, 32 * nb, db), s0);
        E::mma(dqacc[db], tr(sk, 32 * nb + 16, db), s1);
      }
      mma_priority_lo();
    }
  };

  auto step = [&]<int P>(int j) {
    wait_vmcnt<0>();
    wg_barrier();
    if (j + 1 < ntile) issue.template operator()<1 - P>(j + 1);
    if (j >= jw) return;
    const int k0 = kv_lo + j * BN;
    tile.template operator()<P>(k0, (k0 + BN - 1 > w0) || (k0 + BN > t.seg_end));
  };
  for (int j = 0; j < ntile; j += 2) {
    step.template operator()<0>(j);
    if (j + 1 < ntile) step.template operator()<1>(j + 1);
  }

  // Every wave is past its last read of the ring slots: each wave stores its
  // rows through one slot (store_block_rows).
  static_assert(BN * D * sizeof(T) >= 4096, "one 4 KB slot per wave");
  wg_barrier();
  if (!wave_active) return;
  const GBuf gdq(dq + panel_off(ldq, bi, hq), panel_bytes(ldq, t.r_end, D, sizeof(OT)));
  // RoPE: this query's table row (queries past the tile end are not stored)
  const float *rrow =
      rope == nullptr ? nullptr : rope + (size_t)min(min(qi, t.r_end - 1) - t.seg_start, rope_npos - 1) * D;
  lds_t<f32x4> *scr = (lds_t<f32x4> *)(wave == 0 ? kslot.template operator()<0>()
                                       : wave == 1 ? kslot.template operator()<1>()
                                       : wave == 2 ? vslot.template operator()<0>()
                                                   : vslot.template operator()<1>());
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    f32x16 a = dqacc[db] * scale;
    if (rope != nullptr) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 a4;
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = a[4 * g + i];
        rope_back(a4, *reinterpret_cast<const f32x4 *>(rrow + db * 32 + 8 * g + 4 * hh));
#pragma unroll
        for (int i = 0; i < 4; ++i) a[4 * g + i] = a4[i];
      }
    }
    store_block_rows<OT>(a, scr, gdq, w0, ldq.ss, db * 32, lane);
  }
}

template <typename T, typename OT, int D, int BN, int MINB, bool DOC, bool FUSE_DELTA>
__global__ __launch_bounds__(256, MINB) void attn_bwd_dq_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, const OT *__restrict__ o,
    float *__restrict__ delta_out, OT *__restrict__ dq, int S, float c2, float scale,
    const int32_t *__restrict__ cu, int ntiles, int n_seqs, int H, int G, const float *__restrict__ rope,
    int rope_npos, Layout lq, Layout lk, Layout lv, Layout ldo, Layout lo, Layout ldq) {
  bwd_dq_body<T, OT, D, BN, DOC, FUSE_DELTA>(blockIdx.x, gridDim.x, q, k, v, dO, lse, delta, o, delta_out, dq, S,
                                             c2, scale, cu, ntiles, n_seqs, H, G, rope, rope_npos, lq, lk, lv, ldo,
                                             lo, ldq);
}

// ---------------------------------------------------------------------------
// Launchers.

// Small causal grids at D = 64 (16-bit inputs, one K/V head per query head):
// the dK/dV workgroups (blocks 0 .. n_kv - 1) and the dQ workgroups (the
// rest, 64-key tiles) in one launch, Delta coming from the preprocess kernel.
// With fewer workgroups than the GPU holds, the two kernels run back to back
// each with idle wave slots and a tail of its longest chains; in one launch
// they share the CUs.  Each workgroup runs exactly the code of its own
// kernel (bwd_dkdv_body, bwd_dq_body), so the results are bitwise those of
// the two launches.  Measured on MI355X, B16 H6 S512 D64 bf16: dQ and dK/dV
// on two streams without synchronisation took 21.7 us per pair against 31.9
// one after the other (B8 H16 S1024: 77.9 against 80.4).
template <typename T, typename OT>
__global__ __launch_bounds__(256, 1) void attn_bwd_small_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const T *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, OT *__restrict__ dq, OT *__restrict__ dk,
    OT *__restrict__ dv, int S, float c2, float scale, int ntiles, int H, const float *__restrict__ rope,
    int rope_npos, Layout lq, Layout lk, Layout lv, Layout ldo, Layout ldq, Layout ldk, Layout ldv, int n_kv) {
  if ((int)blockIdx.x < n_kv)
    bwd_dkdv_body<T, OT, 64, 64, false, 1>(blockIdx.x, n_kv, q, k, v, dO, lse, delta, dk, dv, S, c2, scale, nullptr,
                                          ntiles, 1, H, 1, 1, 0, rope, rope_npos, lq, lk, lv, ldo, ldk, ldv);
  else
    bwd_dq_body<T, OT, 64, 64, false, false>(blockIdx.x - n_kv, gridDim.x - n_kv, q, k, v, dO, lse, delta, nullptr,
                                             nullptr, dq, S, c2, scale, nullptr, ntiles, 1, H, 1, rope, rope_npos,
                                             lq, lk, lv, ldo, ldq, ldq);
}

// Tile shapes: query tile of the dK/dV kernel (BMQ), key tile of the dQ
// kernel (BN, see dq_bn), and the minimum workgroups per CU each register
// allocation must allow.  Two 64-row slots of Q and dO (or K and V) at D = 128, or in
// fp32, would leave room for one workgroup per CU: those take 32 rows.
template <typename T, int D> struct BwdCfg {
  static constexpr int BMQ = (D == 128 || sizeof(T) == 4) ? 32 : 64;
  static constexpr int BN = (D == 128 && sizeof(T) == 4) ? 32 : 64;
  static constexpr int MINB_DKDV = 1;
  static constexpr int MINB_DQ = 1;
  // dQ key tile: 32 keys leave the bf16 kernel enough registers for more
  // waves per SIMD (D = 64: 124 VGPRs, four; D = 128: two instead of one),
  // measured 9 % (context 1024) and 26 % (S = 8192, D = 128) faster.  Packed
  // documents at D = 64 had run 12 % faster with 64 under the per-document
  // grid of every kernel; with the forward and dK/dV on the ranked schedule
  // 32 is 2 % faster there (same-process A/B, backward 83.1 -> 81.6 us,
  // bitwise equal: the key blocks are accumulated in the same order).  A
  // 32-row tile at D = 32 is too small to split over four waves.
  template <bool DOC>
  static constexpr int dq_bn() {
    return (sizeof(T) == 2 && D > 32) ? 32 : BN;
  }
};

template <typename T, typename OT, int D>
static hipError_t launch_pre_t(const Args &a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int RPB = 256 / (D / VEC);
  const int rows = a.B * a.H * a.S;
  const int blocks = min((rows + RPB - 1) / RPB, 65536);
  hipLaunchKernelGGL((attn_bwd_preprocess_kernel<T, OT, D>), dim3(blocks), dim3(256), 0, a.stream,
                     static_cast<const OT *>(a.o_in), static_cast<const T *>(a.dO), a.delta, rows, a.S, a.H, a.lo,
                     a.ldo);
  return hipGetLastError();
}

// P parts: outputs dk_out, dv_out as in launch_dkdv_pair.
template <typename T, typename OT, int D, bool DOC, int SPLIT>
static hipError_t launch_dkdv_split(const Args &a, int P = 1, OT *dk_out = nullptr, OT *dv_out = nullptr,
                                    int64_t part_stride = 0) {
  // four parts at D = 64 take 32-query tiles: four 64-row rings would leave
  // room for one workgroup per CU
  constexpr int BMQ = (SPLIT == 4 && D == 64) ? 32 : BwdCfg<T, D>::BMQ;
  constexpr int MINB = BwdCfg<T, D>::MINB_DKDV;
  constexpr int BN = 4 * 32 / SPLIT;  // keys per workgroup
  const float c2 = a.scale * kLog2e;
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BN - 1) / BN;
    grid = dim3(a.H_kv * P * doc_blocks_per_unit(a.n_seqs, ntiles, a.S, BN, kRankDocsDkdv));
  } else {
    ntiles = (a.S + BN - 1) / BN;
    grid = dim3(ntiles * a.B * a.H_kv * P);
  }
  Layout ldk = a.ldk, ldv = a.ldv;
  if (P > 1) ldk = ldv = Layout{(int64_t)a.H_kv * a.S * a.D, (int64_t)a.S * a.D, a.D};
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, OT, D, BMQ, MINB, DOC, SPLIT>), grid, dim3(256), 0, a.stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<const T *>(a.dO), a.lse_in, a.delta_in,
                     P > 1 ? dk_out : static_cast<OT *>(a.dk), P > 1 ? dv_out : static_cast<OT *>(a.dv), a.S, c2,
                     a.scale, a.cu_seqlens, ntiles, a.n_seqs, a.H, a.H / a.H_kv, P, part_stride, a.rope,
                     a.rope_npos, a.lq, a.lk, a.lv, a.ldo, ldk, ldv);
  return hipGetLastError();
}

// P parts: the outputs are dk_out, dv_out (P fp32 partial sets part_stride
// elements apart, contiguous [B, H_kv, S, D] each) instead of a.dk, a.dv.
template <typename T, typename OT, int D, bool DOC>
static hipError_t launch_dkdv_pair(const Args &a, int P = 1, OT *dk_out = nullptr, OT *dv_out = nullptr,
                                   int64_t part_stride = 0) {
  constexpr int BN = 64;  // keys per workgroup
  const float c2 = a.scale * kLog2e;
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BN - 1) / BN;
    grid = dim3(a.H_kv * P * doc_blocks_per_unit(a.n_seqs, ntiles, a.S, BN, kRankDocsDkdv));
  } else {
    ntiles = (a.S + BN - 1) / BN;
    grid = dim3(ntiles * a.B * a.H_kv * P);
  }
  Layout ldk = a.ldk, ldv = a.ldv;
  if (P > 1) ldk = ldv = Layout{(int64_t)a.H_kv * a.S * a.D, (int64_t)a.S * a.D, a.D};
  hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<T, OT, D, 1, DOC>), grid, dim3(256), 0, a.stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<const T *>(a.dO), a.lse_in, a.delta_in,
                     P > 1 ? dk_out : static_cast<OT *>(a.dk), P > 1 ? dv_out : static_cast<OT *>(a.dv), a.S, c2,
                     a.scale, a.cu_seqlens, ntiles, a.n_seqs, a.H, a.H / a.H_kv, P, part_stride, a.rope,
                     a.rope_npos, a.lq, a.lk, a.lv, a.ldo, ldk, ldv);
  return hipGetLastError();
}

// 16-bit inputs.  At D = 128, where one wave holding both accumulators
// leaves room for one wave per SIMD, wave pairs (two per SIMD); at D = 64 the
// pairs are slower (LDS for three workgroups per CU, a barrier per 17
// products).  Grouped heads with an even group size can instead split the
// group over two (or, G a multiple of four, four) waves per key group, which
// halves (quarters) the longest workgroup's chain of query tiles.  Measured
// on MI355X (backward, bf16, D = 128, 12 shapes with 2 to 8 K/V heads and S
// from 1024 to 8192): with 64-key units B * H_kv * ceil(S / 64) >= 1024, two
// rounds of the pair kernel's resident workgroups on 256 CUs, the pairs are
// 9-13 % faster than the two-way split; at 512 units within 3 % either way;
// at 256 units 27-29 % slower, the step then waiting on the heads chained in
// the first key tiles.  Four ways against two, B1 H16 S8192 D128: 4 K/V heads
// 1.68 -> 1.47 ms, 2 heads 1.89 -> 1.56, 1 head 3.40 -> 2.33; B8 H16 S1024
// D64: 1 K/V head 209 -> 178 us, 2 heads 132 -> 120, but 4 heads (G = 4)
// 99 -> 109 us, so at D <= 64 four ways only from G = 8.  Else one wave per
// 32 keys.
template <typename T, typename OT, int D, bool DOC>
static hipError_t launch_dkdv_t(const Args &a) {
  if constexpr (sizeof(T) == 2) {
    const int G = a.H / a.H_kv;
    const bool even_group = G % 2 == 0;
    if constexpr (D == 128) {
      const int64_t units = (int64_t)a.B * a.H_kv * ((a.S + 63) / 64);
      if (!even_group || units >= 1024) return launch_dkdv_pair<T, OT, D, DOC>(a);
    }
    if (G % 4 == 0 && (D == 128 || G >= 8)) return launch_dkdv_split<T, OT, D, DOC, 4>(a);
    if (even_group) return launch_dkdv_split<T, OT, D, DOC, 2>(a);
  }
  return launch_dkdv_split<T, OT, D, DOC, 1>(a);
}

template <typename T, typename OT, int D, bool DOC, bool FUSE_DELTA, int BN = BwdCfg<T, D>::template dq_bn<DOC>()>
static hipError_t launch_dq_t(const Args &a) {
  // 16-bit causal D = 64: the 32-key tile's registers allow four waves per
  // SIMD, which only pays when the grid brings them.  A grid of fewer than
  // three workgroups per CU (under 768 on 256 CUs) takes 64-key tiles, whose
  // two blocks are software-pipelined (170 VGPRs, two waves per SIMD).
  // Measured on MI355X, backward, 64-key against 32-key tiles (the choice
  // does not change the results): 256 workgroups (B2 H16 S1024) 48.2 against
  // 53.2 us, 384 (ctx 512) 36.8 / 39.0, 512 (B1 H16 S4096) 157.7 / 174.6; at
  // 768 (B32 H6 S512) 57.8 / 54.6 and at 1024 the 32-key tiles lead.
  if constexpr (sizeof(T) == 2 && D == 64 && !DOC && BN == 32) {
    if ((int64_t)a.B * a.H * ((a.S + 127) / 128) < 768)
      return launch_dq_t<T, OT, D, DOC, FUSE_DELTA, 64>(a);
  }
  constexpr int MINB = BwdCfg<T, D>::MINB_DQ;
  constexpr int BM = 4 * 32;
  const float c2 = a.scale * kLog2e;
  dim3 grid;
  int ntiles;
  if (DOC) {
    ntiles = (a.max_seqlen + BM - 1) / BM;
    grid = dim3(a.H * doc_blocks_per_unit(a.n_seqs, ntiles, a.S, BM, kRankDocsDq));
  } else {
    ntiles = (a.S + BM - 1) / BM;
    grid = dim3(ntiles * a.B * a.H);
  }
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, OT, D, BN, MINB, DOC, FUSE_DELTA>), grid, dim3(256), 0, a.stream,
                     static_cast<const T *>(a.q), static_cast<const T *>(a.k), static_cast<const T *>(a.v),
                     static_cast<const T *>(a.dO), a.lse_in, a.delta_in, static_cast<const OT *>(a.o_in), a.delta,
                     static_cast<OT *>(a.dq), a.S, c2, a.scale, a.cu_seqlens, ntiles, a.n_seqs, a.H, a.H / a.H_kv,
                     a.rope, a.rope_npos, a.lq, a.lk, a.lv, a.ldo, a.lo, a.ldq);
  return hipGetLastError();
}

// Dispatch on D, then on the mask.
template <typename T, typename OT>
static hipError_t launch_pre_dt(const Args &a) {
  switch (a.D) {
    case 32: return launch_pre_t<T, OT, 32>(a);
    case 64: return launch_pre_t<T, OT, 64>(a);
    default: return launch_pre_t<T, OT, 128>(a);
  }
}

template <typename T, typename OT, bool DOC>
static hipError_t launch_dkdv_d(const Args &a) {
  switch (a.D) {
    case 32: return launch_dkdv_t<T, OT, 32, DOC>(a);
    case 64: return launch_dkdv_t<T, OT, 64, DOC>(a);
    default: return launch_dkdv_t<T, OT, 128, DOC>(a);
  }
}

template <typename T, typename OT, bool DOC, bool FUSE_DELTA>
static hipError_t launch_dq_d(const Args &a) {
  switch (a.D) {
    case 32: return launch_dq_t<T, OT, 32, DOC, FUSE_DELTA>(a);
    case 64: return launch_dq_t<T, OT, 64, DOC, FUSE_DELTA>(a);
    default: return launch_dq_t<T, OT, 128, DOC, FUSE_DELTA>(a);
  }
}

}  // namespace attn
