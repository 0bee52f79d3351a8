// attn_device.h - device building blocks shared by the attention kernels (gfx950).
//
// Matrix-core tiling.  Every contraction is built from one 32x32 output block
// per wave and 16-deep reduction steps ("k-blocks"):
//   * bf16 inputs: one v_mfma_f32_32x32x16_bf16 per k-block;
//   * fp32 inputs: eight v_mfma_f32_32x32x2_f32 per k-block (true fp32).
// Lane l = 32*h + c (h = l/32 the wave half, c = l%32) feeds eight k-slots of
// one k-block: A[row c][slot s of half h] and B[slot s of half h][col c], and
// receives the 32x32 result C with register r holding
//     C[row 8*(r/4) + 4*h + r%4][col c].
// Which logical k index a (half, slot) pair stands for is free, as long as A
// and B agree.  Two orders are used:
//   natural   slot (h, s) of k-block kb  <->  k = 16*kb + 8*h + s
//   accum     slot (h, s) of k-block kb  <->  k = 16*kb + 8*(s/4) + 4*h + s%4
// The "accum" order is exactly how a 32x32 result (e.g. P^T, dS) already sits
// in a lane's registers 8*kb .. 8*kb+7, so a result can feed the next
// contraction as its B operand with no data movement at all.  Operands staged
// in LDS for that contraction are stored with their row index permuted to
// match (swap bits 2 and 3 within each 16-row group), so each lane still reads
// its 8 slots with one 16-byte LDS load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int kWaveSize = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element traits: the 8-slot fragment type and the 32x32x16 step.
template <typename T> struct Elem;

template <> struct Elem<bf16> {
  using frag = bf16x8;                  // 8 x bf16 = 16 bytes
  static constexpr int kFragWords = 4;  // 32-bit words per fragment
  __device__ __forceinline__ static void mma(f32x16 &acc, const frag &a, const frag &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  // Round slots 8*j .. 8*j+7 of a 32x32 result to a fragment (RNE).
  __device__ __forceinline__ static frag pack(const f32x16 &acc, int j) {
    frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = (bf16)acc[8 * j + s];
    return f;
  }
};

template <> struct Elem<float> {
  using frag = f32x8;                   // 8 x fp32 = 32 bytes
  static constexpr int kFragWords = 8;
  __device__ __forceinline__ static void mma(f32x16 &acc, const frag &a, const frag &b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static frag pack(const f32x16 &acc, int j) {
    frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = acc[8 * j + s];
    return f;
  }
};

// Row permutation of the "accum" order: swap bits 2 and 3 of the row index.
__device__ __forceinline__ constexpr int perm16(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Load an 8-slot fragment from LDS (16- or 32-byte aligned).
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag lds_frag(const T *p) {
  return *reinterpret_cast<const typename Elem<T>::frag *>(p);
}

// ---------------------------------------------------------------------------
// Global memory through buffer resources.  A resource covers `nbytes` from
// `base`; loads past the end return zeros and stores past the end are
// dropped by the hardware range check, so ragged tiles need no branches (and
// the compiler can track outstanding loads exactly).  All offsets are
// per-lane byte offsets (voffset), so the range check applies to them.
struct GBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ GBuf(const void *base, uint32_t nbytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, 0x00020000)) {}
  __device__ __forceinline__ u32x4 load16(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
  __device__ __forceinline__ float load4(uint32_t off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
  __device__ __forceinline__ void store16(const f32x4 &v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
  }
  __device__ __forceinline__ void store4(float v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
  }
};

// An 8-slot fragment of row `row`, columns [col, col + 8), of a row-major
// [*, D] array behind `g` (zeros past the resource's end).
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag global_frag(const GBuf &g, int row, int col) {
  using frag = typename Elem<T>::frag;
  const uint32_t off = (uint32_t)(row * D + col) * sizeof(T);
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(frag, g.load16(off));
  } else {
    const u32x4 a = g.load16(off);
    const u32x4 b = g.load16(off + 16);
    u32x8 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = a[i];
      w[4 + i] = b[i];
    }
    return __builtin_bit_cast(frag, w);
  }
}

// ---------------------------------------------------------------------------
// LDS tile geometry for a block of R rows x D columns of T.
//   RM (row-major):  element (r, d) at r * ld_rm + d,           ld_rm = D + pad
//   TR (transposed): element (r, d) at d * ld_tr + perm16(r),   ld_tr = R + pad
// The 16-byte row padding keeps 16-byte fragment loads of consecutive rows on
// distinct LDS banks.
template <typename T, int R, int D> struct TileGeom {
  static constexpr int kPad = 16 / sizeof(T);
  static constexpr int kLdRM = D + kPad;
  static constexpr int kLdTR = R + kPad;
  static constexpr int kSizeRM = R * kLdRM;  // elements
  static constexpr int kSizeTR = D * kLdTR;
};

// Cooperative copy of rows [r0, r0 + R) of a row-major [*, D] array into LDS;
// rows past the buffer resource's end read as zeros.  Each thread moves
// 16-byte chunks of two adjacent rows (2p, 2p+1); a wave's load instruction
// covers whole rows, so global reads are fully coalesced.  Split into a
// global->register phase and a register->LDS phase so the next tile can be
// fetched while the current one is in use.
template <typename T, int R, int D, int NT> struct TileLoader {
  static constexpr int kVec = 16 / sizeof(T);      // elements per chunk
  static constexpr int kCPR = D / kVec;            // chunks per row
  static constexpr int kPairsPerPass = NT / kCPR;  // row pairs per pass
  static constexpr int kPasses = (R / 2 + kPairsPerPass - 1) / kPairsPerPass;
  static_assert(D % kVec == 0, "D must be a multiple of the chunk");
  static_assert(NT % kCPR == 0, "thread count must cover whole rows");
  static_assert(R % 16 == 0, "tile rows must be a multiple of 16");
  // every thread has rows in every pass (no guard needed)
  static constexpr bool kExact = kPasses * kPairsPerPass * 2 == R;
  using G = TileGeom<T, R, D>;

  u32x4 regs[kPasses][2];

  __device__ __forceinline__ void load(const GBuf &g, int r0, int tid) {
    const int c = tid % kCPR;
    const int p = tid / kCPR;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int lr = 2 * (ps * kPairsPerPass + p);
      if (kExact || lr < R) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
          regs[ps][e] = g.load16((uint32_t)((r0 + lr + e) * D + c * kVec) * sizeof(T));
      }
    }
  }

  __device__ __forceinline__ void store_rm(T *rm, int tid) const {
    const int c = tid % kCPR;
    const int p = tid / kCPR;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int lr = 2 * (ps * kPairsPerPass + p);
      if (kExact || lr < R) {
        *reinterpret_cast<u32x4 *>(rm + lr * G::kLdRM + c * kVec) = regs[ps][0];
        *reinterpret_cast<u32x4 *>(rm + (lr + 1) * G::kLdRM + c * kVec) = regs[ps][1];
      }
    }
  }

  // Transposed store: rows lr and lr+1 land side by side (perm16 keeps bit 0),
  // so each column element pair is one 32-bit (bf16) or 64-bit (fp32) write.
  __device__ __forceinline__ void store_tr(T *tr, int tid) const {
    const int c = tid % kCPR;
    const int p = tid / kCPR;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int lr = 2 * (ps * kPairsPerPass + p);
      if (kExact || lr < R) {
        const int col = perm16(lr);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < kVec; ++i) {
            const uint32_t a = (regs[ps][0][i / 2] >> (16 * (i & 1))) & 0xffffu;
            const uint32_t b = (regs[ps][1][i / 2] >> (16 * (i & 1))) & 0xffffu;
            *reinterpret_cast<uint32_t *>(tr + (c * kVec + i) * G::kLdTR + col) = a | (b << 16);
          }
        } else {
#pragma unroll
          for (int i = 0; i < kVec; ++i) {
            uint2 w;
            w.x = regs[ps][0][i];
            w.y = regs[ps][1][i];
            *reinterpret_cast<uint2 *>(tr + (c * kVec + i) * G::kLdTR + col) = w;
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Cross-half reductions (lanes c and c + 32 hold the two halves of a column).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, kWaveSize);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize); }

// ---------------------------------------------------------------------------
// Work decomposition.  A "row tile" is BM consecutive rows of one head that one
// workgroup owns; its key range is bounded by the causal diagonal and, for
// packed documents, by its document.
struct RowTile {
  int head;      // b * H + h
  int r_start;   // first row of the tile (sequence index)
  int r_end;     // one past the last valid row of the tile
  int seg_start; // first key the tile may attend (document start or 0)
  int seg_end;   // one past the last key of the segment (document end or S)
  bool valid;
};

// Causal mode: tiles of BM rows, `ntiles` per head.  Block ids are remapped so
// that each XCD (block id mod 8 on MI355X) receives a contiguous range of
// heads, keeping one head's K and V in one XCD's L2, and within a head the
// tiles are visited longest-first (most key tiles first), which shortens the
// tail of the causal triangle.
__device__ __forceinline__ RowTile causal_tile(int bid, int nblocks, int ntiles, int BM, int S,
                                               bool heavy_first) {
  int id = bid;
  if ((nblocks & 7) == 0) {
    const int per_xcd = nblocks >> 3;
    id = (bid & 7) * per_xcd + (bid >> 3);
  }
  RowTile t;
  t.head = id / ntiles;
  int ti = id % ntiles;
  if (heavy_first) ti = ntiles - 1 - ti;
  t.r_start = ti * BM;
  t.r_end = min(t.r_start + BM, S);
  t.seg_start = 0;
  t.seg_end = S;
  t.valid = true;
  return t;
}

// Packed-document mode: grid (tiles per longest document, documents, heads).
__device__ __forceinline__ RowTile doc_tile(const int32_t *__restrict__ cu, int tile_x, int ntiles_x,
                                            int doc, int head, int BM, bool heavy_first) {
  RowTile t;
  const int ds = cu[doc];
  const int de = cu[doc + 1];
  const int ti = heavy_first ? (ntiles_x - 1 - tile_x) : tile_x;
  t.head = head;
  t.r_start = ds + ti * BM;
  t.r_end = min(t.r_start + BM, de);
  t.seg_start = ds;
  t.seg_end = de;
  t.valid = t.r_start < de;
  return t;
}

}  // namespace attn
