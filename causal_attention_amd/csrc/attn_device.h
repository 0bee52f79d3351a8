// attn_device.h - device building blocks shared by the attention kernels (gfx950).
//
// Matrix-core tiling.  Every contraction is built from one 32x32 output block
// per wave and 16-deep reduction steps ("k-blocks"):
//   * bf16 / fp16 inputs: one v_mfma_f32_32x32x16_{bf16,f16} per k-block;
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
// contraction as its B operand with no data movement at all.  An operand that
// must match it (the A operand of a product reducing over the rows of a
// row-major LDS tile) is read with the transposing LDS load, which delivers
// those rows in the same order (TrRead below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "attn_launch.h"  // Layout

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int kWaveSize = 64;

// Instruction-scheduling strategy requested for a tile loop: the compiler's
// instruction-group strategy 3, which interleaves exponentials with
// matrix-core instructions (a hint only; no effect on results).  Measured on
// MI355X it helps the forward and the D = 128 backward by a few percent; for
// the D = 64 backward kernels, whose tile bodies are pipelined by hand, it
// serialises each LDS read with its product and the backward runs 2-3 %
// faster without it.
template <bool ON> __device__ __forceinline__ void sched_hint() {
  if constexpr (ON) __builtin_amdgcn_iglp_opt(3);
}

// Pointers into LDS carry their address space explicitly: the compiler then
// keeps track of which LDS object an access touches, and waits for an
// in-flight direct-to-LDS copy only when a read can overlap its destination.
template <typename T> using lds_t = __attribute__((address_space(3))) T;
// Wave priority around a group of matrix-core instructions: while a wave
// issues its products it goes ahead of the other waves of its SIMD, which
// meanwhile run their vector work (measured: 3 % faster at S = 8192, equal
// at 1024).
__device__ __forceinline__ void mma_priority_hi() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mma_priority_lo() { __builtin_amdgcn_s_setprio(0); }

template <typename T> __device__ __forceinline__ lds_t<T> *lds_cast(T *p) { return (lds_t<T> *)p; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element traits: the 8-slot fragment type and the 32x32x16 step.
template <typename T> struct Elem;

// 16-bit inputs (bf16 or fp16): one 32x32x16 step per k-block.
template <typename T, typename V> struct Elem16 {
  using frag = V;                       // 8 x 16-bit = 16 bytes
  static constexpr int kFragWords = 4;  // 32-bit words per fragment
  __device__ __forceinline__ static void mma(f32x16 &acc, const frag &a, const frag &b) {
    if constexpr (__is_same(T, bf16))
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
  }
  // Round slots 8*j .. 8*j+7 of a 32x32 result to a fragment (RNE).
  __device__ __forceinline__ static frag pack(const f32x16 &acc, int j) {
    frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = (T)acc[8 * j + s];
    return f;
  }
  // pack() and add the eight fp32 values to `sum` (for weights whose largest
  // value is 1, as with an exact per-tile maximum, normalising the rounded
  // weights by the fp32 sum adds only random error below the rounding of the
  // weights themselves).
  __device__ __forceinline__ static frag pack_sum(const f32x16 &acc, int j, float &sum) {
#pragma unroll
    for (int s = 0; s < 8; ++s) sum += acc[8 * j + s];
    return pack(acc, j);
  }
  // pack(), add the eight fp32 values to `sum` and the eight ROUNDED values
  // to `rsum` (one two-element dot product with ones per pair: exact products,
  // fp32 sums).  Weights shifted by something other than the row maximum can
  // have their largest value anywhere; dividing the product with the rounded
  // weights by their own sum cancels the rounding of a dominant weight
  // (a one-key row gives exactly that key's value), which dividing by the
  // unrounded sum does not.
  __device__ __forceinline__ static frag pack_sums(const f32x16 &acc, int j, float &sum, float &rsum) {
#pragma unroll
    for (int s = 0; s < 8; ++s) sum += acc[8 * j + s];
    const frag f = pack(acc, j);
    const u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int s = 0; s < 4; ++s) rsum = dot2_ones(w[s], rsum);
    return f;
  }
  // x.lo + x.hi + acc for a pair of 16-bit values packed in one word.
  __device__ __forceinline__ static float dot2_ones(uint32_t x, float acc) {
    if constexpr (__is_same(T, bf16)) {
      typedef bf16 v2 __attribute__((ext_vector_type(2)));
      const v2 one = {(bf16)1.f, (bf16)1.f};
      return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, x), one, acc, false);
    } else {
      typedef f16 v2 __attribute__((ext_vector_type(2)));
      const v2 one = {(f16)1.f, (f16)1.f};
      return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, x), one, acc, false);
    }
  }
  // Operands of a rank-1 product mma_rows(acc, rows_a(x, hh), rows_b(hh)) that
  // adds x_c to every element of row c of a 32x32 result, x_c being the value
  // lane c passes (lanes 32-63 pass anything).  x is split into three bf16
  // terms whose fp32 sum reproduces it to fp32 precision, times ones.  bf16
  // has fp32's exponent range, so this step uses bf16 for fp16 inputs too
  // (the two instructions accumulate into the same fp32 result).
  using rows_frag = bf16x8;
  __device__ __forceinline__ static void mma_rows(f32x16 &acc, const rows_frag &a, const rows_frag &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  __device__ __forceinline__ static rows_frag rows_a(float x, int hh) {
    const float y = hh == 0 ? x : 0.f;
    const bf16 t0 = (bf16)y;
    const float r0 = y - (float)t0;
    const bf16 t1 = (bf16)r0;
    const bf16 t2 = (bf16)(r0 - (float)t1);
    rows_frag f = {};
    f[0] = t0;
    f[1] = t1;
    f[2] = t2;
    return f;
  }
  __device__ __forceinline__ static rows_frag rows_b(int hh) {
    const bf16 one = (bf16)(hh == 0 ? 1.f : 0.f);
    rows_frag f = {};
    f[0] = one;
    f[1] = one;
    f[2] = one;
    return f;
  }
};
template <> struct Elem<bf16> : Elem16<bf16, bf16x8> {};
template <> struct Elem<f16> : Elem16<f16, f16x8> {};

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
  __device__ __forceinline__ static frag pack_sum(const f32x16 &acc, int j, float &sum) {
    frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      f[s] = acc[8 * j + s];
      sum += f[s];
    }
    return f;
  }
  // fp32 weights are not rounded: the rounded sum is the sum (callers use `sum`).
  __device__ __forceinline__ static frag pack_sums(const f32x16 &acc, int j, float &sum, float &) {
    return pack_sum(acc, j, sum);
  }
  using rows_frag = frag;
  __device__ __forceinline__ static void mma_rows(f32x16 &acc, const frag &a, const frag &b) { mma(acc, a, b); }
  __device__ __forceinline__ static frag rows_a(float x, int hh) {
    frag f = {};
    f[0] = hh == 0 ? x : 0.f;
    return f;
  }
  __device__ __forceinline__ static frag rows_b(int hh) {
    frag f = {};
    f[0] = hh == 0 ? 1.f : 0.f;
    return f;
  }
};

// Load an 8-slot fragment from LDS (16- or 32-byte aligned).
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag lds_frag(const T *p) {
  return *reinterpret_cast<const typename Elem<T>::frag *>(p);
}
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag lds_frag(const lds_t<T> *p) {
  return *(const lds_t<typename Elem<T>::frag> *)p;
}

// Fragment of the TRANSPOSE of a row-major LDS tile (row stride LD elements),
// in "accum" slot order: lane (h, c) receives
//     slot s = tile[row0 + 8*(s/4) + 4*h + s%4][col0 + c],
// i.e. the A operand of a product that reduces over the tile's rows.
// bf16: two ds_read_b64_tr_b16.  Within each group of 16 lanes that
// instruction hands output lane 4a+b, slot k, element b of the 8 bytes
// addressed by source lane a+4k; so source lane i of group g addresses row
// (row0 + 4*h + i/4) at column (col0 + 16*(g%2) + 4*(i%4)), and the second
// read the rows 8 further down.
// fp32: eight ds_read_b32 (no transposing read exists for 32-bit data).
template <typename T, int LD> struct TrRead;

template <typename T, int LD> struct TrRead16 {
  using frag = typename Elem<T>::frag;
  const lds_t<T> *base;   // this lane's source address for row0 = col0 = 0
  const lds_t<T> *base8;  // ... and for the rows 8 further down
  __device__ __forceinline__ TrRead16(const lds_t<T> *tile, int lane) {
    const int g = lane / 16, i = lane % 16, h = g / 2;
    const int off = (4 * h + i / 4) * LD + 16 * (g % 2) + 4 * (i % 4);
    // The second read's offset is kept opaque to constant folding: folded
    // into an immediate, the compiler loses track of which LDS object the
    // read belongs to and waits for every direct-to-LDS copy in flight.
    int off8 = off + 8 * LD;
    asm volatile("" : "+v"(off8));
    base = tile + off;
    base8 = tile + off8;
  }
  __device__ __forceinline__ TrRead16(const T *tile, int lane) : TrRead16(lds_cast(const_cast<T *>(tile)), lane) {}
  __device__ __forceinline__ frag operator()(int row0, int col0) const {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + row0 * LD + col0));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base8 + row0 * LD + col0));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[4 + k] = b[k];
    }
    return __builtin_bit_cast(frag, v);
  }
};

template <int LD> struct TrRead<bf16, LD> : TrRead16<bf16, LD> {
  using TrRead16<bf16, LD>::TrRead16;
};
template <int LD> struct TrRead<f16, LD> : TrRead16<f16, LD> {
  using TrRead16<f16, LD>::TrRead16;
};

template <int LD> struct TrRead<float, LD> {
  using frag = f32x8;
  const lds_t<float> *base;
  __device__ __forceinline__ TrRead(const lds_t<float> *tile, int lane) {
    base = tile + 4 * (lane / 32) * LD + lane % 32;
  }
  __device__ __forceinline__ TrRead(const float *tile, int lane) : TrRead(lds_cast(const_cast<float *>(tile)), lane) {}
  __device__ __forceinline__ frag operator()(int row0, int col0) const {
    const lds_t<float> *p = base + row0 * LD + col0;
    frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = p[(8 * (s / 4) + s % 4) * LD];
    return f;
  }
};

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
  __device__ __forceinline__ void store8(const u32x2 &v, uint32_t off) const {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
  }
};

// Output element type OT: fp32, or the 16-bit input type (rounded to nearest
// even once, at the store).  store_out4 writes four consecutive outputs at
// element offset e; load_out8 reads eight as fp32.
template <typename OT> struct Vec4Of;
template <> struct Vec4Of<bf16> { using type = bf16x4; };
template <> struct Vec4Of<f16> { using type = f16x4; };
template <typename OT> struct Vec8Of;
template <> struct Vec8Of<bf16> { using type = bf16x8; };
template <> struct Vec8Of<f16> { using type = f16x8; };

template <typename OT>
__device__ __forceinline__ void load_out8(const GBuf &g, uint32_t e, float (&x)[8]) {
  if constexpr (sizeof(OT) == 4) {
    const f32x4 a = __builtin_bit_cast(f32x4, g.load16(e * 4u));
    const f32x4 b = __builtin_bit_cast(f32x4, g.load16(e * 4u + 16u));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  } else {
    const typename Vec8Of<OT>::type h = __builtin_bit_cast(typename Vec8Of<OT>::type, g.load16(e * 2u));
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
  }
}

template <typename OT>
__device__ __forceinline__ void store_out4(const GBuf &g, const f32x4 &v, uint32_t e) {
  if constexpr (sizeof(OT) == 4) {
    g.store16(v, e * 4u);
  } else {
    typename Vec4Of<OT>::type h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (OT)v[i];
    g.store8(__builtin_bit_cast(u32x2, h), e * 2u);
  }
}

// Store of one 32 x 32 output block that a wave holds in accumulator layout
// (lane (c, hh) holds row c, columns 8g + 4hh .. 8g + 4hh + 3 in registers
// 4g .. 4g + 3; e.g. O = (O^T)^T with a lane per query), through 4 KB of the
// wave's own LDS, so that every store instruction writes whole rows of the
// block: written straight from the accumulator, each instruction covers 32
// rows with 32 bytes apiece (32 partial cache lines), rearranged it covers 8
// rows with 128 bytes apiece (fp32) or 16 rows with 64 (16-bit outputs), four
// to eight times fewer memory requests for the same bytes.
//   v        the block, already scaled as stored
//   scratch  256 f32x4 of LDS that no other wave touches meanwhile
//   g        output buffer; rows past its range are dropped
//   row0     row of the block's row 0; ss the row stride in elements
//   col0     element column of the block's column 0
// Chunk x (16 bytes) of scratch row r sits at x ^ ((r >> 1) & 7): the 16
// lanes of each write (16 rows, one chunk) and each read (2 rows, 8 chunks)
// then fall on distinct banks.  LDS accesses of one wave complete in order,
// so the reads see the writes; the empty asm keeps the compiler from
// reordering them.
template <typename OT>
__device__ __forceinline__ void store_block_rows(const f32x16 &v, lds_t<f32x4> *scratch, const GBuf &g, int row0,
                                                 int ss, int col0, int lane) {
  // the lane index is re-derived here so that none of this address arithmetic
  // is shared with (and kept live through) the caller's main loop
  asm volatile("" : "+v"(lane));
  const int c = lane % 32, hh = lane / 32;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    f32x4 x4;
#pragma unroll
    for (int i = 0; i < 4; ++i) x4[i] = v[4 * gq + i];
    scratch[c * 8 + ((2 * gq + hh) ^ ((c >> 1) & 7))] = x4;
  }
  asm volatile("" ::: "memory");
  if constexpr (sizeof(OT) == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + lane / 8, x = lane % 8;
      const f32x4 x4 = scratch[r * 8 + (x ^ ((r >> 1) & 7))];
      g.store16(x4, (uint32_t)((row0 + r) * ss + col0 + 4 * x) * 4u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 16 * k + lane / 4, x = 2 * (lane % 4);
      const f32x4 a = scratch[r * 8 + (x ^ ((r >> 1) & 7))];
      const f32x4 b = scratch[r * 8 + ((x + 1) ^ ((r >> 1) & 7))];
      typename Vec8Of<OT>::type h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = (OT)a[i];
        h[4 + i] = (OT)b[i];
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, h), g.r,
                                             (uint32_t)((row0 + r) * ss + col0 + 4 * x) * 2u, 0, 0);
    }
  }
  asm volatile("" ::: "memory");
}

// An 8-slot fragment of row `row`, columns [col, col + 8), of rows `ss`
// elements apart behind `g` (zeros past the resource's end).
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag global_frag_rs(const GBuf &g, int row, int col, int ss) {
  using frag = typename Elem<T>::frag;
  const uint32_t off = (uint32_t)(row * ss + col) * sizeof(T);
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

// The same for a row-major [*, D] array (rows D elements apart).
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
// LDS row strides.  Tiles read as row fragments (16 bytes per lane, lanes on
// consecutive rows) are padded by 16 bytes per row, which spreads consecutive
// rows over distinct LDS banks; tiles read only through the transposing load
// stay unpadded, the stride it reads fastest at.
template <typename T, int D> struct RowStride {
  static constexpr int kPadded = D + 16 / sizeof(T);
  static constexpr int kTrOnly = sizeof(T) == 2 ? D : D + 4;
};

// Cooperative copy of rows [r0, r0 + R) of a row-major [*, D] array into a
// row-major LDS tile with row stride LD; rows past the buffer resource's end
// read as zeros.  Thread `tid` moves 16-byte chunks idx = tid + NT * pass
// (row idx / CPR, chunk idx % CPR), so each wave's load instruction covers
// whole consecutive rows and global reads are fully coalesced.  Split into a
// global->register phase and a register->LDS phase so the next tile can be
// fetched while the current one is in use.
template <typename T, int R, int D, int NT> struct TileLoader {
  static constexpr int kVec = 16 / sizeof(T);          // elements per chunk
  static constexpr int kCPR = D / kVec;                // chunks per row
  static constexpr int kChunks = R * kCPR;
  static constexpr int kPasses = (kChunks + NT - 1) / NT;
  static constexpr bool kFull = kChunks % NT == 0;     // every thread busy in every pass
  static_assert(D % kVec == 0, "D must be a multiple of the chunk");
  static_assert(kFull || (kChunks < NT && kChunks % kWaveSize == 0),
                "a partial pass must end on a wave boundary");

  u32x4 regs[kPasses];

  // Threads past the tile in a partial pass sit out; the test is per wave.
  __device__ __forceinline__ static bool busy(int tid) {
    return kFull || __builtin_amdgcn_readfirstlane(tid / kWaveSize) * kWaveSize < kChunks;
  }

  __device__ __forceinline__ void load(const GBuf &g, int r0, int tid) {
    if (!busy(tid)) return;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int idx = tid + NT * ps;
      regs[ps] = g.load16((uint32_t)((r0 + idx / kCPR) * D + (idx % kCPR) * kVec) * sizeof(T));
    }
  }

  template <int LD>
  __device__ __forceinline__ void store(T *dst, int tid) const {
    if (!busy(tid)) return;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int idx = tid + NT * ps;
      *reinterpret_cast<u32x4 *>(dst + (idx / kCPR) * LD + (idx % kCPR) * kVec) = regs[ps];
    }
  }
};

// ---------------------------------------------------------------------------
// Direct global->LDS tile copies (buffer_load ... lds).  Each wave instruction
// writes 64 lanes x 16 bytes to 1 KB of consecutive LDS; the global chunk each
// lane fetches is free, which places rows without padding.  Rows past the
// buffer resource's end arrive as zeros.  No VGPRs hold the data in flight,
// so tiles can be requested several iterations before they are used; the
// caller waits with wait_vmcnt (each wave counts its own copies) and then
// crosses a workgroup barrier before reading.
//
// Tiles read as row fragments are XOR-swizzled: 16-byte chunk c of row r is
// stored at chunk c ^ (r & SW), which puts the 16-byte reads of consecutive
// rows on distinct LDS banks without padding.
// XOR mask applied to the 16-byte chunk index of row `row` of a swizzled
// tile (chunk x of the row is stored at x ^ mask).  Chosen by measurement so
// that both ways the tiles are read run near the LDS peak: 16-byte row
// fragments (16 consecutive rows at a time, one chunk each) and the
// transposing 8-byte reads (rows 0-3 x chunks 0-3 of a 32-column block, then
// rows 4-7).  For 128-byte rows a mask of row & 7 puts rows r and r + 8 on
// the same banks and halves the row-fragment rate; these masks have period 16.
template <typename T, int D> __device__ __forceinline__ uint32_t swz_mask(uint32_t row) {
  if constexpr (sizeof(T) == 4) {
    return row & 7;
  } else if constexpr (D == 32) {
    return row & 3;
  } else if constexpr (D == 64) {
    return (4 * ((row >> 1) & 1) + ((row >> 2) & 1)) ^ (2 * ((row >> 3) & 1));
  } else {
    return 4 * (row & 3) + ((row >> 2) & 3);
  }
}

template <typename T, int R, int D, int NT, bool SWIZZLE> struct DmaTile {
  static constexpr int kVec = 16 / sizeof(T);                 // elements per chunk
  static constexpr int kCPR = D / kVec;                        // chunks per row
  static constexpr int kBlocks = R * kCPR / kWaveSize;         // 1 KB blocks per tile
  static constexpr int kPerWave = kBlocks / (NT / kWaveSize);  // copy instructions per wave
  static_assert(R * kCPR % NT == 0, "tile must split evenly over the waves");

  __device__ __forceinline__ static void issue(const GBuf &g, lds_t<T> *tile, int r0, int wave, int lane) {
    typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;
      const int p = blk * kWaveSize + lane;
      const uint32_t row = (uint32_t)p / kCPR;
      const uint32_t chunk = (uint32_t)(p % kCPR) ^ (SWIZZLE ? swz_mask<T, D>(row) : 0u);
      const uint32_t col = chunk * kVec;  // swizzled chunk, in elements
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          g.r, (lds_void *)(tile + blk * (1024 / sizeof(T))), 16,
          (((uint32_t)r0 + row) * D + col) * (uint32_t)sizeof(T), 0, 0, 0);
    }
  }

  // The same copy from rows `ss` elements apart (a strided view of the rows),
  // in two parts: lane_offsets() gives each lane's byte offset inside a tile
  // (row times ss, plus the swizzled column), once per kernel; issue_at()
  // adds the tile's first-row offset, which is uniform and kept in a scalar
  // register (row0_bytes() makes it one), so each copy costs one vector add.
  // The whole offset still goes through the range-checked vector offset.
  __device__ __forceinline__ static void lane_offsets(uint32_t (&off)[kPerWave], int wave, int lane, uint32_t ss) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;
      const int p = blk * kWaveSize + lane;
      const uint32_t row = (uint32_t)p / kCPR;
      const uint32_t chunk = (uint32_t)(p % kCPR) ^ (SWIZZLE ? swz_mask<T, D>(row) : 0u);
      off[i] = (row * ss + chunk * kVec) * (uint32_t)sizeof(T);
    }
  }
  __device__ __forceinline__ static uint32_t row0_bytes(int r0, uint32_t ss) {
    return __builtin_amdgcn_readfirstlane((uint32_t)r0 * ss * (uint32_t)sizeof(T));
  }
  __device__ __forceinline__ static void issue_at(const GBuf &g, lds_t<T> *tile, uint32_t r0_bytes,
                                                  const uint32_t (&off)[kPerWave], int wave) {
    typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g.r, (lds_void *)(tile + blk * (1024 / sizeof(T))), 16,
                                               off[i] + r0_bytes, 0, 0, 0);
    }
  }
};

// One direct-to-LDS copy of 64 consecutive floats (elements e0 .. e0+63 of
// the buffer; past its end they arrive as zeros), issued by one wave.
__device__ __forceinline__ void dma_vec64(const GBuf &g, lds_t<float> *dst, int e0, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(g.r, (lds_void *)dst, 4, (uint32_t)(e0 + lane) * 4u, 0, 0, 0);
}

// Fragment of the TRANSPOSE of a swizzled tile written by DmaTile<T, R, D, NT,
// true> (row-major, D columns, chunks permuted by swz_mask), in the same slot
// order as TrRead: operator()(tile, row0, db) gives rows row0 .. row0+15
// (row0 a multiple of 16) of columns 32*db .. 32*db+31.  The object holds
// only this lane's element offsets, so one serves every tile of that shape.
template <typename T, int D> struct TrSwz;

template <typename T, int D> struct TrSwz16 {
  using frag = typename Elem<T>::frag;
  static constexpr int DB = D / 32;
  // [read][db]: the first read covers rows 0-7 of the 16, the second rows
  // 8-15.  Byte offsets, so an address is one add (often folded away).
  uint32_t off[2][DB];
  __device__ __forceinline__ explicit TrSwz16(int lane) {
    const int g = lane / 16, i = lane % 16;
    const int rl = 4 * (g / 2) + i / 4;             // row within an 8-row group
    const int x = 2 * (g % 2) + (i % 4) / 2;        // 16-byte chunk within the 32-column block
    const int e = 4 * (i % 2);                      // element within the chunk
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int r = rl + 8 * k;
        off[k][db] = (uint32_t)(r * D + 8 * (int)((uint32_t)(4 * db + x) ^ swz_mask<T, D>(r)) + e) * sizeof(T);
      }
  }
  // A copy whose offsets the compiler cannot trace back to the loop-invariant
  // originals: taken once per tile, it keeps the sum with each tile's LDS
  // address inside the loop, where the constant part folds into the
  // instruction's offset field instead of occupying a register per tile.
  __device__ __forceinline__ TrSwz16 pinned() const {
    TrSwz16 t = *this;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(t.off[k][db]));
    return t;
  }
  __device__ __forceinline__ frag operator()(const lds_t<T> *tile, int row0, int db) const {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const lds_t<char> *p = (const lds_t<char> *)(tile + row0 * D);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + off[0][db]));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + off[1][db]));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
    return __builtin_bit_cast(frag, v);
  }
};

template <int D> struct TrSwz<bf16, D> : TrSwz16<bf16, D> {
  using TrSwz16<bf16, D>::TrSwz16;
  __device__ __forceinline__ TrSwz(const TrSwz16<bf16, D> &t) : TrSwz16<bf16, D>(t) {}
  __device__ __forceinline__ TrSwz pinned() const { return TrSwz(TrSwz16<bf16, D>::pinned()); }
};
template <int D> struct TrSwz<f16, D> : TrSwz16<f16, D> {
  using TrSwz16<f16, D>::TrSwz16;
  __device__ __forceinline__ TrSwz(const TrSwz16<f16, D> &t) : TrSwz16<f16, D>(t) {}
  __device__ __forceinline__ TrSwz pinned() const { return TrSwz(TrSwz16<f16, D>::pinned()); }
};

template <int D> struct TrSwz<float, D> {
  using frag = f32x8;
  // 4-float chunks, mask row & 7; rows 4h + u (u < 4) of an 8-row group,
  // column c: chunk (8*db + c/4) ^ (4h + u) = 8*db + ((c/4) ^ (4h + u)).
  uint32_t off[4];  // byte offsets
  __device__ __forceinline__ explicit TrSwz(int lane) {
    const int h = lane / 32, c = lane % 32;
#pragma unroll
    for (int u = 0; u < 4; ++u) off[u] = (uint32_t)((4 * h + u) * D + 4 * ((c / 4) ^ (4 * h + u)) + c % 4) * 4u;
  }
  __device__ __forceinline__ TrSwz pinned() const {
    TrSwz t = *this;
#pragma unroll
    for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(t.off[u]));
    return t;
  }
  __device__ __forceinline__ frag operator()(const lds_t<float> *tile, int row0, int db) const {
    frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      f[s] = *(const lds_t<float> *)((const lds_t<char> *)(tile + row0 * D + 32 * db + 8 * D * (s / 4)) + off[s % 4]);
    return f;
  }
};

// Row fragments of a swizzled tile for lanes that own row 32*blk + c (c the
// lane's column index): operator()(tile, blk, kb) gives the 8 slots of that
// row at columns 16*kb + 8*hh .. +7 (natural slot order).  Holds this lane's
// element offsets (the swizzle mask depends on the row modulo 16 only).
template <typename T, int D> struct RowFrag {
  using frag = typename Elem<T>::frag;
  static constexpr int KB = D / 16;
  static constexpr int kVec = 16 / sizeof(T);  // elements per 16-byte chunk
  static constexpr int kReads = sizeof(T) == 2 ? 1 : 2;
  uint32_t off[KB][kReads];  // byte offsets
  __device__ __forceinline__ explicit RowFrag(int lane) {
    const int c = lane % 32, hh = lane / 32;
    const uint32_t m = swz_mask<T, D>((uint32_t)c);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < kReads; ++i) {
        const uint32_t chunk = (uint32_t)((16 * kb + 8 * hh) / kVec + i);
        off[kb][i] = (uint32_t)(c * D + (int)((chunk ^ m) * kVec)) * sizeof(T);
      }
  }
  // See TrSwz::pinned.
  __device__ __forceinline__ RowFrag pinned() const {
    RowFrag t = *this;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < kReads; ++i) asm volatile("" : "+v"(t.off[kb][i]));
    return t;
  }
  __device__ __forceinline__ frag operator()(const lds_t<T> *tile, int blk, int kb) const {
    const lds_t<char> *p = (const lds_t<char> *)(tile + blk * 32 * D);
    if constexpr (sizeof(T) == 2) {
      return *(const lds_t<frag> *)(p + off[kb][0]);
    } else {
      const f32x4 a = *(const lds_t<f32x4> *)(p + off[kb][0]);
      const f32x4 b = *(const lds_t<f32x4> *)(p + off[kb][1]);
      frag f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = a[i];
        f[4 + i] = b[i];
      }
      return f;
    }
  }
};

// Wait until at most N of this wave's vector-memory operations (including
// direct-to-LDS copies) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The same, and also until every LDS access of this wave has completed (its
// LDS writes are then visible to the workgroup after the next barrier).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every copy in flight); LDS visibility of the copies a wave waited
// for is what the barrier publishes.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// Grouped-query attention: H query heads share H / G key/value heads, query
// head h reading K/V head h / G of its batch entry.  Global head indices run
// b * H + h (queries) and b * (H / G) + h / G (keys and values).
__device__ __forceinline__ int kv_head_of(int qhead, int H, int G) { return (qhead / H) * (H / G) + (qhead % H) / G; }

// RoPE gradient: turn two interleaved pairs (a[0], a[1]) and (a[2], a[3])
// back by their angles, cs = (cos, sin) of the first pair, then of the
// second: (x0, x1) -> (x0 c + x1 s, x1 c - x0 s), the transpose of the
// forward rotation (x0 c - x1 s, x0 s + x1 c).
__device__ __forceinline__ void rope_back(f32x4 &a, const f32x4 cs) {
  const float x0 = a[0], x1 = a[1], x2 = a[2], x3 = a[3];
  a[0] = x0 * cs[0] + x1 * cs[1];
  a[1] = x1 * cs[0] - x0 * cs[1];
  a[2] = x2 * cs[2] + x3 * cs[3];
  a[3] = x3 * cs[2] - x2 * cs[3];
}

// Offset of the (b, h) panel of a tensor with layout L (Layout: attn_launch.h).
__device__ __forceinline__ size_t panel_off(const Layout &L, int b, int h) {
  return (size_t)((int64_t)b * L.sb + (int64_t)h * L.sh);
}
// Bytes from a panel's first element to the end of row `rows - 1`.
__device__ __forceinline__ uint32_t panel_bytes(const Layout &L, int rows, int D, int esize) {
  return (uint32_t)(((rows - 1) * L.ss + D) * esize);
}

// Tile schedule.  Workgroups are dealt to the 8 XCDs round-robin (block b
// runs on XCD b % 8) and, within an XCD, to its 32 CUs round-robin (local
// index l = b / 8 on CU l % 32), as measured on MI355X; when every workgroup
// is resident at once, a CU therefore runs local indices l, l+32, l+64, ...
// together.  A launch covers `nunits` independent units (heads, or document x
// head pairs) of `nranks` tiles each, and a tile's rank orders it by work
// (rank 0 the most).  Each XCD gets a contiguous range of units (so re-reads
// of a unit's K/V or Q/dO stay in that XCD's L2); its tiles are sorted by
// rank and dealt in snake order over rounds of 32 (round r, position p ->
// sorted slot 32r + p, or 32r + 31 - p on odd rounds), so each CU gets a heavy
// and a light tile per pair of rounds, and if the launch does not fit at once
// the heaviest tiles still start first.
struct TileSlot {
  int unit;
  int rank;
};
__device__ __forceinline__ TileSlot snake_slot(int bid, int nblocks, int nranks) {
  const int per_xcd = nblocks >> 3;
  if ((nblocks & 7) == 0 && per_xcd % nranks == 0) {
    const int units_x = per_xcd / nranks;  // units on this XCD
    const int l = bid >> 3;
    const int round0 = l & ~31;
    const int m = min(32, per_xcd - round0);  // size of this (possibly partial) round
    const int pos = l & 31;
    const int s = round0 + (((l >> 5) & 1) ? m - 1 - pos : pos);
    return {(bid & 7) * units_x + s % units_x, s / units_x};
  }
  return {bid / nranks, bid % nranks};
}

// Causal mode: 1-D grid of ntiles * B * H blocks; unit = head.  heavy_first:
// tile work grows with the tile index (query tiles: t + 1 key tiles); else it
// shrinks (key tiles of the dK/dV kernel: ntiles - t query tiles).
__device__ __forceinline__ RowTile causal_tile(int bid, int nblocks, int ntiles, int BM, int S,
                                               bool heavy_first) {
  const TileSlot sl = snake_slot(bid, nblocks, ntiles);
  const int ti = heavy_first ? ntiles - 1 - sl.rank : sl.rank;
  RowTile t;
  t.head = sl.unit;
  t.r_start = ti * BM;
  t.r_end = min(t.r_start + BM, S);
  t.seg_start = 0;
  t.seg_end = S;
  t.valid = true;
  return t;
}

// Packed documents.  The tiles of one head are ranked by work across all of
// its documents: a document of L rows has n = ceil(L / BM) tiles (at most
// ntiles, the tile count of max_seqlen), and its tiles have the classes 1..n,
// class c doing about c tiles' worth of work: query tile c - 1 (work grows
// with the tile index: keys from the document start to the diagonal) or key
// tile n - c (work shrinks with it: query rows from the tile to the
// document end).  Rank k is the k-th tile in the order (class descending,
// then document index), so the snake deal above pairs the heaviest tiles of
// the longest documents with the lightest tiles, whatever the mix of lengths.
// A head has at most doc_rank_slots() tiles; the grid holds that many blocks
// per unit, and ranks past the head's actual tile count exit at once.  The
// ranking is recomputed by every wave from cu_seqlens (lane j holds documents
// j, j + 64, ...), which bounds it to kDocRankMax documents and tiles per
// document; larger launches keep the per-document grid.
constexpr int kDocRankMax = 4 * kWaveSize;
__host__ __device__ __forceinline__ bool doc_ranked(int n_seqs, int ntiles) {
  return n_seqs <= kDocRankMax && ntiles <= kDocRankMax;
}
// Upper bound on one head's tiles: n_seqs * ntiles, and, since the documents
// cover the S rows, sum ceil(L_d / BM) <= (S + n_seqs * (BM - 1)) / BM.
__host__ __device__ __forceinline__ int doc_rank_slots(int n_seqs, int ntiles, int S, int BM) {
  const int64_t a = (int64_t)n_seqs * ntiles;
  const int64_t b = ((int64_t)S + (int64_t)n_seqs * (BM - 1)) / BM;
  return (int)(a < b ? a : b);
}
// Blocks per unit in packed mode; `rank` is the kernel's choice of the
// ranked schedule (and it applies where doc_ranked allows it).
__host__ __device__ __forceinline__ int doc_blocks_per_unit(int n_seqs, int ntiles, int S, int BM, bool rank) {
  return rank && doc_ranked(n_seqs, ntiles) ? doc_rank_slots(n_seqs, ntiles, S, BM) : n_seqs * ntiles;
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int o = 1; o < kWaveSize; o <<= 1) x += __shfl_xor(x, o, kWaveSize);
  return x;
}

// Rank k of one head -> document * 2^32 + class, or -1 when the head has k
// tiles or fewer.  Wave-uniform inputs and result: the classes are scanned
// from the top, each taking as many ranks as there are documents with that
// many tiles or more (ballot counts; at most kDocRankMax classes).
__device__ __forceinline__ int64_t doc_rank_item(const int32_t *__restrict__ cu, int n_seqs, int ntiles, int BM,
                                                 int k) {
  constexpr int J = kDocRankMax / kWaveSize;
  const int lane = threadIdx.x % kWaveSize;
  int nd[J];  // tiles of documents lane + 64 j
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int d = lane + kWaveSize * j;
    nd[j] = d < n_seqs ? min((cu[d + 1] - cu[d] + BM - 1) / BM, ntiles) : 0;
  }
  for (int c = ntiles; c >= 1; --c) {
    uint64_t m[J];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      m[j] = __ballot(nd[j] >= c);
      cnt += __popcll(m[j]);
    }
    if (k < cnt) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int cj = __popcll(m[j]);
        if (k < cj) {
          uint64_t x = m[j];
          for (int r = 0; r < k; ++r) x &= x - 1;
          return (int64_t)(kWaveSize * j + __builtin_ctzll(x)) << 32 | c;
        }
        k -= cj;
      }
    }
    k -= cnt;
  }
  return -1;
}

// Packed-document mode.  Ranked (doc_ranked): 1-D grid of units *
// doc_rank_slots() blocks; unit = head.  Otherwise: units * n_seqs * ntiles
// blocks, unit = head * n_seqs + document, tiles past a document's end exit
// at once.  heavy_first as for causal_tile.
__device__ __forceinline__ RowTile doc_tile(const int32_t *__restrict__ cu, int bid, int nblocks, int ntiles,
                                            int n_seqs, int BM, int S, bool heavy_first, bool rank) {
  RowTile t;
  if (rank && doc_ranked(n_seqs, ntiles)) {
    const TileSlot sl = snake_slot(bid, nblocks, doc_rank_slots(n_seqs, ntiles, S, BM));
    const int64_t item = doc_rank_item(cu, n_seqs, ntiles, BM, sl.rank);
    t.valid = item >= 0;
    if (!t.valid) return t;
    const int doc = __builtin_amdgcn_readfirstlane((int)(item >> 32));
    const int cls = __builtin_amdgcn_readfirstlane((int)item);
    const int ds = cu[doc];
    const int de = cu[doc + 1];
    const int ti = heavy_first ? cls - 1 : min((de - ds + BM - 1) / BM, ntiles) - cls;
    t.head = sl.unit;
    t.r_start = ds + ti * BM;
    t.r_end = min(t.r_start + BM, de);
    t.seg_start = ds;
    t.seg_end = de;
    return t;
  }
  const TileSlot sl = snake_slot(bid, nblocks, ntiles);
  const int doc = sl.unit % n_seqs;
  const int ds = cu[doc];
  const int de = cu[doc + 1];
  const int ti = heavy_first ? ntiles - 1 - sl.rank : sl.rank;
  t.head = sl.unit / n_seqs;
  t.r_start = ds + ti * BM;
  t.r_end = min(t.r_start + BM, de);
  t.seg_start = ds;
  t.seg_end = de;
  t.valid = t.r_start < de;
  return t;
}

}  // namespace attn
