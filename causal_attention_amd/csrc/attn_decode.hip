// attn_decode.hip - one decode step against a key/value cache.
//
// Each (batch entry b, query head h) has one new query, the newest token,
// whose own key is already in the cache; it attends keys 0 .. len_b - 1 of its
// K/V head (causality admits every cached key).  This is the generation step
// that Forge plans next (Forge, "Roadmap").  The work is reading the
// cache: 2 * len * D elements per K/V head against ~4 * len * D * G flops for
// the G query heads of that K/V head, so the kernel is bound by HBM bandwidth.
//
// gfx950 mapping.
//  * Split over the keys: one wave per (b, K/V head, chunk of keys) computes,
//    for all G <= 32 query heads of the group at once, the chunk's softmax
//    (online, exact maximum per 32-key tile) and its normalised partial output
//    O_c and log-normaliser LSE_c.  Scores are S^T = K Q^T on the matrix cores
//    with the G queries as the 32 columns (zero columns past G), so each K row
//    read from HBM serves every query head of its group.
//  * K row fragments are read straight from global memory into registers (one
//    tile ahead); V tiles come by direct global->LDS copy into two ring slots
//    and are read through the transposing LDS load for O^T += V^T P^T.
//  * A second kernel merges the chunks of each (b, h) exactly:
//    M = max_c LSE_c, O = sum_c e^(LSE_c - M) O_c / sum_c e^(LSE_c - M),
//    LSE = M + ln sum_c e^(LSE_c - M).  With one chunk the first kernel writes
//    the result directly.
#include <mutex>

#include "attn_api.h"
#include "attn_device.h"
#include "attn_launch.h"

// Chunk partials of attn_decode_noalloc: a static buffer on every GPU the
// library runs on (callers that cannot allocate).  In host code `scratch`
// names a host-side stand-in; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_SCRATCH_BYTES];

namespace attn {

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_decode_kernel(const T *__restrict__ q, const T *__restrict__ kc,
                                                         const T *__restrict__ vc,
                                                         const int32_t *__restrict__ lens,
                                                         float *__restrict__ o_part, float *__restrict__ lse_part,
                                                         float *__restrict__ o, float *__restrict__ lse, int B,
                                                         int H, int Hkv, int S_max, int nsplit, int chunk,
                                                         float c2) {
  constexpr int BN = 32;  // keys per tile
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int PB = BN / 16;
  using E = Elem<T>;
  using frag = typename E::frag;
  using VTile = DmaTile<T, BN, D, kWaveSize, false>;

  __shared__ __attribute__((aligned(1024))) T sV0[BN * D];
  __shared__ __attribute__((aligned(1024))) T sV1[BN * D];

  const int split = blockIdx.x % nsplit;
  const int kvh = blockIdx.x / nsplit;  // b * Hkv + K/V head
  const int b = kvh / Hkv;
  const int G = H / Hkv;
  const int len = lens[b];
  const int lo = split * chunk;
  if (lo >= len) return;  // the merge reads only the chunks that hold keys
  const int hi = min(lo + chunk, len);
  const int ntile = (hi - lo + BN - 1) / BN;

  const int lane = threadIdx.x;
  const int hh = lane / 32;
  const int c = lane % 32;  // query head g of the group (valid for c < G)
  const int qh0 = b * H + (kvh % Hkv) * G;  // first query head of the group
  const GBuf gq(q + (size_t)qh0 * D, (uint32_t)(G * D * sizeof(T)));  // rows past G read 0
  const size_t kvbase = (size_t)kvh * S_max * D;
  const GBuf gk(kc + kvbase, (uint32_t)(hi * D * sizeof(T)));
  const GBuf gv(vc + kvbase, (uint32_t)(hi * D * sizeof(T)));

  auto vslot = [&]<int P>() { return lds_cast(P == 0 ? sV0 : sV1); };
  auto kfrags = [&](frag (&kf)[KB], int k0) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kf[kb] = global_frag<T, D>(gk, k0 + c, 16 * kb + 8 * hh);
  };

  frag qf[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) qf[kb] = global_frag<T, D>(gq, c, 16 * kb + 8 * hh);

  frag kcur[KB];
  kfrags(kcur, lo);
  VTile::issue(gv, vslot.template operator()<0>(), lo, 0, lane);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;  // running maximum (scaled, base 2)
  float l = 0.f;        // this lane-half's running sum

  auto step = [&]<int P>(int t) {
    wait_vmcnt<0>();  // this tile's K fragments and V copy
    const int k0 = lo + t * BN;
    frag knext[KB];
    if (t + 1 < ntile) {
      VTile::issue(gv, vslot.template operator()<1 - P>(), k0 + BN, 0, lane);
      kfrags(knext, k0 + BN);
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) E::mma(s, kcur[kb], qf[kb]);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r / 4) + 4 * hh + (r % 4);
      s[r] = key < hi ? s[r] * c2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, swap_halves(mx));
    const float mnew = fmaxf(m, mx);  // finite: every tile holds at least one key below hi
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r] - mnew);
    frag pf[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) pf[j] = E::pack_sum(s, j, l);
    const TrRead<T, D> vr(vslot.template operator()<P>(), lane);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < PB; ++j) E::mma(oacc[db], vr(16 * j, 32 * db), pf[j]);
    if (t + 1 < ntile) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kcur[kb] = knext[kb];
    }
  };
  for (int t = 0; t < ntile; t += 2) {
    step.template operator()<0>(t);
    if (t + 1 < ntile) step.template operator()<1>(t + 1);
  }

  const float lt = l + swap_halves(l);
  const float inv = 1.0f / lt;
  const float lse_c = (m + __log2f(lt)) * kLn2;
  if (c >= G) return;
  const int h = qh0 + c;  // global query head b * H + g
  float *dst = nsplit == 1 ? o + (size_t)h * D : o_part + ((size_t)split * B * H + h) * D;
  const GBuf go(dst, (uint32_t)(D * sizeof(float)));
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4 val;
#pragma unroll
      for (int i = 0; i < 4; ++i) val[i] = oacc[db][4 * g4 + i] * inv;
      go.store16(val, (uint32_t)(db * 32 + 8 * g4 + 4 * hh) * sizeof(float));
    }
  if (hh == 0) {
    if (nsplit == 1) {
      if (lse != nullptr) lse[h] = lse_c;
    } else {
      lse_part[(size_t)split * B * H + h] = lse_c;
    }
  }
}

// Exact merge of the chunks of one (b, h): one workgroup per query head,
// thread d handles output column d.
template <int D>
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(const float *__restrict__ o_part,
                                                              const float *__restrict__ lse_part,
                                                              const int32_t *__restrict__ lens,
                                                              float *__restrict__ o, float *__restrict__ lse,
                                                              int B, int H, int nsplit, int chunk) {
  const int h = blockIdx.x;  // b * H + head
  const int b = h / H;
  const int d = threadIdx.x;
  const int n = min(nsplit, (lens[b] + chunk - 1) / chunk);  // chunks that hold keys
  float mx = -INFINITY;
  for (int s = 0; s < n; ++s) mx = fmaxf(mx, lse_part[(size_t)s * B * H + h]);
  float wsum = 0.f, acc = 0.f;
  for (int s = 0; s < n; ++s) {
    const float w = __expf(lse_part[(size_t)s * B * H + h] - mx);
    wsum += w;
    acc += w * o_part[((size_t)s * B * H + h) * D + d];
  }
  o[(size_t)h * D + d] = acc / wsum;
  if (d == 0 && lse != nullptr) lse[h] = mx + __logf(wsum);
}

// Waves per CU the key split aims for across the launch.  Measured on
// B8 H16 D128 with 8192-token caches: 4 -> 102 us, 8 -> 106, 16 -> 119,
// 32 -> 136 (each extra chunk repeats a wave's set-up and first-tile wait).
constexpr int kDecodeWavesPerCU = 4;

// Key chunk per wave: enough chunks for about kDecodeWavesPerCU waves per CU
// across the launch, at least one 32-key tile each.
void decode_split(int B, int H_kv, int max_len, int *nsplit, int *chunk) {
  const int tiles = (max_len + 31) / 32;
  int want = (kDecodeWavesPerCU * 256 + B * H_kv - 1) / (B * H_kv);
  want = max(1, min(want, tiles));
  const int tiles_per = (tiles + want - 1) / want;
  *chunk = tiles_per * 32;
  *nsplit = (max_len + *chunk - 1) / *chunk;
}

template <typename T, int D>
static hipError_t launch_decode_t(const DecodeArgs &a) {
  int nsplit, chunk;
  decode_split(a.B, a.H_kv, a.max_len, &nsplit, &chunk);
  const float c2 = a.scale * kLog2e;
  const int waves = nsplit * a.B * a.H_kv;
  hipLaunchKernelGGL((attn_decode_kernel<T, D>), dim3(waves), dim3(64), 0, a.stream, static_cast<const T *>(a.q),
                     static_cast<const T *>(a.k_cache), static_cast<const T *>(a.v_cache), a.cache_lens, a.o_part,
                     a.lse_part, a.o, a.lse, a.B, a.H, a.H_kv, a.S_max, nsplit, chunk, c2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  hipLaunchKernelGGL((attn_decode_merge_kernel<D>), dim3(a.B * a.H), dim3(D), 0, a.stream, a.o_part, a.lse_part,
                     a.cache_lens, a.o, a.lse, a.B, a.H, nsplit, chunk);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_dt(const DecodeArgs &a) {
  switch (a.D) {
    case 32: return launch_decode_t<T, 32>(a);
    case 64: return launch_decode_t<T, 64>(a);
    default: return launch_decode_t<T, 128>(a);
  }
}

hipError_t launch_decode(const DecodeArgs &a) {
  switch (a.dtype) {
    case 1: return launch_decode_dt<bf16>(a);
    case 2: return launch_decode_dt<f16>(a);
    default: return launch_decode_dt<float>(a);
  }
}

size_t decode_scratch_bytes() { return sizeof(scratch); }

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Device address of this device's `scratch` (the current device), looked up
// on the first call on that device with the device current.
hipError_t scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_decode_noalloc(DecodeArgs a) {
  const size_t need = decode_workspace_bytes(a.B, a.H, a.H_kv, a.D, a.max_len);
  if (need > sizeof(scratch)) return hipErrorInvalidValue;  // the caller checks first
  a.o_part = nullptr;
  a.lse_part = nullptr;
  if (need > 0) {
    void *base = nullptr;
    const hipError_t e = scratch_for_current_device(&base);
    if (e != hipSuccess) return e;
    // the same partition of the partials as attn_decode's workspace
    a.o_part = static_cast<float *>(base);
    a.lse_part = static_cast<float *>(base) + (need / sizeof(float)) / (a.D + 1) * a.D;
  }
  return launch_decode(a);
}

size_t decode_workspace_bytes(int B, int H, int H_kv, int D, int max_len) {
  int nsplit, chunk;
  decode_split(B, H_kv, max_len, &nsplit, &chunk);
  if (nsplit == 1) return 0;
  return (size_t)nsplit * B * H * (D + 1) * sizeof(float);
}

}  // namespace attn
