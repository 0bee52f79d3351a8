/*
 * attn_api.h - C ABI of the fused causal scaled-dot-product attention library
 * (libcausal_attn.so), forward and backward, for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch b and head h, with queries and keys the
 * same sequence of S tokens and head dimension D:
 *
 *   S_ij   = scale * sum_d Q_id K_jd           (ARK: multi-head SDPA attention)
 *   S_ij   = -inf unless key j is allowed      (ARK: causal mask fused into the SDPA)
 *   P      = softmax over j of S (per row i)
 *   O      = P V,  LSE_i = ln sum_j exp(S_ij)  (natural log)
 *
 * and, given the upstream gradient dO, the analytic backward
 *
 *   Delta_i = sum_d dO_id O_id,  dP = dO V^T,  dS = P o (dP - Delta)
 *   dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO
 *
 * computed flash-attention style (Forge, "What this is" and "Acknowledgements":
 * forward and backward after FlashAttention-2): the forward keeps a running
 * row maximum and sum and stores only O and LSE; the backward recomputes P from
 * LSE tile by tile.  No S x S matrix is ever stored.
 *
 * Masks.
 *   ATTN_MASK_CAUSAL:     key j allowed for query i iff j <= i.
 *   ATTN_MASK_DOC_CAUSAL: packed documents (Cort33x, "Preserving context in
 *     the data"): the sequence is the concatenation of n_seqs documents with
 *     boundaries cu_seqlens[0] = 0 <= cu_seqlens[1] <= ... <= cu_seqlens[n_seqs] = S
 *     (a document may be empty: it owns no rows and adds nothing);
 *     key j allowed for query i iff j <= i and both lie in the same document.
 *
 * Layout.  Q, K, V, dO, O, dQ, dK, dV are contiguous [B, H, S, D] row-major
 * (D fastest); LSE and Delta are contiguous [B, H, S].  In DOC_CAUSAL mode
 * B must be 1.  Q, K, V and dO share one input dtype (ATTN_DTYPE_F32, _BF16
 * or _F16; the 16-bit types run on the bf16 / fp16 matrix cores with fp32
 * accumulation, P and dS rounded to the input type); O, LSE, Delta, dQ, dK
 * and dV are always float32.
 *
 * Ownership.  Every pointer except where noted is a DEVICE pointer on the
 * current HIP device, allocated and owned by the caller.  The library never
 * allocates, frees, copies between host and device or synchronises, and it is
 * safe to call from several threads.  It keeps no state between calls, with
 * one exception: attn_decode_noalloc's static device buffer and that buffer's
 * per-device address, looked up once under a lock.
 * Outputs are fully overwritten (no accumulation, no need to clear them first).
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls
 * return after enqueueing; results are valid once the stream has completed.
 *
 * Errors.  Arguments are validated before any HIP call; an invalid call
 * returns a negative attn_status and touches no memory.  A failed kernel
 * launch returns ATTN_ERR_HIP.  The library never aborts and never throws.
 * The contents of device cu_seqlens are NOT validated (that would need a
 * synchronisation); a malformed array gives unspecified results.
 *
 * Supported: D in {32, 64, 128}; S >= 1; B, H >= 1; B*H*S*D < 2^31;
 * S*D < 2^29 (one head's fp32 output under 2 GiB); scale finite and > 0.
 */
#ifndef CAUSAL_ATTN_API_H
#define CAUSAL_ATTN_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,          /* a required pointer is NULL                       */
  ATTN_ERR_SHAPE = -2,         /* B, H or S out of range, or sizes overflow        */
  ATTN_ERR_HEAD_DIM = -3,      /* D not in {32, 64, 128}                           */
  ATTN_ERR_DTYPE = -4,         /* unknown input dtype                              */
  ATTN_ERR_MASK = -5,          /* unknown mask mode                                */
  ATTN_ERR_SEQLENS = -6,       /* DOC_CAUSAL with B != 1, n_seqs < 1, max_seqlen
                                  outside 1..S, or ceil(max_seqlen/64)*n_seqs*H >= 2^31
                                  (n_seqs may exceed S when documents are empty) */
  ATTN_ERR_HIP = -7,           /* a HIP runtime call or kernel launch failed       */
  ATTN_ERR_UNIMPLEMENTED = -8, /* valid request the library does not implement     */
  ATTN_ERR_SCALE = -9,         /* scale not finite or not > 0                      */
  ATTN_ERR_HEADS = -10,        /* H_kv not a divisor of H (grouped-query calls)    */
  ATTN_ERR_WORKSPACE = -11,    /* workspace missing, misaligned or too small       */
  ATTN_ERR_ROPE = -12,         /* RoPE table NULL or shorter than the positions,
                                  or base not finite and > 0                       */
  ATTN_ERR_STRIDE = -13,       /* attn_params strides out of range                 */
  ATTN_ERR_SCRATCH = -14       /* attn_decode_noalloc: the split needs more than
                                  ATTN_DECODE_SCRATCH_BYTES of scratch             */
} attn_status;

enum { ATTN_MASK_CAUSAL = 0, ATTN_MASK_DOC_CAUSAL = 1 };
enum { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1, ATTN_DTYPE_F16 = 2 };

/*
 * Forward.  Reads q, k, v [B,H,S,D] (dtype), writes o [B,H,S,D] float32 and,
 * unless lse is NULL, lse [B,H,S] float32 (natural-log logsumexp of each
 * row's scaled, masked scores; the backward needs it).
 * cu_seqlens: device int32 [n_seqs+1], used only in DOC_CAUSAL mode (may be
 * NULL otherwise); n_seqs and max_seqlen (the longest document, 1..S) are
 * host integers used to size the launch, ignored in CAUSAL mode.
 */
int attn_fwd(const void *q, const void *k, const void *v, float *o, float *lse,
             int B, int H, int S, int D, float scale, int mask_mode,
             const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
             int dtype, void *stream);

/*
 * Backward.  Reads q, k, v, dO (dtype), o and lse (float32, from attn_fwd
 * with the same arguments) and writes dq, dk, dv [B,H,S,D] float32.
 * delta: caller-owned float32 workspace of B*H*S elements; on return it holds
 * Delta_i = sum_d dO_id O_id.  The call is exactly attn_bwd_dq_delta, then
 * attn_bwd_dkdv, below (bit for bit).
 */
int attn_bwd(const void *q, const void *k, const void *v, const float *o,
             const void *dO, const float *lse, float *dq, float *dk, float *dv,
             float *delta, int B, int H, int S, int D, float scale, int mask_mode,
             const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
             int dtype, void *stream);

/*
 * The backward's stages, exported separately so that callers (and timing
 * harnesses) can schedule or measure them one by one.
 *
 * attn_bwd_preprocess: delta[B*H*S] = rowsum(dO o O).  S, D, dtype as above.
 * attn_bwd_dkdv: dk, dv from q, k, v, dO, lse, delta (loops over query tiles
 *   for each key tile).
 * attn_bwd_dq: dq from q, k, v, dO, lse, delta (loops over key tiles for
 *   each query tile).
 * attn_bwd_dq_delta: delta and dq in one call, from o instead of delta.
 *   16-bit inputs: one kernel, the dQ kernel computing each row's Delta from
 *   O and dO on the way (one pass over O and dO fewer); fp32 inputs:
 *   attn_bwd_preprocess then attn_bwd_dq.  Either way delta and dq are bit
 *   for bit those of attn_bwd_preprocess followed by attn_bwd_dq.
 *
 * attn_bwd is attn_bwd_dq_delta, then attn_bwd_dkdv; dK/dV needs only the
 * Delta that the first stage writes.
 */
int attn_bwd_preprocess(const float *o, const void *dO, float *delta,
                        int B, int H, int S, int D, int dtype, void *stream);

int attn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dO,
                  const float *lse, const float *delta, float *dk, float *dv,
                  int B, int H, int S, int D, float scale, int mask_mode,
                  const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                  int dtype, void *stream);

int attn_bwd_dq(const void *q, const void *k, const void *v, const void *dO,
                const float *lse, const float *delta, float *dq,
                int B, int H, int S, int D, float scale, int mask_mode,
                const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                int dtype, void *stream);

int attn_bwd_dq_delta(const void *q, const void *k, const void *v, const float *o,
                      const void *dO, const float *lse, float *dq, float *delta,
                      int B, int H, int S, int D, float scale, int mask_mode,
                      const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                      int dtype, void *stream);

/*
 * Grouped-query attention (Forge, "Architecture": attention with GQA behind
 * an interface).  H query heads share H_kv key/value heads (H_kv divides H;
 * H_kv = H is plain multi-head attention, H_kv = 1 multi-query): query head h
 * of batch entry b attends with key/value head h / (H / H_kv) of that entry.
 * k, v, dk, dv are [B, H_kv, S, D]; q, o, dO, dq are [B, H, S, D]; lse and
 * delta [B, H, S].  dK and dV of a key/value head sum the contributions of
 * all its query heads, in a fixed order (no atomics: results are bitwise
 * reproducible).  Other arguments and rules as attn_fwd / attn_bwd, which are
 * these calls with H_kv = H.  Returns ATTN_ERR_HEADS if H_kv does not divide H.
 */
int attn_fwd_gqa(const void *q, const void *k, const void *v, float *o, float *lse,
                 int B, int H, int H_kv, int S, int D, float scale, int mask_mode,
                 const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                 int dtype, void *stream);

int attn_bwd_gqa(const void *q, const void *k, const void *v, const float *o,
                 const void *dO, const float *lse, float *dq, float *dk, float *dv,
                 float *delta, int B, int H, int H_kv, int S, int D, float scale,
                 int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                 int dtype, void *stream);

/*
 * attn_bwd_gqa with a workspace, for few key/value heads at long context.
 * dK and dV of a key/value head sum over its G = H / H_kv query heads; the
 * plain call runs the G heads one after the other through each key block,
 * so with few key/value heads few, long chains of work set the time.  Given
 * a workspace, the call splits each group into P parts of G / P heads run
 * side by side; each part writes its dK and dV into the workspace, then
 * the parts are added in part order (deterministic, bitwise reproducible;
 * rounded differently from attn_bwd_gqa, which sums the heads in one chain).
 * The split applies to 16-bit inputs with fewer than 1024 dK/dV workgroups
 * (B * H_kv * ceil(S / bn), or n_seqs * H_kv * ceil(max_seqlen / bn) for
 * packed documents): at D = 128 with an even group size (bn = 64 keys per
 * workgroup), at D <= 64 with G >= 8 (bn = 128). P is the smallest divisor
 * of G that brings the workgroups to 1024, else G.
 * attn_bwd_gqa_workspace_bytes returns the bytes the split needs for these
 * arguments: 2 * P * B * H_kv * S * D * 4, or 0 where the split does not
 * apply (and for invalid arguments). With 0 bytes, workspace may be NULL
 * and the call is exactly attn_bwd_gqa.
 * workspace: caller-owned DEVICE memory, 16-byte aligned, of at least that
 * many bytes. Its contents on return are unspecified. It must not overlap
 * the other arguments. Arguments and errors as attn_bwd_gqa, plus
 * ATTN_ERR_WORKSPACE if the workspace is needed and is NULL, misaligned or
 * too small. attn_bwd_ex takes the same workspace in attn_params (with any
 * output type, strides and RoPE; the size is the same).
 */
size_t attn_bwd_gqa_workspace_bytes(int B, int H, int H_kv, int S, int D, int mask_mode,
                                    int n_seqs, int max_seqlen, int dtype);

int attn_bwd_gqa_ws(const void *q, const void *k, const void *v, const float *o,
                    const void *dO, const float *lse, float *dq, float *dk, float *dv,
                    float *delta, int B, int H, int H_kv, int S, int D, float scale,
                    int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                    int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode step against a key/value cache (Forge, "Roadmap": KV cache for
 * generation).  For each batch entry b and query head h, one new query -- the
 * newest token, whose own key and value are already appended to the cache --
 * attends keys 0 .. cache_lens[b] - 1 of its key/value head h / (H / H_kv):
 *
 *   O[b,h] = softmax_j(scale * q[b,h] . k_cache[b,kv,j]) v_cache[b,kv,:],
 *   LSE[b,h] = ln sum_j exp(scale * q[b,h] . k_cache[b,kv,j]).
 *
 * q: [B, H, D] (dtype); k_cache, v_cache: [B, H_kv, S_max, D] (dtype; only the
 * first cache_lens[b] rows of batch entry b are read); cache_lens: DEVICE
 * int32 [B], each in 1 .. max_len; max_len: host int, the largest length
 * (sizes the launch), 1 <= max_len <= S_max.  o: [B, H, D] float32; lse:
 * [B, H] float32 or NULL.  H / H_kv <= 32.
 * workspace: caller-owned device memory of attn_decode_workspace_bytes(B, H,
 * H_kv, D, max_len) bytes (the keys are split into chunks whose partial results
 * are merged exactly; 0 bytes, and workspace may be NULL, when one chunk
 * suffices).  Contents on return are unspecified.  Errors as for attn_fwd;
 * ATTN_ERR_WORKSPACE if the workspace is missing or too small,
 * ATTN_ERR_UNIMPLEMENTED if H / H_kv > 32.  cache_lens is not validated.
 */
size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int D, int max_len);

int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                const int32_t *cache_lens, float *o, float *lse,
                void *workspace, size_t workspace_bytes,
                int B, int H, int H_kv, int S_max, int D, float scale, int max_len,
                int dtype, void *stream);

/*
 * The same decode step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument, and no allocation by the library.  The
 * chunk partials go to a static device buffer of ATTN_DECODE_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends (its
 * address is looked up once per device, on the first call there).  The
 * kernels, the split and the results are those of attn_decode.  Calls whose
 * split needs more than ATTN_DECODE_SCRATCH_BYTES (attn_decode_workspace_bytes
 * larger) return ATTN_ERR_SCRATCH and touch no memory.  Every call on one GPU
 * shares that GPU's buffer: calls that overlap on one GPU (different streams,
 * or threads) race and must be ordered by the caller; calls on one stream are
 * ordered by it.  Nothing in the buffer needs clearing: each call writes every
 * partial it reads.  Other arguments and errors as attn_decode.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *cache_lens, float *o, float *lse,
                        int B, int H, int H_kv, int S_max, int D, float scale, int max_len,
                        int dtype, void *stream);

/*
 * Rotary position embedding (RoPE) of queries and keys: RoFormer (Su et al.
 * 2021, cited by ARK, whose model applies it from precomputed sine/cosine
 * tables: ARK, "Inference architecture (EKO)" and the model table's
 * "Positional encoding" row; Forge, "Architecture": attention with GQA and
 * RoPE).  Pair i = (x[2i], x[2i+1]) of a row at position p turns by the angle
 * p * theta_i, theta_i = base^(-2i/D):
 *
 *   y[2i]   = x[2i] cos(p theta_i) - x[2i+1] sin(p theta_i)
 *   y[2i+1] = x[2i] sin(p theta_i) + x[2i+1] cos(p theta_i)
 *
 * Positions are sequence indices 0 .. S-1 (ATTN_MASK_CAUSAL) or offsets from
 * the start of the row's document (ATTN_MASK_DOC_CAUSAL: every document is
 * its own sequence).  Values are not rotated.
 *
 * attn_rope_table: fills tab, DEVICE float32 [n_pos, D/2, 2], with
 *   tab[p][i] = (cos(p theta_i), sin(p theta_i)), angles computed in double
 *   precision.  A model builds it once and passes it to every call below.
 *   Errors: ATTN_ERR_NULL, ATTN_ERR_HEAD_DIM, ATTN_ERR_SHAPE (n_pos < 1 or
 *   n_pos * D >= 2^31), ATTN_ERR_ROPE (base not finite and > 0).
 *
 * attn_rope: q_rot = rotate(q) [B, H, S, D], k_rot = rotate(k) [B, H_kv, S, D],
 *   computed in fp32 and stored in the input dtype (16-bit: round to nearest
 *   even).  q_rot may equal q and k_rot may equal k (in place); other
 *   overlaps are undefined.
 *
 * attn_fwd_rope: attn_rope, then attn_fwd_gqa on q_rot and k_rot.  The caller
 *   keeps q_rot and k_rot (caller-owned, [B, H, S, D] and [B, H_kv, S, D] in
 *   the input dtype) for the backward, as saved activations.
 *
 * attn_bwd_rope: attn_bwd_gqa on q_rot, k_rot (as written by attn_fwd_rope),
 *   with dq and dk turned back by the opposite angles in the kernels'
 *   epilogues: dq, dk are gradients with respect to the UNROTATED q and k
 *   (the rotation's derivative; the dtype rounding of q_rot, k_rot passes the
 *   gradient unchanged).  dv, delta as attn_bwd_gqa.
 *
 * tab must hold n_pos >= S positions (causal) or n_pos >= max_seqlen (packed
 * documents), else ATTN_ERR_ROPE.  Other arguments, layouts, ownership and
 * errors as attn_fwd_gqa / attn_bwd_gqa.
 */
int attn_rope_table(float *tab, int n_pos, int D, float base, void *stream);

int attn_rope(const void *q, const void *k, void *q_rot, void *k_rot,
              const float *tab, int n_pos, int B, int H, int H_kv, int S, int D,
              int mask_mode, const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
              int dtype, void *stream);

int attn_fwd_rope(const void *q, const void *k, const void *v, void *q_rot, void *k_rot,
                  float *o, float *lse, const float *tab, int n_pos,
                  int B, int H, int H_kv, int S, int D, float scale, int mask_mode,
                  const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                  int dtype, void *stream);

int attn_bwd_rope(const void *q_rot, const void *k_rot, const void *v, const float *o,
                  const void *dO, const float *lse, float *dq, float *dk, float *dv,
                  float *delta, const float *tab, int n_pos,
                  int B, int H, int H_kv, int S, int D, float scale, int mask_mode,
                  const int32_t *cu_seqlens, int n_seqs, int max_seqlen,
                  int dtype, void *stream);

/*
 * One forward or backward call with every option at once: grouped key/value
 * heads, RoPE, and 16-bit outputs.  Zero-initialise an attn_params, then set
 * the fields the call uses; the plain entry points above are these calls with
 * H_kv = H, no RoPE and fp32 outputs (same kernels, same results).
 *
 *   q, k, v       inputs, [B, H, S, D] and [B, H_kv, S, D] in `dtype`.  With
 *                 RoPE these are the UNROTATED q and k: attn_fwd_ex rotates
 *                 them into q_rot, k_rot; attn_bwd_ex does not read them.
 *   dO            backward only: dL/dO, [B, H, S, D] in `dtype`.
 *   o             [B, H, S, D] in `out_dtype`: forward output, backward input.
 *   lse           [B, H, S] fp32: forward output (may be NULL there),
 *                 backward input.
 *   dq, dk, dv    backward outputs in `out_dtype`: [B, H, S, D] and
 *                 [B, H_kv, S, D] twice; gradients of the unrotated q, k.
 *   delta         backward workspace [B, H, S] fp32 (holds Delta on return),
 *                 computed from `o` as stored.
 *   B, H, H_kv, S, D, scale, mask_mode, cu_seqlens, n_seqs, max_seqlen,
 *   dtype         as attn_fwd_gqa (H_kv = 0 means H).
 *   out_dtype     ATTN_DTYPE_F32 (0) for fp32 outputs, or `dtype` itself
 *                 (bf16 or fp16 inputs only) to store O, dQ, dK and dV in the
 *                 input type, rounded to nearest even once at the store.
 *                 Anything else: ATTN_ERR_DTYPE.  LSE and Delta stay fp32.
 *   rope_table    NULL: no RoPE.  Else a table from attn_rope_table with
 *   rope_npos     rope_npos positions (>= S, or >= max_seqlen for packed
 *                 documents; else ATTN_ERR_ROPE).
 *   q_rot, k_rot  with RoPE: the rotated q and k in `dtype` (caller-owned,
 *                 contiguous), written by attn_fwd_ex and read by
 *                 attn_bwd_ex.
 *   strides       element strides {batch, head, sequence} of q, k, v, o, dO,
 *                 dq, dk, dv (ATTN_STRIDE_Q ... ATTN_STRIDE_DV); the D
 *                 elements of a row are always contiguous.  A row of zeros
 *                 means that tensor is contiguous [B, H, S, D] (H_kv heads
 *                 for k, v, dk, dv), so a zero-initialised struct is the
 *                 contiguous layout.  This is how [B, S, H, D] tensors
 *                 ({S*H*D, D, H*D}) or q, k, v slices of a fused projection
 *                 are passed without copies.  Each given row needs batch and
 *                 head strides >= 0, a sequence stride >= D, and
 *                 ((S + 255) * sequence stride + D) * element size < 2^31
 *                 bytes; else ATTN_ERR_STRIDE.  Inputs may overlap (a zero
 *                 head stride broadcasts one head); outputs must not overlap
 *                 one another or the inputs (not checked).
 *   workspace,    attn_bwd_ex only: NULL (no workspace), or a device
 *   workspace_bytes  workspace as for attn_bwd_gqa_ws, of at least
 *                 attn_bwd_gqa_workspace_bytes(B, H, H_kv, S, D, mask_mode,
 *                 n_seqs, max_seqlen, dtype) bytes, with which grouped heads
 *                 split their dK/dV step (ATTN_ERR_WORKSPACE if too small or
 *                 misaligned).  attn_fwd_ex ignores both.
 *
 * Errors, ownership and stream rules as the entry points above; a NULL
 * params pointer returns ATTN_ERR_NULL.
 */
typedef struct attn_params {
  const void *q, *k, *v, *dO;
  void *o;
  float *lse;
  void *dq, *dk, *dv;
  float *delta;
  int B, H, H_kv, S, D;
  float scale;
  int mask_mode;
  const int32_t *cu_seqlens;
  int n_seqs, max_seqlen;
  int dtype, out_dtype;
  const float *rope_table;
  int rope_npos;
  void *q_rot, *k_rot;
  int64_t strides[8][3];
  void *workspace;
  size_t workspace_bytes;
} attn_params;

enum {
  ATTN_STRIDE_Q = 0, ATTN_STRIDE_K, ATTN_STRIDE_V, ATTN_STRIDE_O, ATTN_STRIDE_DO, ATTN_STRIDE_DQ,
  ATTN_STRIDE_DK, ATTN_STRIDE_DV
};

int attn_fwd_ex(const attn_params *p, void *stream);

int attn_bwd_ex(const attn_params *p, void *stream);

/*
 * Measurement helper, not part of the attention path: one wave that reads the
 * shader-clock counter and the constant 100 MHz real-time counter, sleeps
 * between reads until `ticks` real-time ticks have passed (or 2^24 reads),
 * then writes out[0] = shader-clock cycles elapsed and out[1] = real-time
 * ticks elapsed (out: DEVICE memory, 2 x uint64, caller-owned).  Launched on
 * a stream of its own while a workload runs, out[0] / out[1] x 100 MHz is
 * the graphics clock of the chiplet it ran on during the workload.  Errors:
 * ATTN_ERR_NULL, ATTN_ERR_SHAPE (ticks 0), ATTN_ERR_HIP.
 */
int attn_clock_probe(unsigned long long *out, unsigned long long ticks, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *attn_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int attn_abi_version(void);

/*
 * Static, NUL-terminated identifier of the sources this library was built
 * from: a digest of the kernel sources, this header and the compiler flags,
 * fixed at build time.  A caller that holds the sources can recompute it and
 * refuse a library built from other sources.
 */
const char *attn_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* CAUSAL_ATTN_API_H */
