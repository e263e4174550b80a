/*
 * attn_jvp.h — C ABI of the MI355X (gfx950) attention forward + JVP library.
 *
 * One call computes, for every (batch b, head h), softmax attention and its
 * forward-mode derivative (Jacobian-vector product) along the tangents
 * (tQ, tK, tV):
 *
 *   S   = scale * Q K^T                    P  = row-softmax(S)
 *   O   = P V                              lse = log(sum_j exp(S_ij))  (natural log)
 *   tS  = scale * (tQ K^T + Q tK^T)        mu = sum_j P_ij tS_ij
 *   tO  = P tV + (P * (tS - mu)) V
 *
 * This is the fused "FlashAttention-2 forward with the JVP embedded" that the
 * rCM pages describe: papernotes.org reading notes on "Large Scale Diffusion
 * Distillation via Score-Regularized Continuous-Time Consistency", section
 * "Key designs", item 1 (a kernel returning the attention output together with
 * its JVP, for self- and cross-attention); ai.info summary of the same paper,
 * "Key Contributions" item 1 and "Methodology in Plain English" (tangents
 * carried through the same block-wise tiling, layers exposing forward/tangent
 * functions).  The JVP itself is the Jacobian applied to the tangent (notes on
 * "Consistent Distribution Matching for Data-Free Diffusion Distillation",
 * prerequisites, "JVP").  Self-attention is Lq == Lk with shared sequence
 * length; cross-attention is any Lq != Lk.
 *
 * Readings where the pages are silent: scale carries no tangent; lse uses the
 * natural log of the scaled logits; there is no mask, dropout or bias.
 */
#ifndef ATTN_JVP_H
#define ATTN_JVP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_JVP_VERSION 10400 /* 1.4.0 */

/* Largest number of partial results one attn_jvp_merge call combines. */
#define ATTN_JVP_MAX_MERGE_PARTS 16

/* Element type of q, k, v, tq, tk, tv, o and to (lse is always float32). */
typedef enum {
  ATTN_JVP_FP32 = 0,        /* float32 in, float32 out.  The logits q.k are
                               accumulated in float64 (exact products of the
                               float32 operands) and each softmax exponent is
                               formed in float64 and rounded once to float32;
                               every other product and sum is float32.  O and tO
                               stay within 1e-5 of the largest element of the
                               exact result whatever the logits' magnitude
                               (tested up to scaled logits of standard deviation
                               100, and logits rising into the hundreds).
                               Key shards merged by attn_jvp_merge carry each
                               shard's float32 lse: their weights are exact to
                               about 2^-24 |lse|, so at |lse| near 1000 the
                               merged O and tO are off by up to ~2.5e-5 */
  ATTN_JVP_BF16 = 1,        /* bfloat16 in, bfloat16 out (round to nearest even),
                               bf16 matrix products with float32 accumulation.
                               P and P*tS meet V as bf16 values; O and tO are
                               normalised by the sum of those bf16 weights (lse
                               by the float32 sum), so the tangent-logit
                               centring cancels where one key carries a row.
                               At d = 128 the tangent logits are centred on a
                               per-row value before P*tS is rounded, so its
                               rounding scales with |scale*tS - c|, not
                               |scale*tS|.  Tested within 2e-2 of tO's and O's
                               largest element up to scaled-logit standard
                               deviations of 65-130 and tangent logits in the
                               hundreds */
  ATTN_JVP_BF16_F32OUT = 2  /* bfloat16 inputs as ATTN_JVP_BF16, o and to written as
                               float32 (attn_jvp_fwd, attn_jvp_fwd_part); for
                               attn_jvp_merge: float32 partials, bfloat16 result.
                               Key-shard partials kept in float32 are rounded to
                               bf16 once, after the merge.  Not accepted by
                               attn_jvp_proj or attn_jvp_rmsnorm_rope
                               (ATTN_JVP_EUNSUPPORTED). */
} attn_jvp_dtype_t;

typedef enum {
  ATTN_JVP_OK = 0,
  ATTN_JVP_EINVAL = 1,       /* NULL pointer, negative size, Lk == 0 with work to do,
                                scale not finite or not > 0, unknown dtype */
  ATTN_JVP_EUNSUPPORTED = 2, /* head dim not 64 or 128, or a size beyond the limits below */
  ATTN_JVP_EALIGN = 3,       /* a tensor pointer not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_JVP_ELAUNCH = 4       /* the HIP launch failed (no device, bad stream, ...);
                                attn_jvp_last_error() holds the HIP message */
} attn_jvp_status_t;

/*
 * attn_jvp_fwd — enqueue one fused attention forward + JVP pass.
 *
 * Arguments
 *   q, tq   [B, H, Lq, d]  queries and their tangent                (device, read only)
 *   k, tk   [B, H, Lk, d]  keys and their tangent                   (device, read only)
 *   v, tv   [B, H, Lk, d]  values and their tangent                 (device, read only)
 *           tk and tv may both be NULL: a frozen context, tK = tV = 0 (the
 *           text cross-attention of the pages: papernotes.org notes, "Key
 *           designs" item 1).  The bf16 path then skips the tK and tV
 *           products and copies (8 instead of 12 flops per logit and head
 *           dim); the result equals passing zero-filled tk, tv.
 *   o, to   [B, H, Lq, d]  outputs: attention output and its tangent (device, written),
 *                          float32 for ATTN_JVP_BF16_F32OUT
 *   lse     [B, H, Lq]     float32 row log-sum-exp of scale*QK^T     (device, written)
 *   B, H, Lq, Lk, d        sizes; d in {64, 128}
 *   scale                  logit scale (usually 1/sqrt(d)); finite and > 0
 *   dtype                  attn_jvp_dtype_t for all tensors but lse
 *   stream                 a hipStream_t passed as void*; NULL is the null stream
 *
 * Layout: every tensor is dense and contiguous, row-major in the order given,
 * d innermost.  Pointers are device addresses (memory from hipMalloc or a
 * framework allocator on the current device).
 *
 * Ownership: all buffers belong to the caller.  The library allocates nothing,
 * keeps no state between calls and may be called from several host threads.
 * Inputs are never written.  o, to and lse are fully overwritten; they must not
 * overlap any input or each other (results are undefined if they do).
 *
 * Execution: the work is enqueued on `stream` and the call returns without
 * synchronising.  For identical inputs and sizes the results are bitwise
 * reproducible.
 *
 * Errors: all argument checks run on the host before any HIP call, and a
 * failed check launches nothing.  Exactly one of tk, tv NULL is
 * ATTN_JVP_EINVAL.  B*H*Lq == 0 is a no-op returning ATTN_JVP_OK
 * (pointers are then not inspected).  Limits: Lq*d and Lk*d below 2^29
 * elements per head; B*H*ceil(Lq/128), the number of 256-thread workgroups,
 * below 2^24 (a launch keeps its thread count below 2^32); beyond them the
 * call returns ATTN_JVP_EUNSUPPORTED and launches nothing.  The library never
 * aborts.
 * Non-finite input values propagate into the outputs; they are not detected.
 */
int attn_jvp_fwd(const void* q, const void* k, const void* v,
                 const void* tq, const void* tk, const void* tv,
                 void* o, void* to, float* lse,
                 int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                 float scale, int dtype, void* stream);

/*
 * attn_jvp_fwd_part — attn_jvp_fwd over one shard of the keys, returning the
 * partial state that attn_jvp_merge combines exactly.
 *
 * The pages describe the fused kernel as usable under context parallelism,
 * with the tangents of Q, K and V distributed like Q, K and V themselves
 * (ai.info summary of "Large Scale Diffusion Distillation via Score-Regularized
 * Continuous-Time Consistency", "Methodology in Plain English"; papernotes.org
 * notes, "Key designs" item 1).  With the keys split over shards, each shard's
 * softmax-normalised result is a complete description of its keys once the
 * tangent of its log-sum-exp is kept as well:
 *
 *   tlse = d/dt lse = sum_j P_ij tS_ij     (mu above; natural-log units)
 *
 * Arguments are those of attn_jvp_fwd, plus
 *   k, tk, v, tv   point at the first key row of the shard in [B, H, kv_rows, d]
 *                  tensors: head (b, h) of the shard starts (b*H + h)*kv_rows*d
 *                  elements after the pointer, and its Lk rows are used
 *   kv_rows        rows per head of the K/V tensors in memory, >= Lk, < 2^31
 *   tlse [B, H, Lq] float32, written with mu; may be NULL (then not written)
 * With kv_rows == Lk and tlse == NULL this is attn_jvp_fwd.
 * Errors: as attn_jvp_fwd; kv_rows < Lk is ATTN_JVP_EINVAL.
 */
int attn_jvp_fwd_part(const void* q, const void* k, const void* v,
                      const void* tq, const void* tk, const void* tv,
                      void* o, void* to, float* lse, float* tlse,
                      int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t kv_rows, int64_t d,
                      float scale, int dtype, void* stream);

/*
 * attn_jvp_merge — exact merge of n results over disjoint key shards.
 *
 * For each of `rows` query rows (B*H*Lq for [B, H, Lq, d] tensors), with the
 * shard results (O_s, tO_s, lse_s, tlse_s) of attn_jvp_fwd_part:
 *   lse  = log sum_s exp(lse_s),      w_s = exp(lse_s - lse)
 *   O    = sum_s w_s O_s
 *   tlse = sum_s w_s tlse_s
 *   tO   = sum_s w_s (tO_s + (tlse_s - tlse) O_s)
 * which is the attention-JVP over the union of the shards' keys (up to
 * rounding; bf16 partials carry their own bf16 rounding into the merge).
 *
 * Arguments
 *   n                      number of shards, 1 .. ATTN_JVP_MAX_MERGE_PARTS
 *   o_parts, to_parts      host arrays of n device pointers, [rows, d] each, dtype
 *                          (float32 for ATTN_JVP_BF16_F32OUT, whose result is bf16)
 *   lse_parts, tlse_parts  host arrays of n device pointers, [rows] float32 each
 *   o, to                  [rows, d] outputs (device, written)
 *   lse                    [rows] float32 output (device, written)
 *   tlse                   [rows] float32 output, may be NULL (then not written)
 *   rows, d                d in {64, 128}
 *   dtype, stream          as attn_jvp_fwd (arithmetic is float32): FP32 parts give an
 *                          FP32 result, BF16 parts a BF16 result, BF16_F32OUT float32
 *                          parts a BF16 result
 * Ownership, alignment (16 bytes for [rows, d] tensors, 4 for [rows]),
 * execution and errors follow attn_jvp_fwd; rows == 0 is a no-op; outputs must
 * not overlap any input.  The host arrays are read during the call only.
 * Limit: ceil(rows*d/2048) (the workgroup count) below 2^24, else
 * ATTN_JVP_EUNSUPPORTED.
 */
int attn_jvp_merge(int n, const void* const* o_parts, const void* const* to_parts,
                   const float* const* lse_parts, const float* const* tlse_parts,
                   void* o, void* to, float* lse, float* tlse,
                   int64_t rows, int64_t d, int dtype, void* stream);

/*
 * attn_jvp_proj — the projection of hidden states into attention heads, with
 * its tangent: the layer that hands Q, K, V and their tangents to attn_jvp_fwd.
 *
 * The rCM pages refactor every layer of the distilled networks to take and
 * return tangents, and distribute the tangents of Q, K and V like Q, K and V
 * (ai.info summary of "Large Scale Diffusion Distillation via Score-Regularized
 * Continuous-Time Consistency", "Methodology in Plain English" and "Key
 * Contributions" item 1).  They name no architecture; this is the plain
 * reading, a linear layer with bias whose JVP is its linear part applied to
 * the tangent (a constant bias has no tangent):
 *
 *   Y  = X W^T + b          TY = TX W^T
 *
 * with output feature f = (n*H + h)*d + j of token t of batch b written to
 * element [n, b, h, t, j]: projection n (Q, K, V in that order for n_out = 3),
 * head h, in the [B, H, L, d] layout attn_jvp_fwd reads.  One pass computes
 * both products from the same weight tiles.
 *
 * Arguments
 *   x, tx  [B, L, D]            hidden states and their tangent (device, read only).
 *                               tx and ty may both be NULL: a frozen input (the text
 *                               context of a cross-attention), no tangent computed
 *   w      [n_out*H*d, D]       weight, row f holds output feature f (the layout of a
 *                               linear layer's weight)                  (device, read only)
 *   bias   [n_out*H*d] or NULL  added to Y only                         (device, read only)
 *   y, ty  [n_out, B, H, L, d]  outputs; projection n of the batch starts
 *                               n*B*H*L*d elements after the pointer     (device, written)
 *   B, L, D, n_out, H, d        sizes; d in {64, 128}; D a positive multiple of 64
 *   dtype                       ATTN_JVP_BF16 (bf16 products, float32 accumulation,
 *                               outputs rounded to nearest even); ATTN_JVP_FP32 is
 *                               ATTN_JVP_EUNSUPPORTED
 *   stream                      as attn_jvp_fwd
 *
 * Layout, ownership, alignment (16 bytes for every pointer), execution and
 * errors follow attn_jvp_fwd.  Exactly one of tx, ty NULL is ATTN_JVP_EINVAL;
 * B*L == 0 or n_out*H == 0 is a no-op.  Limits: L*D, n_out*H*d*D and L*d below
 * 2^31 elements, D below 2^22, and B*ceil(L/128)*ceil(n_out*H*d/256) (the
 * workgroup count) below 2^24; beyond them ATTN_JVP_EUNSUPPORTED.  Outputs must
 * not overlap any input.
 */
int attn_jvp_proj(const void* x, const void* tx, const void* w, const void* bias,
                  void* y, void* ty,
                  int64_t B, int64_t L, int64_t D, int64_t n_out, int64_t H, int64_t d,
                  int dtype, void* stream);

/*
 * attn_jvp_rmsnorm_rope — RMS normalisation and rotary position embedding of
 * the queries (or keys) of an attention layer, with the tangent: the layer
 * between attn_jvp_proj and attn_jvp_fwd.
 *
 * The rCM pages make every layer take and return tangents and hand the
 * tangents of Q and K to the attention kernel laid out like Q and K (ai.info
 * summary of "Large Scale Diffusion Distillation via Score-Regularized
 * Continuous-Time Consistency", "Methodology in Plain English" and "Key
 * Contributions" item 1); they do not describe the layer itself.  This is the
 * reading taken: each row x of d elements (token t of one head) is
 * normalised by its root mean square with a gain g, then adjacent pairs
 * (2i, 2i+1) are rotated by the angle of position t, given as tables; gain,
 * eps and angles are constants (no tangent):
 *
 *   r  = (mean_j x_j^2 + eps)^(-1/2)        n  = g * x * r
 *   tn = g * (tx * r - x * r^3 * mean_j x_j tx_j)
 *   y_2i = c n_2i - s n_2i+1,  y_2i+1 = s n_2i + c n_2i+1   (c = cos[t,i], s = sin[t,i])
 *   ty   = the same rotation of tn
 *
 * Arguments
 *   x, tx      [B, H, L, d]  rows and their tangent (device, read only); tx and ty may
 *                            both be NULL (no tangent)
 *   y, ty      [B, H, L, d]  outputs (device, written); y may be x and ty may be tx
 *                            (in place); any other overlap is undefined
 *   gamma      [d] gain in the element type, or NULL (gain 1)     (device, read only)
 *   rope_cos,  [L, d/2] float32 cos and sin of the angle of pair i at position t,
 *   rope_sin   or both NULL (no rotation: normalisation only)     (device, read only)
 *   B, H, L, d sizes; d in {64, 128}
 *   eps        finite, >= 0
 *   dtype      ATTN_JVP_BF16 (bf16 in and out, float32 arithmetic, outputs rounded to
 *              nearest even) or ATTN_JVP_FP32
 *   stream     as attn_jvp_fwd
 *
 * Alignment: every pointer 16 bytes.  Ownership, execution and errors follow
 * attn_jvp_fwd; exactly one of tx, ty NULL, or one of rope_cos, rope_sin, or a
 * negative or non-finite eps is ATTN_JVP_EINVAL; B*H*L == 0 is a no-op.
 * Limits: B*H and the workgroup count B*H*ceil(L/R) below 2^24, where R =
 * 2048/d rows per workgroup for bf16 and 1024/d for fp32; L below 2^31.
 */
int attn_jvp_rmsnorm_rope(const void* x, const void* tx, void* y, void* ty,
                          const void* gamma, const float* rope_cos, const float* rope_sin,
                          int64_t B, int64_t H, int64_t L, int64_t d, float eps,
                          int dtype, void* stream);

/* Static description of a status code ("unknown status" for others). */
const char* attn_jvp_status_string(int status);

/* Detail of the last failed call on the calling host thread ("" if none). */
const char* attn_jvp_last_error(void);

/* ATTN_JVP_VERSION of the built library. */
int attn_jvp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_JVP_H */
