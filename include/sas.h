/*
 * sas.h -- C ABI of libsas, SAS (Simple Attention Sparsification) gated
 * block-sparse attention for AMD Instinct MI355X (gfx950).
 *
 * The method, as the pages describe it:
 *   - block-sparse attention: the context is cut into blocks of b tokens, a
 *     selector scores each block, and a query attends only to the Top-K
 *     blocks (shibing624 blog post, section 问题动机 "motivation", block-sparse
 *     attention formula; jaehun.me review "SAS: Simple Attention
 *     Sparsification via End-to-End Optimization of Context Ranking",
 *     section "Background", paper Eq. 2 and Eq. 3);
 *   - SAS training attention: o = softmax(q K_S^T + log g_S) V_S with
 *     g = softmax(s) over the query's history blocks and gate 1 (bias 0) on the
 *     query's own block (blog section 方法核心 "method core"; review section
 *     "New Approach", paper Eq. 4 and Eq. 9; log g = s - LSE(s) in review
 *     section "Why the Four Design Choices Matter");
 *   - inference: hard Top-K on the scores, no gate (review section "How It
 *     Works: A Concrete Walkthrough", Step 6, paper Alg. 2);
 *   - the gate designs the pages compare SAS with (sigmoid gate, raw logit,
 *     gate outside the softmax, hard gate with a straight-through estimator:
 *     review section "Why the Four Design Choices Matter"; blog 方法核心,
 *     ablation table): sas_gated_attn_fwd_gate / sas_gated_attn_bwd_gate.
 *
 * Conventions shared by every call
 * --------------------------------
 *   Tensors are device memory owned by the caller, dense and row-major:
 *     q, o, dq, dO       [B, Hq,  N, D]    (decode: [B, Hq, D])
 *     k, v, dk, dv       [B, Hkv, N, D]    (decode caches: [B, Hkv, L_max, D])
 *     kbar               [B, Hkv, C, D]    pooled block keys, C = N / block
 *                                          (integer division; decode C = L_max / block)
 *     scores, ds         [B, Hq,  N, C]    fp32 (decode: [B, Hq, C])
 *     group-summed scores[B, Hkv, N, C]    fp32 (decode: [B, Hkv, C])
 *     idx                [B, Hkv, N, topk] int32 (decode: [B, Hkv, topk])
 *     lse, lse_s         [B, Hq,  N]       fp32 (decode lse: [B, Hq])
 *   `dtype` (sas_dtype) is the element type of q, k, v, o, dO, dq, dk, dv
 *   and kbar.  Query head h reads KV head h / (Hq / Hkv) (grouped-query
 *   attention).  `scale` multiplies q.k in the logits and in the selector
 *   score (1/sqrt(D) in the usual setting); it must be positive and finite.
 *
 *   Positions.  Training calls (cache_len == NULL) place query t at position
 *   t.  Decode calls place the single new token of sequence b at position
 *   cache_len[b] - 1 (its K and V are already in the cache); lengths above
 *   L_max count as L_max and a length <= 0 marks an idle sequence.
 *   The current block of a query at position p is c = p / block; its history
 *   is blocks 0 .. c-1 (complete blocks only).  The current block is always
 *   attended, causally, with bias 0.
 *
 *   idx: hard Top-K output, per (query token, KV head).  Entries outside
 *   [0, c) are ignored and a repeated entry counts once.  idx == NULL in the
 *   attention calls means full scope (every history block).
 *
 *   Every call validates all arguments on the host before touching the GPU;
 *   on failure it returns a negative sas_status, launches nothing, and
 *   sas_last_error() describes the problem.  Work is enqueued asynchronously
 *   on `stream` (a hipStream_t; NULL is the null stream): inputs must stay
 *   valid and outputs untouched until the stream reaches that point.  The
 *   library allocates no memory; calls that need scratch take a caller
 *   workspace of at least sas_workspace_bytes() bytes.  A workspace carries
 *   nothing from one call to the next, so calls enqueued in order on one
 *   stream may share one buffer of the largest size they need (the sparse
 *   forward and backward of a training step, for instance).  No call keeps a
 *   pointer after it returns.  Calls are thread-safe (the error string is
 *   thread-local).  Sizes of zero (B, Hq, N or L_max) are valid and do nothing.
 */
#ifndef SAS_H_
#define SAS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAS_OK = 0,
  SAS_EINVAL = -1,        /* an argument is invalid (shape, pointer, value) */
  SAS_EUNSUPPORTED = -2,  /* valid, but outside what the library implements */
  SAS_EHIP = -3,          /* the HIP runtime reported an error at launch */
  SAS_EWORKSPACE = -4     /* workspace missing or smaller than required */
} sas_status;

typedef enum { SAS_F32 = 0, SAS_BF16 = 1 } sas_dtype;

typedef enum {
  SAS_OP_SCORE = 1,
  SAS_OP_TOPK = 2,
  SAS_OP_FWD = 3,
  SAS_OP_BWD = 4,
  SAS_OP_DECODE = 5,
  SAS_OP_SELECTOR_BWD = 6,
  SAS_OP_PAGED_DECODE = 7,
  SAS_OP_FWD_GATE = 8,   /* sas_gated_attn_fwd_gate, any gate */
  SAS_OP_BWD_GATE = 9,   /* sas_gated_attn_bwd_gate, any gate */
  SAS_OP_DECODE_STEP = 10, /* sas_decode_step */
  SAS_OP_PREFILL = 11,     /* sas_prefill_paged (n_or_lmax = N, topk ignored) */
  SAS_OP_CTX = 12          /* the saved context of sas_gated_attn_fwd_ctx /
                              sas_gated_attn_bwd_ctx (0: none is used) */
} sas_op;

/* Gate activation of the gated attention (blog 方法核心, the ablation table's
   gate-activation row; review "Why the Four Design Choices Matter", gate
   activation): the SAS softmax gate and the two non-competitive gates the
   pages compare it with. */
typedef enum {
  SAS_GATE_SOFTMAX = 0,  /* log g = s - LSE_s over the history (SAS) */
  SAS_GATE_SIGMOID = 1,  /* log g = log sigmoid(s), per block */
  SAS_GATE_RAW = 2,      /* log g = s: the raw logit injected as a bias */
  SAS_GATE_OUTER = 3,    /* g = softmax(s) outside the softmax: it scales
                            each block's value contribution (review "Why
                            the Four Design Choices Matter", gate placement) */
  SAS_GATE_STE = 4       /* hard gate, straight-through estimator (same
                            section, ranking preservation) */
} sas_gate;

/*
 * sas_score_blocks -- block mean-pooling and selector scores.
 *   K̄[b,g,m,:] = mean of k over the `block` tokens of block m  (pooling-based
 *   block summaries: review section "Our Perspective", Limitations), and
 *   s[b,h,t,m] = scale * q[b,h,t] . K̄[b,h/G,m] for every history block
 *   m < c(t); all other columns are written as -inf (review "Background",
 *   paper Eq. 3: one relevance score per block).
 * k:          if non-NULL, kbar is first computed from k ([B,Hkv,L,D]) for
 *             all C = L/block complete blocks and written; if NULL, kbar is an
 *             input (decode: pooled keys kept beside the cache).
 * kbar:       [B,Hkv,C,D] in `dtype` (the mean is taken in fp32, then rounded).
 * scores:     fp32 output; [B,Hq,Nq,C], or with group_sum != 0 the per-KV-head
 *             sum [B,Hkv,Nq,C] (query heads added in index order, fp32).
 * cache_len:  NULL for training (Nq must equal L; query t at position t);
 *             device int32 [B] for decode (Nq must be 1).
 * Errors: SAS_EINVAL for null required pointers, Hq % Hkv != 0, block < 1,
 *         Nq/L mismatch; SAS_EUNSUPPORTED for D outside {64, 128} or, in decode
 *         mode, more than 16 query heads per KV head.
 */
int sas_score_blocks(const void* q, const void* k, void* kbar, float* scores,
                     const int32_t* cache_len, int B, int Hq, int Hkv, int Nq,
                     int L, int D, int block, float scale, int group_sum,
                     int dtype, void* stream);

/*
 * sas_score_blocks_lse -- the training-mode sas_score_blocks (cache_len NULL,
 *   group_sum 0, Nq = L = N) that also writes the softmax gate's normaliser
 *   LSE_s(t) = log sum_{m < c(t)} exp(s[t,m]) per query row (review "Why the
 *   Four Design Choices Matter": log g = s - LSE(s); -inf for rows without
 *   history), so that the forward need not read the scores a second time for
 *   it (sas_gated_attn_fwd_lse).
 * lse_s:   fp32 [B,Hq,N] output.  With bf16 and block % 16 == 0 the score
 *          kernel computes it from the scores it writes (fp32 running max and
 *          sum per row); otherwise a pass over the written scores does.  It
 *          matches the lse_s of sas_gated_attn_fwd up to fp32 summation order.
 * scores:  only the history columns m < c(t) of each row are written; the
 *          others (-inf in sas_score_blocks) are left as they are, since no
 *          call reads them: a caller that wants the dense form fills the
 *          tensor with -inf once.
 * Other arguments and errors: as sas_score_blocks.
 */
int sas_score_blocks_lse(const void* q, const void* k, void* kbar, float* scores,
                         float* lse_s, int B, int Hq, int Hkv, int N, int D,
                         int block, float scale, int dtype, void* stream);

/*
 * sas_topk_select -- hard Top-K over each row's history blocks (review
 *   "Background", paper Eq. 3; training selection per query token and KV
 *   head; review "A Concrete Walkthrough" Step 3 and Step 6).
 * scores:        fp32 [B, Hkv*heads_per_row, Nq, C]; the heads_per_row rows
 *                of one KV head are summed in fp32 in index order
 *                (heads_per_row = 1: already summed).
 * idx:           int32 [B, Hkv, Nq, topk] output: the min(topk, c) best
 *                history blocks, score descending, ties to the lower block
 *                index (-0.0 equals +0.0, NaN ranks as -inf), remaining slots
 *                -1.  Bit-exact and deterministic.
 * cache_len:     NULL: row t has c = t / block candidates (training, Nq rows);
 *                device int32 [B]: decode, Nq must be 1, c = min((len-1)/block, C)
 *                (0 for len <= 0).  Top-K does not know the cache capacity
 *                L_max: for every length up to L_max this is the history of
 *                sas_score_blocks and sas_sparse_decode, but a length above
 *                L_max with L_max a multiple of block makes block C-1 (the
 *                current block there, scored -inf) a candidate.  Callers that
 *                may pass such lengths clamp them to L_max first;
 *                sas_paged_decode does so itself.
 * workspace:     unused (no scratch is needed); may be NULL with size 0.
 *                sas_workspace_bytes(SAS_OP_TOPK, ...) returns 0.
 * Errors: SAS_EINVAL (pointers, sizes, topk < 0, heads_per_row < 1);
 *         SAS_EUNSUPPORTED for topk > 256 or C > 16384.
 */
int sas_topk_select(const float* scores, int32_t* idx, const int32_t* cache_len,
                    int B, int Hkv, int heads_per_row, int Nq, int C, int block,
                    int topk, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * sas_topk_select_gated -- sas_topk_select on training rows (cache_len NULL,
 *   c = t / block candidates) that also writes, for the selection, the
 *   softmax gate's base-2 log gates (review "Why the Four Design Choices
 *   Matter": log g = s - LSE(s)), which sas_gated_attn_fwd_ctx can take
 *   instead of gathering them from the scores again.
 * scores, idx:  as sas_topk_select; idx is the same, bit for bit.
 * lse_s:        fp32 [B, Hkv*heads_per_row, Nq] LSE_s of each query row (as
 *               sas_score_blocks_lse writes it).
 * gates:        fp32 [B, Hkv, Nq, topk, heads_per_row] output: slot j of row
 *               t holds, for the j-th smallest selected block m (ascending
 *               block order, j < min(topk, c)), (s[t,m] - LSE_s(t)) log2 e of
 *               each query head of the group, computed in fp32 in that
 *               order; slots from min(topk, c) on are not written.
 * Errors: as sas_topk_select; SAS_EUNSUPPORTED for C > 1024, topk > 64 or
 *         heads_per_row other than 1, 2, 4 and 8.
 */
int sas_topk_select_gated(const float* scores, const float* lse_s, int32_t* idx,
                          float* gates, int B, int Hkv, int heads_per_row,
                          int Nq, int C, int block, int topk, void* stream);

/*
 * sas_gated_attn_fwd -- SAS gated attention forward (blog 方法核心; review
 *   "New Approach", paper Eq. 9; tiled FlashAttention-style evaluation with
 *   an online softmax: review "A Concrete Walkthrough", kernel paragraph).
 *   z[t,j] = scale * q_t . k_j + bias, bias = 0 on the own block (j <= t),
 *   log g[t,m] = s[t,m] - LSE_s(t) on a gated history block m, -inf
 *   elsewhere; o = softmax(z) v.
 * scores:  fp32 [B,Hq,N,C] selector scores (columns m >= c(t) are not read).
 * idx:     NULL for full scope, else int32 [B,Hkv,N,topk] (sparse scope).
 * o:       [B,Hq,N,D] output in dtype.
 * lse:     fp32 [B,Hq,N] output, log-sum-exp of z per row.
 * lse_s:   fp32 [B,Hq,N] output, log-sum-exp of the row's history scores
 *          (-inf for rows without history).
 * N must be >= 0; a last block shorter than `block` is allowed.
 * Errors: SAS_EINVAL, SAS_EUNSUPPORTED (D outside {64, 128}; sparse scope
 *         with C > 16384 or topk > 256), SAS_EWORKSPACE.
 */
int sas_gated_attn_fwd(const void* q, const void* k, const void* v,
                       const float* scores, const int32_t* idx, void* o,
                       float* lse, float* lse_s, int B, int Hq, int Hkv, int N,
                       int D, int block, int topk, float scale, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * sas_gated_attn_fwd_lse -- sas_gated_attn_fwd with LSE_s given: lse_s
 *   (fp32 [B,Hq,N], e.g. from sas_score_blocks_lse on the same scores) is an
 *   input and is only read; the forward skips its own pass over the scores
 *   for it.  o and lse as sas_gated_attn_fwd; same workspace
 *   (SAS_OP_FWD) and errors.  Passing an LSE_s that does not belong to
 *   `scores` gives the attention of a different gate (no check is made).
 */
int sas_gated_attn_fwd_lse(const void* q, const void* k, const void* v,
                           const float* scores, const int32_t* idx,
                           const float* lse_s, void* o, float* lse, int B,
                           int Hq, int Hkv, int N, int D, int block, int topk,
                           float scale, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * sas_gated_attn_fwd_ctx / sas_gated_attn_bwd_ctx -- a training step's forward
 *   and backward with a saved context, as a framework keeps tensors from the
 *   forward for the backward.  The forward is sas_gated_attn_fwd_lse (LSE_s
 *   given); it also writes into `ctx` what the backward would otherwise
 *   rebuild or gather again: the selection lists of idx (the per-block lists
 *   of selecting tokens the key-major kernels walk) and, per (KV head, list
 *   entry, query head of the group), the base-2 log gate (s - LSE_s) log2 e
 *   of that history entry (review "Why the Four Design Choices Matter":
 *   log g = s - LSE(s)).  The backward is sas_gated_attn_bwd for the same
 *   inputs, reading the lists and log gates from `ctx` instead.
 * ctx:       caller-owned device buffer of at least
 *            sas_workspace_bytes(SAS_OP_CTX, B, Hq, Hkv, N, D, block, topk,
 *            dtype) bytes.  That is 0 where the context is not used (full
 *            scope, fp32, or shapes outside the matrix-core path); then ctx
 *            may be NULL and the calls equal sas_gated_attn_fwd_lse and
 *            sas_gated_attn_bwd.  Between the two calls the caller keeps it
 *            unchanged and passes the same scores, idx and LSE_s (no check is
 *            made: a context of other inputs gives wrong gradients).
 *            Unlike a workspace, it carries data from one call to the next.
 * gates (forward): NULL, or the log gates that sas_topk_select_gated wrote
 *            for these scores, LSE_s and idx (fp32 [B, Hkv, N, topk, Hq/Hkv]);
 *            the forward then reads them instead of gathering each selected
 *            entry's score (same values, so the same results).  Read only;
 *            SAS_EINVAL without idx.
 * ds (backward): the history columns m < c(t) as in sas_gated_attn_bwd; the
 *            other columns (0 there) may be left unwritten: a caller that
 *            wants the dense form fills ds with zeros once.
 * Other arguments, and errors: as sas_gated_attn_fwd_lse and
 *   sas_gated_attn_bwd; a missing or short ctx is SAS_EWORKSPACE.
 */
int sas_gated_attn_fwd_ctx(const void* q, const void* k, const void* v,
                           const float* scores, const int32_t* idx,
                           const float* lse_s, const float* gates, void* o,
                           float* lse, int B, int Hq, int Hkv, int N, int D,
                           int block, int topk, float scale, int dtype,
                           void* ctx, size_t ctx_bytes, void* workspace,
                           size_t workspace_bytes, void* stream);
int sas_gated_attn_bwd_ctx(const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* scores,
                           const int32_t* idx, const float* lse,
                           const float* lse_s, const void* ctx,
                           size_t ctx_bytes, void* dq, void* dk, void* dv,
                           float* ds, int B, int Hq, int Hkv, int N, int D,
                           int block, int topk, float scale, int dtype,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * sas_gated_attn_bwd -- gradients of the forward for an upstream dO
 *   (blog 方法核心, inner-gate gradient; review "Why the Four Design Choices
 *   Matter", paper Eq. 5; gradient path o -> g -> s of review "A Concrete
 *   Walkthrough", Step 5).
 *   With P = softmax(z), Delta = rowsum(dO * o), dZ = P * (dO V^T - Delta):
 *     dq = scale dZ K,  dk = scale dZ^T Q,  dv = P^T dO  (dk, dv summed over the
 *     query heads sharing a KV head); dq, dk, dv are taken at fixed s.
 *     dbeta[t,m] = sum of dZ over the keys of gated history block m,
 *     ds[t,m] = dbeta[t,m] - g[t,m] * sum_m' dbeta[t,m']   (m < c(t)), else 0.
 * o, lse, lse_s: the forward's outputs for the same inputs.
 * ds:      fp32 [B,Hq,N,C] output (dense: also unselected history blocks).
 * dq, dk, dv: outputs in dtype.
 * Errors: as for the forward.
 */
int sas_gated_attn_bwd(const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* scores,
                       const int32_t* idx, const float* lse, const float* lse_s,
                       void* dq, void* dk, void* dv, float* ds, int B, int Hq,
                       int Hkv, int N, int D, int block, int topk, float scale,
                       int dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * sas_gated_attn_fwd_gate / sas_gated_attn_bwd_gate -- the forward and the
 *   backward above with another gate activation (sas_gate).  Only the gated
 *   history blocks' bias and ds change; the own block keeps bias 0 and, at
 *   sparse scope, unselected blocks keep -inf:
 *     SAS_GATE_SOFTMAX  exactly sas_gated_attn_fwd / _bwd.
 *     SAS_GATE_SIGMOID  bias log sigmoid(s[t,m]); ds = dbeta (1 - sigmoid(s)).
 *     SAS_GATE_RAW      bias s[t,m];               ds = dbeta.
 *     SAS_GATE_OUTER    no bias on gated blocks; with p = softmax(z) and
 *                       g = softmax(s) over the history (1 on the own block),
 *                       o = sum_j g p_j v_j, and lse is the log-sum-exp of the
 *                       ungated z.  dg_m = sum over block m of p dO.v (paper
 *                       Eq. 5, outer), ds = g (dg - sum_m' g dg).
 *     SAS_GATE_STE      the forward is plain block-sparse attention over the
 *                       own and the selected blocks (lse = their LSE_S);
 *                       dq, dk, dv are its gradients; for every history
 *                       block, selected or dropped, dh_m = sum over block m
 *                       of exp(z - LSE_S) dO.(v - o), and ds = g (dh -
 *                       sum_m' g dh) with g = softmax(s).  The backward
 *                       visits every history block (full-scope work).
 *   The sigmoid and raw gates have no normaliser: their forward writes
 *   lse_s = 0, their backward ignores lse_s (it may be NULL), and ds of an
 *   unselected history block is 0.  The outer and STE gates write and read
 *   lse_s = LSE(s) as the softmax gate does.
 * gate:       a sas_gate value; anything else is SAS_EINVAL.
 * workspace:  sas_workspace_bytes(SAS_OP_FWD_GATE or SAS_OP_BWD_GATE, ...)
 *             bytes (the sigmoid gate keeps log sigmoid(s), fp32 [B,Hq,N,C],
 *             in it, the STE gate zero scores of that size and scratch
 *             gradients); SAS_GATE_SOFTMAX needs only SAS_OP_FWD / SAS_OP_BWD.
 * Other arguments, layouts, ownership and errors: as for the calls above.
 */
int sas_gated_attn_fwd_gate(const void* q, const void* k, const void* v,
                            const float* scores, const int32_t* idx, void* o,
                            float* lse, float* lse_s, int B, int Hq, int Hkv,
                            int N, int D, int block, int topk, float scale,
                            int dtype, int gate, void* workspace,
                            size_t workspace_bytes, void* stream);
int sas_gated_attn_bwd_gate(const void* q, const void* k, const void* v,
                            const void* o, const void* dout,
                            const float* scores, const int32_t* idx,
                            const float* lse, const float* lse_s, void* dq,
                            void* dk, void* dv, float* ds, int B, int Hq,
                            int Hkv, int N, int D, int block, int topk,
                            float scale, int dtype, int gate, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * sas_sparse_decode -- one decode step: each sequence's new token attends to
 *   its current block plus the selected history blocks, with no gate
 *   (review "A Concrete Walkthrough", Step 6, paper Alg. 2; block-sparse
 *   attention of blog 问题动机 and review "Background", paper Eq. 2).
 * q:          [B,Hq,D]; k_cache, v_cache [B,Hkv,L_max,D]; cache_len int32 [B]
 *             on the device.
 * idx:        int32 [B,Hkv,topk] selected history blocks, or NULL for dense
 *             decode over every cached position.
 * o:          [B,Hq,D] output in dtype (zeros for idle sequences).
 * lse:        optional fp32 [B,Hq] output (-inf for idle sequences).
 * Errors: SAS_EINVAL, SAS_EUNSUPPORTED (D outside {64, 128}, more than 16
 *         query heads per KV head, topk > 256), SAS_EWORKSPACE.
 */
int sas_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cache_len, const int32_t* idx, void* o,
                      float* lse, int B, int Hq, int Hkv, int L_max, int D,
                      int block, int topk, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * sas_decode_step -- one whole decode step for the new token of each sequence:
 *   group-summed selector scores of its history blocks from the pooled keys
 *   (as sas_score_blocks with group_sum), hard Top-K of them (as
 *   sas_topk_select, lengths clamped to L_max), then attention over the
 *   selected blocks and the current block with no gate (as sas_sparse_decode):
 *   the inference path of review "A Concrete Walkthrough", Step 6, paper
 *   Alg. 2, where at long contexts the selection stage is the bottleneck
 *   (review "Decoding Efficiency", Fig. 7c; "Our Perspective", Limitations).
 *   One call enqueues the separate calls' kernels in sequence (scores, Top-K,
 *   per-block attention partials, their merge) on one workspace; the results
 *   are those of the separate calls.
 * q:          [B,Hq,D]; kbar [B,Hkv,C,D] pooled keys (C = L_max / block, e.g.
 *             from sas_score_blocks with k = the cache); k_cache, v_cache
 *             [B,Hkv,L_max,D]; cache_len int32 [B] (above L_max counts as
 *             L_max; <= 0 is an idle sequence: o = 0, lse = -inf).
 * topk:       0 .. 256 blocks (0: the current block only).
 * o:          [B,Hq,D] output in dtype; lse optional fp32 [B,Hq] output.
 * idx_out:    optional int32 [B,Hkv,topk] output: the selected history blocks,
 *             score descending, ties to the lower index, -1 padding.
 * workspace:  sas_workspace_bytes(SAS_OP_DECODE_STEP, B, Hq, Hkv, L_max, D,
 *             block, topk, dtype) bytes, contents ignored.  After the call its
 *             first B*Hkv*C floats hold the group-summed scores [B,Hkv,C] the
 *             selection was made on (-inf for non-candidates).
 * Errors: SAS_EINVAL, SAS_EUNSUPPORTED (D outside {64, 128}, more than 16
 *         query heads per KV head, topk > 256, more than 16384 blocks),
 *         SAS_EWORKSPACE.
 */
int sas_decode_step(const void* q, const void* kbar, const void* k_cache,
                    const void* v_cache, const int32_t* cache_len, int topk,
                    void* o, float* lse, int32_t* idx_out, int B, int Hq, int Hkv,
                    int L_max, int D, int block, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sas_sparse_decode_noalloc -- sas_sparse_decode without a workspace argument,
 *   for callers that cannot allocate device memory (code under HIP graph
 *   capture, tight serving loops, harnesses that forbid allocation).  Same
 *   arguments, layouts, results and errors as sas_sparse_decode, minus the
 *   workspace; the same kernels run.
 * Scratch:    the attention partials go to a fixed scratch array of 8 MiB in
 *             the library, one per GPU, reserved when the library's code is
 *             loaded on that GPU and held until the process ends.  The call
 *             allocates nothing (no hipMalloc, hipFree or allocating library
 *             routine); its first call on a device looks up that device's
 *             array address once.  Every call on one GPU shares that GPU's
 *             array, so calls that overlap in time on one GPU (concurrent
 *             streams, or threads) race and must be serialised by the caller.
 *             No part of the array needs clearing between calls.
 * Errors:     as sas_sparse_decode; SAS_EUNSUPPORTED (with the byte count in
 *             sas_last_error) when the sizes need more scratch than the
 *             8 MiB array (sas_workspace_bytes(SAS_OP_DECODE, ...) > 8 MiB;
 *             e.g. dense decode far beyond 512K tokens per sequence),
 *             SAS_EHIP if the array's address cannot be obtained.
 */
int sas_sparse_decode_noalloc(const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* cache_len,
                              const int32_t* idx, void* o, float* lse, int B,
                              int Hq, int Hkv, int L_max, int D, int block,
                              int topk, float scale, int dtype, void* stream);

/*
 * Paged KV cache.  A page holds one block (`block` tokens) of one sequence for
 * every KV head: k_pages, v_pages [num_pages, Hkv, block, D], so each block
 * of each head stays one contiguous run.  block_table int32 [B, max_blocks]
 * on the device maps logical block m of sequence b to its page; the entries
 * for m <= (cache_len[b] - 1) / block must be valid page indices (they are
 * not checked).  kbar_pages [num_pages, Hkv, D] holds each full page's pooled
 * keys.
 *
 * sas_pool_pages -- kbar_pages[p, g] = mean of the block keys of page p, head g
 *   (pooling-based block summaries, review "Our Perspective"), for the n_pages
 *   page indices in `pages` (int32, device).  Errors: SAS_EINVAL,
 *   SAS_EUNSUPPORTED (D outside {64, 128}).
 */
int sas_pool_pages(const void* k_pages, void* kbar_pages, const int32_t* pages,
                   int n_pages, int Hkv, int D, int block, int dtype, void* stream);

/*
 * sas_paged_decode -- one decode step over a paged cache, the whole chain:
 *   group-summed selector scores of the history blocks from their pages'
 *   pooled keys (as sas_score_blocks), Top-K (as sas_topk_select), then
 *   attention over the selected blocks and the current block with no gate
 *   (as sas_sparse_decode; review "A Concrete Walkthrough", Step 6, paper
 *   Alg. 2).  It runs as sas_decode_step does, reading blocks and pooled
 *   keys through the block table.
 * q:          [B,Hq,D]; cache_len int32 [B] (a length above max_blocks *
 *             block counts as that; <= 0 is an idle sequence).
 * topk:       0 .. 256 blocks (0: the current block only).
 * o:          [B,Hq,D] output; lse optional fp32 [B,Hq] output.
 * idx_out:    optional int32 [B,Hkv,topk] output, the selected blocks
 *             (history blocks only: lengths are clamped to max_blocks * block).
 * workspace:  sas_workspace_bytes(SAS_OP_PAGED_DECODE, B, Hq, Hkv,
 *             max_blocks * block, D, block, topk, dtype) bytes.  After the
 *             call its first B*Hkv*max_blocks floats hold the group-summed
 *             scores [B,Hkv,max_blocks] the selection was made on (-inf for
 *             non-candidates), so a caller can check or reuse them.
 * bf16 only.  Errors: SAS_EINVAL, SAS_EUNSUPPORTED (fp32, D outside {64,
 *         128}, more than 16 query heads per KV head, topk > 256,
 *         max_blocks > 16384), SAS_EWORKSPACE.
 */
int sas_paged_decode(const void* q, const void* k_pages, const void* v_pages,
                     const void* kbar_pages, const int32_t* block_table,
                     int max_blocks, const int32_t* cache_len, int topk, void* o,
                     float* lse, int32_t* idx_out, int B, int Hq, int Hkv, int D,
                     int block, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * sas_prefill_paged -- the dense prefill of a serving engine that then decodes
 *   sparsely (blog 方法核心, kernel paragraph: dense prefill, sparse decode;
 *   review "Our Perspective", Strengths: paged KV cache): plain causal
 *   attention over each prompt (no gate: every key at or before the row), and
 *   the prompt's keys and values written into the pages of its blocks with the
 *   pooled key (mean of the block's keys, taken in fp32) of every complete
 *   block, ready for sas_paged_decode.
 * q:          [B,Hq,N,D]; k, v [B,Hkv,N,D]: the prompts, padded to N tokens.
 * seq_len:    int32 [B] on the device: prompt lengths (above N counts as N;
 *             <= 0: nothing is written to the pages of that sequence).
 * o:          [B,Hq,N,D] output; rows t < seq_len[b] hold the attention
 *             output (rows of padding tokens hold finite values of no meaning).
 * lse:        optional fp32 [B,Hq,N] output (log-sum-exp of each row's logits).
 * k_pages, v_pages [num_pages,Hkv,block,D], kbar_pages [num_pages,Hkv,D] and
 *             block_table int32 [B,max_blocks] as for sas_paged_decode; the
 *             entries for blocks m <= (seq_len[b] - 1) / block must be valid
 *             page indices (not checked).  Rows t < seq_len[b] are written to
 *             row t % block of page block_table[b, t / block]; kbar_pages is
 *             written for the complete blocks only (a partial last block is
 *             pooled with sas_pool_pages once it fills during decode).
 * workspace:  sas_workspace_bytes(SAS_OP_PREFILL, B, Hq, Hkv, N, D, block, 0,
 *             dtype) bytes, contents ignored.
 * Errors: SAS_EINVAL (pointers, sizes, N > max_blocks * block), SAS_EUNSUPPORTED
 *         (D outside {64, 128}), SAS_EWORKSPACE.
 */
int sas_prefill_paged(const void* q, const void* k, const void* v,
                      const int32_t* seq_len, void* o, float* lse,
                      void* k_pages, void* v_pages, void* kbar_pages,
                      const int32_t* block_table, int max_blocks, int B, int Hq,
                      int Hkv, int N, int D, int block, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * sas_selector_bwd -- gradient of the mean-pool selector score for an upstream
 *   ds (the last link of the gradient path output -> gate -> score ->
 *   selector, review "A Concrete Walkthrough", Step 5; pooling-based block
 *   summaries, review "Our Perspective").  With s[b,h,t,m] = scale q.K̄ for
 *   history blocks m < c(t) = t / block (sas_score_blocks) and K̄ the mean of
 *   each complete block of k:
 *     dq[b,h,t]  = scale * sum_{m < c(t)} ds[b,h,t,m] kbar[b,g,m]
 *     dkbar[b,g,m] = scale * sum_{h of group g} sum_{t: m < c(t)} ds[b,h,t,m] q[b,h,t]
 *     dk[b,g,j]  = dkbar[b,g,j / block] / block  (j in a complete block; 0 in the tail)
 *   Entries of ds with m >= c(t) are ignored.
 * q:          [B,Hq,N,D] in dtype; kbar: [B,Hkv,C,D] in dtype, C = N / block
 *             (the pooled keys the scores were computed from).
 * ds:         fp32 [B,Hq,N,C] (e.g. the ds output of sas_gated_attn_bwd).
 * dq, dk:     [B,Hq,N,D] / [B,Hkv,N,D] outputs in dtype.  accumulate = 0
 *             overwrites them; 1 adds this gradient to what they hold (the
 *             sum is formed in fp32 and rounded once), e.g. to the dq and dk
 *             of sas_gated_attn_bwd.
 * dkbar:      optional fp32 [B,Hkv,C,D] output (NULL: not written).
 * workspace:  sas_workspace_bytes(SAS_OP_SELECTOR_BWD, ...) bytes (fp32
 *             partial sums of dkbar over token chunks), contents ignored.
 * bf16 contracts ds rounded to bf16 on the matrix cores (fp32 accumulation);
 * fp32 accumulates in fp32 throughout.
 * Errors: SAS_EINVAL, SAS_EUNSUPPORTED (D outside {64, 128}), SAS_EWORKSPACE.
 */
int sas_selector_bwd(const void* q, const void* kbar, const float* ds, void* dq,
                     void* dk, float* dkbar, int B, int Hq, int Hkv, int N, int D,
                     int block, float scale, int accumulate, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * sas_workspace_bytes -- device workspace a call with these sizes needs
 *   (0 if none).  `n_or_lmax` is N for training calls and L_max for decode;
 *   `topk` < 0 means full scope / dense decode.  Returns (size_t)-1 for
 *   invalid sizes.
 */
size_t sas_workspace_bytes(int op, int B, int Hq, int Hkv, int n_or_lmax, int D,
                           int block, int topk, int dtype);

/*
 * Kernel timing (diagnostics; not part of the method).
 * sas_profile_enable(1) makes every later kernel launch record a HIP event on
 *   its stream just before and just after the kernel; (0) stops recording.
 *   Events are host-side objects: no device memory is allocated.
 * sas_profile_read waits for every recorded launch, sums the durations per
 *   kernel name, writes up to max_entries of them (name as a NUL-terminated
 *   string in a slot of name_bytes bytes of `names`, total milliseconds in
 *   ms[i], launches in counts[i]), clears the record and returns the number of
 *   distinct kernels (which may exceed max_entries).  SAS_EINVAL for bad
 *   arguments, SAS_EHIP if an event could not be read.
 */
int sas_profile_enable(int on);
int sas_profile_read(int max_entries, char* names, int name_bytes, double* ms,
                     int* counts);

/* Message for the last non-OK status returned on this thread. */
const char* sas_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int sas_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAS_H_ */
