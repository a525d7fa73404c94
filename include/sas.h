/*
 * sas.h -- C ABI of libsas: SAS (Simple Attention Sparsification) gated
 * block-sparse attention on AMD MI355X (gfx950).
 *
 * The method (sources named by page title and section):
 *   - "SAS close reading" = liuzhao09.github.io, SAS：用最终预测损失学习有限注意力预算下的上下文排序
 *   - "SAS reproduction note" = daiwk.github.io, SAS：用语言模型损失端到端学习稀疏注意力排序
 *   - "SAS summary" = hyper.ai summary of paper 2609.13141, section 方法 (Method)
 *   - "MSA notes" = papercache.org notes on MiniMax Sparse Attention
 *
 * A query at position T-1 attends to the current block B0 (always kept,
 * causal, unit gate) plus the Top-K of the C = (T-1)/64 complete history
 * blocks ranked by a selector score s; the selected blocks' logits get the
 * bias log g_m = s_m - LSE(s) (softmax gate over all C history blocks):
 *     o = softmax(q K_S^T * scale + log g_S) V_S
 * (SAS close reading 2.1 and 2.2; SAS reproduction note, core formula).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer to contiguous row-major memory,
 *    head-major:  q [B,Hq,d] (decode) or Q/O/dO/dQ [B,Hq,S,d] (prefill);
 *    K/V/dK/dV [B,Hkv,t_max,d];  summ [B,Hkv,t_max/64,d_sel] fp32;
 *    Wq_sel/Wk_sel [d_sel,d] fp32, shared by all groups;
 *    idx (int32), log_gate / dlog_gate (fp32) [B,Hkv,rows,k];
 *    score_lse fp32 [B,Hkv,rows]; lse fp32 [B,Hq] (decode) or [B,Hq,S].
 *    rows = 1 for decode, ceil(S/64) for prefill tiles (tile t covers queries
 *    [64t, 64t+64) and its history is blocks [0, t)).
 *  - Query head h belongs to group h / G, G = Hq/Hkv (adjacent heads share a
 *    KV head; MSA notes 2.1).
 *  - idx lists the chosen history blocks in ascending order, padded with -1;
 *    log_gate holds log g of each chosen block, padded with -inf.
 *  - Q/K/V/O/dQ/dK/dV use sas_dims.dtype; everything else is fp32/int32.
 *  - Ownership: the caller allocates and owns every buffer, including the
 *    workspace sized by sas_workspace_bytes().  The library allocates and
 *    frees nothing and keeps no pointer after a call returns.
 *  - A workspace holds intermediate results of one call only (no state is
 *    carried between calls; its initial contents do not matter).  Calls that
 *    share one workspace must not run concurrently.
 *  - Execution: each call validates its arguments on the host, then enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *    The caller synchronises.  Results are bitwise deterministic.
 *  - Errors: a call that returns SAS_ERR_INVALID_ARGUMENT, SAS_ERR_UNSUPPORTED
 *    or SAS_ERR_WORKSPACE_TOO_SMALL has enqueued nothing and left every
 *    output untouched.  SAS_ERR_HIP means a launch failed after validation;
 *    sas_last_error() has the text.
 *  - Device-side contents are trusted: seq_lens must lie in [1, t_max] (the
 *    kernels clamp them into that range); idx entries must be -1 or a valid
 *    history block of their row.  Inputs must be finite.
 *  - The library keeps no global mutable state apart from a thread-local
 *    error string.
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
  SAS_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, Hq % Hkv != 0, seq_len > t_max, ... */
  SAS_ERR_UNSUPPORTED = 2,        /* valid but not built: block != 64, d or d_sel not 64/128, ... */
  SAS_ERR_WORKSPACE_TOO_SMALL = 3,
  SAS_ERR_HIP = 4                 /* a HIP runtime/launch error; see sas_last_error() */
} sas_status;

typedef enum { SAS_F32 = 0, SAS_BF16 = 1 } sas_dtype;

typedef enum { SAS_SELECT_DECODE = 0, SAS_SELECT_TILES = 1, SAS_SELECT_QUERIES = 2 } sas_select_mode;

typedef enum {
  SAS_OP_SELECT_DECODE = 0,
  SAS_OP_SELECT_TILES = 1,
  SAS_OP_DECODE_FWD = 2,
  SAS_OP_PREFILL_FWD = 3,
  SAS_OP_BWD = 4,
  SAS_OP_DECODE_STEP = 5,
  SAS_OP_SELECTOR_BWD = 6,
  SAS_OP_SELECT_QUERIES = 7,
  SAS_OP_PREFILL_FWD_QUERIES = 8,
  SAS_OP_BWD_QUERIES = 9,
  SAS_OP_SELECTOR_BWD_QUERIES = 10
} sas_op;

/* Problem sizes.  Supported: block_size 64; head_dim and sel_dim 64 or 128;
 * G = n_q_heads/n_kv_heads in {1,2,4,8}; 0 <= top_k <= 64; t_max >= 1. */
typedef struct {
  int32_t batch;        /* B */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv */
  int32_t head_dim;     /* d */
  int32_t sel_dim;      /* d_sel */
  int32_t block_size;   /* b (64) */
  int32_t top_k;        /* k: history blocks kept per row */
  int32_t t_max;        /* row capacity of K/V (and of summ: t_max/64 blocks) */
  int32_t dtype;        /* sas_dtype of Q/K/V/O and their gradients */
} sas_dims;

/* Block summaries (SAS close reading 2.1, block summary; mean pooling):
 *     summ[b,r,m,:] = Wk_sel . mean_{j in block m} K[b,r,j,:]
 * for every complete history block m < C_b = (seq_lens[b]-1)/64 with
 * blk_begin <= m < blk_end (fp32 accumulation).  Other rows of summ are not
 * written, so a decode loop can refresh just the block that completed.
 * In prefill pass seq_lens[b] = S: tile t needs blocks [0, t).
 * K: dtype [B,Hkv,t_max,d]; seq_lens: int32 [B]; Wk_sel: fp32 [d_sel,d];
 * summ: fp32 [B,Hkv,t_max/64,d_sel].  0 <= blk_begin <= blk_end required. */
sas_status sas_block_summaries(const sas_dims* dims, const void* K, const int32_t* seq_lens,
                               const float* Wk_sel, int32_t blk_begin, int32_t blk_end,
                               float* summ, void* stream);

/* Selector score, gate and Top-K (SAS close reading 2.1 and 2.2; SAS summary,
 * Method).  Per group r and row:
 *     s_m  = mean_{h in r, queries of the row} (Wq_sel q) . summ_m / sqrt(d_sel)
 *     score_lse = LSE(s) over all history blocks of the row (-inf if none),
 *     idx  = the min(k, C) largest s (ties -> lower m), ascending,
 *     log_gate = s_idx - score_lse.
 * Top-K runs on the fp32 scores themselves (MSA notes 4.1); -0 equals +0.
 * mode SAS_SELECT_DECODE: Q is q [B,Hq,d], one row per (b,r), C = (seq_lens[b]-1)/64;
 *   q_len is ignored.
 * mode SAS_SELECT_TILES:  Q is [B,Hq,q_len,d], rows = ceil(q_len/64), row t has
 *   C = t history blocks and averages over its min(64, q_len-64t) queries;
 *   seq_lens may be NULL; q_len <= t_max and rows <= 1024.
 * mode SAS_SELECT_QUERIES: Q is [B,Hq,q_len,d], rows = q_len, one row per
 *   query (SAS close reading 2.4: the training kernel masks each query by its
 *   own gate threshold); row i has C = i/64 history blocks (those before the
 *   query's own block) and averages over the G heads of query i only, i.e.
 *   the decode selection of a query at position i; seq_lens may be NULL;
 *   q_len <= t_max and ceil(q_len/64) <= 1024.
 * scores (nullable): fp32 [B,Hkv,rows,t_max/64]; entry m < C of a row gets s_m.
 * summ must hold the summaries of every block the rows read.
 * ws: at least sas_workspace_bytes(SAS_OP_SELECT_DECODE, _TILES or _QUERIES,
 * dims, q_len). */
sas_status sas_select(const sas_dims* dims, int32_t mode, const void* Q, int32_t q_len,
                      const int32_t* seq_lens, const float* Wq_sel, const float* summ,
                      int32_t* idx, float* log_gate, float* score_lse, float* scores,
                      void* ws, size_t ws_bytes, void* stream);

/* One decode step of gated sparse attention (SAS reproduction note, core
 * formula; SAS summary, Method, fused kernel): for every query head h of group r
 *     z_j = q_h . k_j * scale + beta_j  over  j in B0 = [64C, T)  and the
 *     blocks idx[b,r,0,:],  beta = log_gate on history, 0 on B0;
 *     o = softmax(z) V,  lse = log-sum-exp of z.
 * log_gate == NULL gives the ungated inference rule (beta = 0 everywhere;
 * SAS close reading 2.1/2.3).  Streams only the selected 64-token blocks and
 * B0 (split-KV), then merges the partial softmax states.
 * q, o: dtype [B,Hq,d]; K, V: dtype [B,Hkv,t_max,d]; seq_lens int32 [B] (T per
 * sequence, including the current token, whose K/V must already be stored);
 * idx/log_gate [B,Hkv,1,k]; lse (nullable) fp32 [B,Hq].
 * ws: at least sas_workspace_bytes(SAS_OP_DECODE_FWD, dims, 0). */
sas_status sas_decode_fwd(const sas_dims* dims, const void* q, const void* K, const void* V,
                          const int32_t* seq_lens, const int32_t* idx, const float* log_gate,
                          float scale, void* o, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

/* One whole decode step of the selection and the attention, fused (SAS
 * close reading 2.1-2.2; SAS summary, Method, fused kernel): the same outputs,
 * bit for bit, as sas_select(SAS_SELECT_DECODE, ...) followed by
 * sas_decode_fwd(..., gated ? log_gate : NULL, ...) on its selection, in
 * fewer launches: the merge of the selection's per-chunk candidates runs
 * inside the attention's split kernel instead of a kernel of its own, and
 * the split workgroup of each (sequence, group) that finishes last merges
 * the attention partials (counted with one integer atomic per row in ws,
 * which the step zeroes itself: ws needs no initial content, but two calls
 * in flight on one ws race).
 * Wk_sel (nullable) fp32 [d_sel,d]: when given, the step first refreshes the
 * summary of each sequence's newest complete history block m = C-1 (C =
 * (seq_lens[b]-1)/64 >= 1), exactly as sas_block_summaries(..., C-1, C, ...)
 * would (same bits), writes it into summ and scores with it: the same
 * outputs, summ included, as that call followed by the two above.  summ is
 * then read and written; with Wk_sel NULL it is only read.
 * Arguments as in those calls; idx/log_gate [B,Hkv,1,k] and score_lse
 * [B,Hkv,1] are outputs here; gated = 0 gives the ungated inference rule for
 * the attention (log_gate is still written).
 * ws: at least sas_workspace_bytes(SAS_OP_DECODE_STEP, dims, 0). */
sas_status sas_decode_step(const sas_dims* dims, const void* q, const void* K, const void* V,
                           const int32_t* seq_lens, const float* Wq_sel, const float* Wk_sel,
                           float* summ,
                           int32_t gated, float scale, int32_t* idx, float* log_gate,
                           float* score_lse, void* o, float* lse, void* ws, size_t ws_bytes,
                           void* stream);

/* Paged K/V cache (SAS close reading 2.4, closing paragraph on serving: the
 * served system keeps K/V in a paged cache).  A page is one 64-token block of
 * every KV head of one sequence: K_pages/V_pages dtype [n_pages,Hkv,64,d].
 * page_table int32 [B,max_pages]: logical block m of sequence b (tokens
 * 64m..64m+63) is page page_table[b*max_pages+m]; entries m <= C_b =
 * (seq_lens[b]-1)/64 must name valid pages (the caller owns the pool and the
 * table; pages may be shared between sequences).  dims->t_max is the logical
 * capacity per sequence, at most 64*max_pages.  Summaries stay logical, fp32
 * [B,Hkv,t_max/64,d_sel] as for a contiguous cache, so the selection reads
 * them without a table lookup.
 *
 * sas_block_summaries_paged: sas_block_summaries on a paged cache (same
 * block range rules, same bits for the same block contents). */
sas_status sas_block_summaries_paged(const sas_dims* dims, const void* K_pages,
                                     const int32_t* page_table, int32_t max_pages,
                                     const int32_t* seq_lens, const float* Wk_sel,
                                     int32_t blk_begin, int32_t blk_end, float* summ,
                                     void* stream);

/* sas_decode_step on a paged cache: the same computation and outputs, bit
 * for bit, as sas_decode_step on the contiguous cache holding the same
 * blocks (idx holds logical block numbers; with Wk_sel the newest complete
 * block's summary is refreshed into summ first).  Invalid sizes or NULL
 * required pointers return an error and enqueue nothing.
 * ws: at least sas_workspace_bytes(SAS_OP_DECODE_STEP, dims, 0). */
sas_status sas_decode_step_paged(const sas_dims* dims, const void* q, const void* K_pages,
                                 const void* V_pages, const int32_t* page_table,
                                 int32_t max_pages, const int32_t* seq_lens,
                                 const float* Wq_sel, const float* Wk_sel, float* summ,
                                 int32_t gated, float scale, int32_t* idx, float* log_gate,
                                 float* score_lse, void* o, float* lse, void* ws,
                                 size_t ws_bytes, void* stream);

/* Causal prefill / training forward with one selection per 64-query tile
 * (SAS summary, Method, fused kernel; SAS close reading 2.4): query i of tile
 * t attends to the selected blocks of (b, r, t) with bias log_gate and to
 * tokens 64t..i of its own block with bias 0.  bf16 only, fp32 softmax and
 * accumulation on matrix cores.
 * Q, O: bf16 [B,Hq,seq_len,d]; K, V: bf16 [B,Hkv,t_max,d] (seq_len <= t_max);
 * idx/log_gate [B,Hkv,ceil(seq_len/64),k] (log_gate NULL = ungated);
 * lse: fp32 [B,Hq,seq_len] (natural log), needed by sas_bwd.
 * ws: at least sas_workspace_bytes(SAS_OP_PREFILL_FWD, dims, seq_len). */
sas_status sas_prefill_fwd(const sas_dims* dims, const void* Q, const void* K, const void* V,
                           int32_t seq_len, const int32_t* idx, const float* log_gate,
                           float scale, void* O, float* lse, void* ws, size_t ws_bytes,
                           void* stream);

/* Causal prefill / training forward with one selection per query (SAS close
 * reading 2.4: the fused kernel adds log g to the selected blocks' logits
 * and masks the others by each query's own gate threshold, skipping blocks
 * that no query of a tile selected): query i attends to the blocks
 * idx[b,r,i,:] with bias log_gate and to tokens 64*(i/64)..i of its own block
 * with bias 0, i.e. a decode step at T = i+1.  bf16 only.
 * Q, O: bf16 [B,Hq,seq_len,d]; K, V: bf16 [B,Hkv,t_max,d] (seq_len <= t_max);
 * idx/log_gate [B,Hkv,seq_len,k] as written by sas_select(SAS_SELECT_QUERIES)
 * (ascending, -1 padded, every entry < i/64; log_gate NULL = ungated);
 * lse: fp32 [B,Hq,seq_len] (natural log); ceil(seq_len/64) <= 1024.
 * ws: at least sas_workspace_bytes(SAS_OP_PREFILL_FWD_QUERIES, dims, seq_len)
 * (0 today).  Errors as sas_prefill_fwd. */
sas_status sas_prefill_fwd_queries(const sas_dims* dims, const void* Q, const void* K,
                                   const void* V, int32_t seq_len, const int32_t* idx,
                                   const float* log_gate, float scale, void* O, float* lse,
                                   void* ws, size_t ws_bytes, void* stream);

/* Backward of sas_prefill_fwd for L with upstream gradient dO (SAS close
 * reading 2.4 and 2.2 eq. 5; SAS summary, Method): recompute P from lse;
 * D = rowsum(dO*O); dS = P*(dO V^T - D); dQ = scale dS K; dK = scale dS^T Q;
 * dV = P^T dO; and
 *     dlog_gate[b,r,t,slot] = sum over heads of r, queries of t and tokens
 *                             of block idx[b,r,t,slot] of dS.
 * B0 carries no gate; empty slots get 0.  The log-gate is an independent
 * input (the chain into the selector is not part of this call).
 * Q, O, dO, dQ: bf16 [B,Hq,seq_len,d]; K, V, dK, dV: bf16 [B,Hkv,t_max,d]
 * (rows >= seq_len of dK/dV are not written); lse fp32 [B,Hq,seq_len];
 * idx/log_gate/dlog_gate [B,Hkv,ceil(seq_len/64),k].
 * ws: at least sas_workspace_bytes(SAS_OP_BWD, dims, seq_len). */
sas_status sas_bwd(const sas_dims* dims, const void* Q, const void* K, const void* V,
                   const void* O, const void* dO, const float* lse, int32_t seq_len,
                   const int32_t* idx, const float* log_gate, float scale, void* dQ, void* dK,
                   void* dV, float* dlog_gate, void* ws, size_t ws_bytes, void* stream);

/* Backward of sas_prefill_fwd_queries (one selection per query; SAS close
 * reading 2.4 and 2.2 eq. 5): as sas_bwd with each query's own token set,
 * and one log-gate gradient per query and slot:
 *     dlog_gate[b,r,i,slot] = sum over the heads of r and the tokens of block
 *                             idx[b,r,i,slot] of dS of query i.
 * Empty slots get 0.  Q, O, dO, dQ: bf16 [B,Hq,seq_len,d]; K, V, dK, dV: bf16
 * [B,Hkv,t_max,d] (rows >= seq_len of dK/dV are not written); lse fp32
 * [B,Hq,seq_len]; idx/log_gate/dlog_gate [B,Hkv,seq_len,k] (idx as for
 * sas_prefill_fwd_queries); ceil(seq_len/64) <= 1024.
 * ws: at least sas_workspace_bytes(SAS_OP_BWD_QUERIES, dims, seq_len): that of
 * sas_bwd plus per-head log-gate partials (B*Hq*seq_len*k floats) and per-tile
 * union bitmaps and gate rows (B*Hkv*(1 + n(n-1)/2)*64 floats, n the number
 * of 64-query tiles).  Errors as sas_bwd. */
sas_status sas_bwd_queries(const sas_dims* dims, const void* Q, const void* K, const void* V,
                           const void* O, const void* dO, const float* lse, int32_t seq_len,
                           const int32_t* idx, const float* log_gate, float scale, void* dQ,
                           void* dK, void* dV, float* dlog_gate, void* ws, size_t ws_bytes,
                           void* stream);

/* Backward of the selector into its weights, for the tile rows of a prefill
 * (SAS close reading 2.2, gate equation; 2.3, eq. 8, sparse scope; 2.4 and
 * the training description after it).  With the selection held fixed and
 * dlog_gate of the selected slots (from sas_bwd), for each row t of group r
 * and each of its C = t history blocks m:
 *     ds_m = dlog_gate[slot of m] [m selected] - g_m * sum_slots dlog_gate,
 *     g_m  = exp(s_m - score_lse),
 * and through s_m = (Wq_sel qbar) . summ_m / sqrt(d_sel), summ_m = Wk_sel kbar_m
 * (qbar: mean of the tile's queries over the group's heads; kbar_m: mean key
 * of block m):
 *     dWq_sel = sum over rows and m of ds_m summ_m qbar^T / sqrt(d_sel),
 *     dWk_sel = sum over rows and m of ds_m (Wq_sel qbar / sqrt(d_sel)) kbar_m^T.
 * The chain into Q and K through the selector is not formed (the backbone is
 * held fixed while the selector trains).
 * Q: dtype [B,Hq,q_len,d]; K: dtype [B,Hkv,t_max,d]; Wq_sel fp32 [d_sel,d];
 * summ fp32 [B,Hkv,t_max/64,d_sel] (sas_block_summaries of K); idx/dlog_gate
 * [B,Hkv,rows,k] and score_lse [B,Hkv,rows] (sas_select in SAS_SELECT_TILES
 * mode, then sas_bwd); rows = ceil(q_len/64) <= 1024, q_len <= t_max.
 * ds (nullable) fp32 [B,Hkv,rows,t_max/64]: entries m < t of row t are written.
 * dWq_sel, dWk_sel fp32 [d_sel,d] are overwritten (summed over the batch).
 * Results are bitwise reproducible (no atomics).
 * ws: at least sas_workspace_bytes(SAS_OP_SELECTOR_BWD, dims, q_len). */
sas_status sas_selector_bwd(const sas_dims* dims, const void* Q, int32_t q_len, const void* K,
                            const float* Wq_sel, const float* summ, const int32_t* idx,
                            const float* score_lse, const float* dlog_gate, float* ds,
                            float* dWq_sel, float* dWk_sel, void* ws, size_t ws_bytes,
                            void* stream);

/* The selector backward for per-query rows (one selection per query, as
 * written by sas_select(SAS_SELECT_QUERIES) and differentiated by
 * sas_bwd_queries; SAS close reading 2.2-2.4): row (b, r, i) has the C = i/64
 * blocks before query i's block and the pooled query qbar_i (mean of query i
 * over the group's heads); ds over those blocks as for sas_selector_bwd, and
 *     dWq_sel = sum_rows sum_m ds_m summ_m qbar_i^T / sqrt(d_sel),
 *     dWk_sel = sum_rows sum_m ds_m (Wq_sel qbar_i / sqrt(d_sel)) kbar_m^T,
 * computed through H = sum_rows (sum_m ds_m kbar_m) qbar_i^T as
 * Wk_sel H / sqrt(d_sel) and Wq_sel H^T / sqrt(d_sel) (hence Wk_sel).
 * Q: [B,Hq,q_len,d]; K: [B,Hkv,t_max,d]; Wq_sel, Wk_sel: fp32 [d_sel,d];
 * summ as read by the selection; idx/dlog_gate [B,Hkv,q_len,k]; score_lse
 * [B,Hkv,q_len]; ds (nullable) fp32 [B,Hkv,q_len,t_max/64] (entry m < C of a
 * row); dWq_sel, dWk_sel fp32 [d_sel,d], overwritten.  q_len <= t_max and
 * ceil(q_len/64) <= 1024.  Bitwise reproducible (no atomics).
 * ws: at least sas_workspace_bytes(SAS_OP_SELECTOR_BWD_QUERIES, dims, q_len). */
sas_status sas_selector_bwd_queries(const sas_dims* dims, const void* Q, int32_t q_len,
                                    const void* K, const float* Wq_sel, const float* Wk_sel,
                                    const float* summ, const int32_t* idx,
                                    const float* score_lse, const float* dlog_gate, float* ds,
                                    float* dWq_sel, float* dWk_sel, void* ws, size_t ws_bytes,
                                    void* stream);

/* Workspace bytes an op needs for these sizes (q_len: prefill/tiles length,
 * ignored otherwise).  Returns SIZE_MAX if the sizes are invalid or
 * unsupported. */
size_t sas_workspace_bytes(int32_t op, const sas_dims* dims, int32_t q_len);

/* Static text of a status code. */
const char* sas_status_str(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* sas_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SAS_H_ */
