// C entry points of libsas: argument validation, workspace sizing, dispatch.
// All checks run on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>

#include "sas_internal.h"

namespace sas {

static thread_local char g_last_error[512] = "";

sas_status fail(sas_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

sas_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SAS_OK;
}

// Shared size checks.  `need_bf16`: prefill/backward are built for bf16 only.
static sas_status check_dims(const sas_dims* d, bool need_bf16) {
  if (!d) return fail(SAS_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->sel_dim < 1 || d->block_size < 1 || d->t_max < 1)
    return fail(SAS_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d Hq=%d Hkv=%d d=%d "
                "d_sel=%d b=%d t_max=%d)", d->batch, d->n_q_heads, d->n_kv_heads, d->head_dim,
                d->sel_dim, d->block_size, d->t_max);
  if (d->top_k < 0) return fail(SAS_ERR_INVALID_ARGUMENT, "top_k=%d is negative", d->top_k);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(SAS_ERR_INVALID_ARGUMENT, "n_q_heads=%d is not a multiple of n_kv_heads=%d",
                d->n_q_heads, d->n_kv_heads);
  if (d->dtype != SAS_F32 && d->dtype != SAS_BF16)
    return fail(SAS_ERR_INVALID_ARGUMENT, "dtype=%d is not a sas_dtype", d->dtype);
  if (d->block_size != kBlock)
    return fail(SAS_ERR_UNSUPPORTED, "block_size=%d (only 64 is built)", d->block_size);
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SAS_ERR_UNSUPPORTED, "group size %d (built: 1, 2, 4, 8)", G);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SAS_ERR_UNSUPPORTED, "head_dim=%d (built: 64, 128)", d->head_dim);
  if (d->sel_dim != 64 && d->sel_dim != 128)
    return fail(SAS_ERR_UNSUPPORTED, "sel_dim=%d (built: 64, 128)", d->sel_dim);
  if (d->top_k > kMaxTopK)
    return fail(SAS_ERR_UNSUPPORTED, "top_k=%d (built up to %d)", d->top_k, kMaxTopK);
  if (need_bf16 && d->dtype != SAS_BF16)
    return fail(SAS_ERR_UNSUPPORTED, "prefill and backward are built for bf16 only");
  // Every index computed in the kernels stays inside int64; element counts of
  // one tensor must fit in 2^31 rows of 64-bit addressing, checked loosely here.
  const long long kv_elems = 1LL * d->batch * d->n_kv_heads * d->t_max * d->head_dim;
  if (kv_elems <= 0 || kv_elems > (1LL << 40))
    return fail(SAS_ERR_INVALID_ARGUMENT, "K/V size out of range");
  return SAS_OK;
}

static sas_status check_len(const sas_dims* d, int32_t len, const char* name) {
  if (len < 1) return fail(SAS_ERR_INVALID_ARGUMENT, "%s=%d must be >= 1", name, len);
  if (len > d->t_max)
    return fail(SAS_ERR_INVALID_ARGUMENT, "%s=%d exceeds t_max=%d", name, len, d->t_max);
  return SAS_OK;
}

#define SAS_TRY(x)                 \
  do {                             \
    sas_status st__ = (x);         \
    if (st__ != SAS_OK) return st__; \
  } while (0)

#define SAS_NONNULL(p)                                                        \
  do {                                                                        \
    if (!(p)) return fail(SAS_ERR_INVALID_ARGUMENT, "%s is NULL", #p);        \
  } while (0)

static sas_status check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return SAS_OK;
  if (!ws || ws_bytes < need)
    return fail(SAS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu%s", need,
                ws_bytes, ws ? "" : " (NULL)");
  return SAS_OK;
}

}  // namespace sas

using namespace sas;

extern "C" {

sas_status sas_block_summaries(const sas_dims* dims, const void* K, const int32_t* seq_lens,
                               const float* Wk_sel, int32_t blk_begin, int32_t blk_end,
                               float* summ, void* stream) {
  SAS_TRY(check_dims(dims, false));
  if (blk_begin < 0 || blk_end < blk_begin)
    return fail(SAS_ERR_INVALID_ARGUMENT, "block range [%d, %d) is invalid", blk_begin, blk_end);
  const int c_max = dims->t_max / kBlock;
  if (blk_end > c_max) blk_end = c_max;
  if (blk_begin >= blk_end) return SAS_OK;  // nothing to do (summ may then be empty/NULL)
  SAS_NONNULL(K);
  SAS_NONNULL(seq_lens);
  SAS_NONNULL(Wk_sel);
  SAS_NONNULL(summ);
  return launch_block_summaries(*dims, K, seq_lens, Wk_sel, blk_begin, blk_end, summ,
                                static_cast<hipStream_t>(stream));
}

sas_status sas_select(const sas_dims* dims, int32_t mode, const void* Q, int32_t q_len,
                      const int32_t* seq_lens, const float* Wq_sel, const float* summ,
                      int32_t* idx, float* log_gate, float* score_lse, float* scores,
                      void* ws, size_t ws_bytes, void* stream) {
  SAS_TRY(check_dims(dims, false));
  SAS_NONNULL(Q);
  SAS_NONNULL(Wq_sel);
  if (dims->t_max >= kBlock) SAS_NONNULL(summ);  // no history block fits otherwise
  if (dims->top_k > 0) {
    SAS_NONNULL(idx);
    SAS_NONNULL(log_gate);
  }
  SAS_NONNULL(score_lse);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == SAS_SELECT_DECODE) {
    SAS_NONNULL(seq_lens);
    SAS_TRY(check_ws(select_decode_ws_bytes(*dims), ws, ws_bytes));
    return launch_select_decode(*dims, Q, seq_lens, Wq_sel, summ, idx, log_gate, score_lse,
                                scores, ws, st);
  }
  if (mode == SAS_SELECT_TILES) {
    SAS_TRY(check_len(dims, q_len, "q_len"));
    if (cdiv(q_len, kBlock) > kMaxTileRows)
      return fail(SAS_ERR_UNSUPPORTED, "q_len=%d gives more than %d tiles", q_len,
                  kMaxTileRows);
    return launch_select_tiles(*dims, Q, q_len, Wq_sel, summ, idx, log_gate, score_lse,
                               scores, st);
  }
  if (mode == SAS_SELECT_QUERIES) {
    SAS_TRY(check_len(dims, q_len, "q_len"));
    if (cdiv(q_len, kBlock) > kMaxTileRows)
      return fail(SAS_ERR_UNSUPPORTED, "q_len=%d gives more than %d tiles", q_len,
                  kMaxTileRows);
    return launch_select_queries(*dims, Q, q_len, Wq_sel, summ, idx, log_gate, score_lse,
                                 scores, st);
  }
  return fail(SAS_ERR_INVALID_ARGUMENT, "mode=%d is not a sas_select_mode", mode);
}

sas_status sas_decode_fwd(const sas_dims* dims, const void* q, const void* K, const void* V,
                          const int32_t* seq_lens, const int32_t* idx, const float* log_gate,
                          float scale, void* o, float* lse, void* ws, size_t ws_bytes,
                          void* stream) {
  SAS_TRY(check_dims(dims, false));
  SAS_NONNULL(q);
  SAS_NONNULL(K);
  SAS_NONNULL(V);
  SAS_NONNULL(seq_lens);
  SAS_NONNULL(o);
  if (dims->top_k > 0) SAS_NONNULL(idx);
  if (!(scale > 0.0f))
    return fail(SAS_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  SAS_TRY(check_ws(decode_ws_bytes(*dims), ws, ws_bytes));
  return launch_decode_fwd(*dims, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws,
                           static_cast<hipStream_t>(stream));
}

sas_status sas_decode_step(const sas_dims* dims, const void* q, const void* K, const void* V,
                           const int32_t* seq_lens, const float* Wq_sel, const float* Wk_sel,
                           float* summ,
                           int32_t gated, float scale, int32_t* idx, float* log_gate,
                           float* score_lse, void* o, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  SAS_TRY(check_dims(dims, false));
  SAS_NONNULL(q);
  SAS_NONNULL(K);
  SAS_NONNULL(V);
  SAS_NONNULL(seq_lens);
  SAS_NONNULL(Wq_sel);
  if (dims->t_max >= kBlock) SAS_NONNULL(summ);
  if (dims->top_k > 0) {
    SAS_NONNULL(idx);
    SAS_NONNULL(log_gate);
  }
  SAS_NONNULL(score_lse);
  SAS_NONNULL(o);
  if (!(scale > 0.0f))
    return fail(SAS_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  SAS_TRY(check_ws(decode_step_ws_bytes(*dims), ws, ws_bytes));
  return launch_decode_step(*dims, q, K, V, seq_lens, Wq_sel, summ, Wk_sel, KvPages{nullptr, 0},
                            gated != 0, scale, idx,
                            log_gate, score_lse, o, lse, ws, static_cast<hipStream_t>(stream));
}

sas_status sas_block_summaries_paged(const sas_dims* dims, const void* K_pages,
                                     const int32_t* page_table, int32_t max_pages,
                                     const int32_t* seq_lens, const float* Wk_sel,
                                     int32_t blk_begin, int32_t blk_end, float* summ,
                                     void* stream) {
  SAS_TRY(check_dims(dims, false));
  if (max_pages < 1 || static_cast<long>(dims->t_max) > static_cast<long>(max_pages) * kBlock)
    return fail(SAS_ERR_INVALID_ARGUMENT, "t_max=%d needs at least %d page-table entries per "
                "sequence, got %d", dims->t_max, cdiv(dims->t_max, kBlock), max_pages);
  if (blk_begin < 0 || blk_end < blk_begin)
    return fail(SAS_ERR_INVALID_ARGUMENT, "block range [%d, %d) is invalid", blk_begin, blk_end);
  const int c_max = dims->t_max / kBlock;
  if (blk_end > c_max) blk_end = c_max;
  if (blk_begin >= blk_end) return SAS_OK;
  SAS_NONNULL(K_pages);
  SAS_NONNULL(page_table);
  SAS_NONNULL(seq_lens);
  SAS_NONNULL(Wk_sel);
  SAS_NONNULL(summ);
  return launch_block_summaries_paged(*dims, K_pages, KvPages{page_table, max_pages}, seq_lens,
                                      Wk_sel, blk_begin, blk_end, summ,
                                      static_cast<hipStream_t>(stream));
}

sas_status sas_decode_step_paged(const sas_dims* dims, const void* q, const void* K_pages,
                                 const void* V_pages, const int32_t* page_table,
                                 int32_t max_pages, const int32_t* seq_lens,
                                 const float* Wq_sel, const float* Wk_sel, float* summ,
                                 int32_t gated, float scale, int32_t* idx, float* log_gate,
                                 float* score_lse, void* o, float* lse, void* ws,
                                 size_t ws_bytes, void* stream) {
  SAS_TRY(check_dims(dims, false));
  if (max_pages < 1 || static_cast<long>(dims->t_max) > static_cast<long>(max_pages) * kBlock)
    return fail(SAS_ERR_INVALID_ARGUMENT, "t_max=%d needs at least %d page-table entries per "
                "sequence, got %d", dims->t_max, cdiv(dims->t_max, kBlock), max_pages);
  SAS_NONNULL(q);
  SAS_NONNULL(K_pages);
  SAS_NONNULL(V_pages);
  SAS_NONNULL(page_table);
  SAS_NONNULL(seq_lens);
  SAS_NONNULL(Wq_sel);
  if (dims->t_max >= kBlock) SAS_NONNULL(summ);
  if (dims->top_k > 0) {
    SAS_NONNULL(idx);
    SAS_NONNULL(log_gate);
  }
  SAS_NONNULL(score_lse);
  SAS_NONNULL(o);
  if (!(scale > 0.0f))
    return fail(SAS_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  SAS_TRY(check_ws(decode_step_ws_bytes(*dims), ws, ws_bytes));
  return launch_decode_step(*dims, q, K_pages, V_pages, seq_lens, Wq_sel, summ, Wk_sel,
                            KvPages{page_table, max_pages}, gated != 0, scale, idx, log_gate,
                            score_lse, o, lse, ws, static_cast<hipStream_t>(stream));
}

sas_status sas_prefill_fwd(const sas_dims* dims, const void* Q, const void* K, const void* V,
                           int32_t seq_len, const int32_t* idx, const float* log_gate,
                           float scale, void* O, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  SAS_TRY(check_dims(dims, true));
  SAS_TRY(check_len(dims, seq_len, "seq_len"));
  SAS_NONNULL(Q);
  SAS_NONNULL(K);
  SAS_NONNULL(V);
  SAS_NONNULL(O);
  SAS_NONNULL(lse);
  if (dims->top_k > 0) SAS_NONNULL(idx);
  if (!(scale > 0.0f)) return fail(SAS_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  SAS_TRY(check_ws(prefill_ws_bytes(*dims, seq_len), ws, ws_bytes));
  return launch_prefill_fwd(*dims, Q, K, V, seq_len, idx, log_gate, scale, O, lse, ws,
                            static_cast<hipStream_t>(stream));
}

sas_status sas_prefill_fwd_queries(const sas_dims* dims, const void* Q, const void* K,
                                   const void* V, int32_t seq_len, const int32_t* idx,
                                   const float* log_gate, float scale, void* O, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;   // no workspace
  SAS_TRY(check_dims(dims, true));
  SAS_TRY(check_len(dims, seq_len, "seq_len"));
  SAS_NONNULL(Q);
  SAS_NONNULL(K);
  SAS_NONNULL(V);
  SAS_NONNULL(O);
  SAS_NONNULL(lse);
  if (dims->top_k > 0) SAS_NONNULL(idx);
  if (!(scale > 0.0f)) return fail(SAS_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  if (cdiv(seq_len, kBlock) > kMaxTileRows)
    return fail(SAS_ERR_UNSUPPORTED, "seq_len=%d gives more than %d tiles", seq_len,
                kMaxTileRows);
  return launch_prefill_fwd_queries(*dims, Q, K, V, seq_len, idx, log_gate, scale, O, lse,
                                    static_cast<hipStream_t>(stream));
}

sas_status sas_bwd(const sas_dims* dims, const void* Q, const void* K, const void* V,
                   const void* O, const void* dO, const float* lse, int32_t seq_len,
                   const int32_t* idx, const float* log_gate, float scale, void* dQ, void* dK,
                   void* dV, float* dlog_gate, void* ws, size_t ws_bytes, void* stream) {
  SAS_TRY(check_dims(dims, true));
  SAS_TRY(check_len(dims, seq_len, "seq_len"));
  SAS_NONNULL(Q);
  SAS_NONNULL(K);
  SAS_NONNULL(V);
  SAS_NONNULL(O);
  SAS_NONNULL(dO);
  SAS_NONNULL(lse);
  SAS_NONNULL(dQ);
  SAS_NONNULL(dK);
  SAS_NONNULL(dV);
  if (dims->top_k > 0) {
    SAS_NONNULL(idx);
    SAS_NONNULL(dlog_gate);
  }
  if (!(scale > 0.0f)) return fail(SAS_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  SAS_TRY(check_ws(bwd_ws_bytes(*dims, seq_len), ws, ws_bytes));
  return launch_bwd(*dims, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK, dV,
                    dlog_gate, ws, static_cast<hipStream_t>(stream));
}

sas_status sas_bwd_queries(const sas_dims* dims, const void* Q, const void* K, const void* V,
                           const void* O, const void* dO, const float* lse, int32_t seq_len,
                           const int32_t* idx, const float* log_gate, float scale, void* dQ,
                           void* dK, void* dV, float* dlog_gate, void* ws, size_t ws_bytes,
                           void* stream) {
  SAS_TRY(check_dims(dims, true));
  SAS_TRY(check_len(dims, seq_len, "seq_len"));
  SAS_NONNULL(Q);
  SAS_NONNULL(K);
  SAS_NONNULL(V);
  SAS_NONNULL(O);
  SAS_NONNULL(dO);
  SAS_NONNULL(lse);
  SAS_NONNULL(dQ);
  SAS_NONNULL(dK);
  SAS_NONNULL(dV);
  if (dims->top_k > 0) {
    SAS_NONNULL(idx);
    SAS_NONNULL(dlog_gate);
  }
  if (!(scale > 0.0f)) return fail(SAS_ERR_INVALID_ARGUMENT, "scale must be a positive number");
  SAS_TRY(check_ws(bwd_queries_ws_bytes(*dims, seq_len), ws, ws_bytes));
  return launch_bwd_queries(*dims, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK,
                            dV, dlog_gate, ws, static_cast<hipStream_t>(stream));
}

sas_status sas_selector_bwd(const sas_dims* dims, const void* Q, int32_t q_len, const void* K,
                            const float* Wq_sel, const float* summ, const int32_t* idx,
                            const float* score_lse, const float* dlog_gate, float* ds,
                            float* dWq_sel, float* dWk_sel, void* ws, size_t ws_bytes,
                            void* stream) {
  SAS_TRY(check_dims(dims, false));
  SAS_TRY(check_len(dims, q_len, "q_len"));
  if (cdiv(q_len, kBlock) > kMaxTileRows)
    return fail(SAS_ERR_UNSUPPORTED, "q_len=%d gives more than %d tiles", q_len, kMaxTileRows);
  SAS_NONNULL(Q);
  SAS_NONNULL(K);
  SAS_NONNULL(Wq_sel);
  SAS_NONNULL(score_lse);
  SAS_NONNULL(dWq_sel);
  SAS_NONNULL(dWk_sel);
  if (dims->t_max >= kBlock) SAS_NONNULL(summ);
  if (dims->top_k > 0) {
    SAS_NONNULL(idx);
    SAS_NONNULL(dlog_gate);
  }
  SAS_TRY(check_ws(selector_bwd_ws_bytes(*dims, q_len), ws, ws_bytes));
  return launch_selector_bwd(*dims, Q, q_len, K, Wq_sel, summ, idx, score_lse, dlog_gate, ds,
                             dWq_sel, dWk_sel, ws, static_cast<hipStream_t>(stream));
}

sas_status sas_selector_bwd_queries(const sas_dims* dims, const void* Q, int32_t q_len,
                                    const void* K, const float* Wq_sel, const float* Wk_sel,
                                    const float* summ, const int32_t* idx,
                                    const float* score_lse, const float* dlog_gate, float* ds,
                                    float* dWq_sel, float* dWk_sel, void* ws, size_t ws_bytes,
                                    void* stream) {
  SAS_TRY(check_dims(dims, false));
  SAS_TRY(check_len(dims, q_len, "q_len"));
  if (cdiv(q_len, kBlock) > kMaxTileRows)
    return fail(SAS_ERR_UNSUPPORTED, "q_len=%d gives more than %d tiles", q_len, kMaxTileRows);
  SAS_NONNULL(Q);
  SAS_NONNULL(K);
  SAS_NONNULL(Wq_sel);
  SAS_NONNULL(Wk_sel);
  SAS_NONNULL(score_lse);
  SAS_NONNULL(dWq_sel);
  SAS_NONNULL(dWk_sel);
  if (dims->t_max >= kBlock) SAS_NONNULL(summ);
  if (dims->top_k > 0) {
    SAS_NONNULL(idx);
    SAS_NONNULL(dlog_gate);
  }
  SAS_TRY(check_ws(selector_bwd_queries_ws_bytes(*dims, q_len), ws, ws_bytes));
  return launch_selector_bwd_queries(*dims, Q, q_len, K, Wq_sel, Wk_sel, summ, idx, score_lse,
                                     dlog_gate, ds, dWq_sel, dWk_sel, ws,
                                     static_cast<hipStream_t>(stream));
}

size_t sas_workspace_bytes(int32_t op, const sas_dims* dims, int32_t q_len) {
  const bool bf16_only = (op == SAS_OP_PREFILL_FWD || op == SAS_OP_BWD ||
                          op == SAS_OP_PREFILL_FWD_QUERIES || op == SAS_OP_BWD_QUERIES);
  if (check_dims(dims, bf16_only) != SAS_OK) return SIZE_MAX;
  switch (op) {
    case SAS_OP_SELECT_DECODE: return select_decode_ws_bytes(*dims);
    case SAS_OP_SELECT_TILES: return 0;
    case SAS_OP_SELECT_QUERIES: return 0;
    case SAS_OP_PREFILL_FWD_QUERIES:
      if (check_len(dims, q_len, "q_len") != SAS_OK) return SIZE_MAX;
      return 0;
    case SAS_OP_DECODE_FWD: return decode_ws_bytes(*dims);
    case SAS_OP_DECODE_STEP: return decode_step_ws_bytes(*dims);
    case SAS_OP_SELECTOR_BWD:
      if (check_len(dims, q_len, "q_len") != SAS_OK) return SIZE_MAX;
      return selector_bwd_ws_bytes(*dims, q_len);
    case SAS_OP_PREFILL_FWD:
      if (check_len(dims, q_len, "q_len") != SAS_OK) return SIZE_MAX;
      return prefill_ws_bytes(*dims, q_len);
    case SAS_OP_BWD:
      if (check_len(dims, q_len, "q_len") != SAS_OK) return SIZE_MAX;
      return bwd_ws_bytes(*dims, q_len);
    case SAS_OP_BWD_QUERIES:
      if (check_len(dims, q_len, "q_len") != SAS_OK) return SIZE_MAX;
      return bwd_queries_ws_bytes(*dims, q_len);
    case SAS_OP_SELECTOR_BWD_QUERIES:
      if (check_len(dims, q_len, "q_len") != SAS_OK) return SIZE_MAX;
      return selector_bwd_queries_ws_bytes(*dims, q_len);
    default:
      fail(SAS_ERR_INVALID_ARGUMENT, "op=%d is not a sas_op", op);
      return SIZE_MAX;
  }
}

const char* sas_status_str(int32_t status) {
  switch (status) {
    case SAS_OK: return "SAS_OK";
    case SAS_ERR_INVALID_ARGUMENT: return "SAS_ERR_INVALID_ARGUMENT";
    case SAS_ERR_UNSUPPORTED: return "SAS_ERR_UNSUPPORTED";
    case SAS_ERR_WORKSPACE_TOO_SMALL: return "SAS_ERR_WORKSPACE_TOO_SMALL";
    case SAS_ERR_HIP: return "SAS_ERR_HIP";
    default: return "SAS_UNKNOWN_STATUS";
  }
}

const char* sas_last_error(void) { return g_last_error; }

}  // extern "C"
