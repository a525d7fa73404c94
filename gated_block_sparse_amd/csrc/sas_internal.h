// Internal declarations shared by the libsas translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/sas.h"

namespace sas {

constexpr int kBlock = 64;          // tokens per block (the only size built)
constexpr int kMaxTopK = 64;        // largest k built
constexpr int kChunkGridCap = 256;   // decode select: at most this many chunk workgroups ...
constexpr int kChunkKeysCap = 512;   // ... and merged candidate keys per row for chunks < 256 blocks
constexpr int kMaxTileRows = 1024;  // prefill tiles supported by the tile selector
constexpr int kMaxMergeKeys = 2048; // chunk candidates one decode row may merge
constexpr int kHotBlocks = 16;      // dK/dV: the first blocks may be split across workgroups ...
constexpr int kHotCap = 96;         // ... into chunks of this many reading tiles

// Set the thread-local error text (printf-style) and return `st`.
sas_status fail(sas_status st, const char* fmt, ...);
// Check hipGetLastError() after a launch; returns SAS_OK or SAS_ERR_HIP.
sas_status check_launch(const char* what);

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// ------------------------------------------------------ K/V cache layout ---
// Contiguous (table == nullptr): K/V [B,Hkv,t_max,d].  Paged: logical block
// m of sequence b lives in page table[b * max_pages + m] of a pool K/V
// [n_pages,Hkv,64,d].  Block summaries are [B,Hkv,t_max/64,d_sel] by logical
// block in both layouts (a selection reads them without a table lookup).
struct KvPages {
  const int32_t* table;
  int max_pages;
};
// Index of the first K/V row of block m of (b, r).
__device__ __forceinline__ size_t kv_block_row(const KvPages& pg, int b, int r, int m, int Hkv,
                                               int t_max) {
  if (pg.table)
    return (static_cast<size_t>(pg.table[static_cast<size_t>(b) * pg.max_pages + m]) * Hkv + r) *
           kBlock;
  return (static_cast<size_t>(b) * Hkv + r) * t_max + static_cast<size_t>(m) * kBlock;
}

// ---------------------------------------------------------------- bf16 ---
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------- launchers ---
// Each returns SAS_OK or an error after enqueuing on `st`.  Arguments are
// already validated by the C entry points.

sas_status launch_block_summaries(const sas_dims& d, const void* K, const int32_t* seq_lens,
                                  const float* Wk, int blk_begin, int blk_end, float* summ,
                                  hipStream_t st);
// The same on a paged cache (pg.table non-null); summ stays logical.
sas_status launch_block_summaries_paged(const sas_dims& d, const void* K, KvPages pg,
                                        const int32_t* seq_lens, const float* Wk, int blk_begin,
                                        int blk_end, float* summ, hipStream_t st);

size_t select_decode_ws_bytes(const sas_dims& d);
sas_status launch_select_decode(const sas_dims& d, const void* q, const int32_t* seq_lens,
                                const float* Wq, const float* summ, int32_t* idx, float* log_gate,
                                float* score_lse, float* scores, void* ws, hipStream_t st);
// One selection row per query (rows = q_len; row i has C = i / 64).
sas_status launch_select_queries(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                                 const float* summ, int32_t* idx, float* log_gate,
                                 float* score_lse, float* scores, hipStream_t st);
sas_status launch_select_tiles(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                               const float* summ, int32_t* idx, float* log_gate,
                               float* score_lse, float* scores, hipStream_t st);

// Where the decode selection keeps its per-chunk state in its workspace:
// part[rows * nchunk] (max, sum-exp) and cand[rows * nchunk * kc] sorted keys.
struct SelectDecodeLayout {
  int nchunk, nlist, kc;  // chunks per row, chunks rounded up to a power of two, keys per chunk
  float2* part;
  uint64_t* cand;
};
SelectDecodeLayout select_decode_layout(const sas_dims& d, void* ws);
// The first stage of the decode selection alone (scores, per-chunk state);
// when a row fits one chunk it also writes the final idx/log_gate/score_lse.
// With Wk non-null, the workgroup holding each row's newest complete block
// C-1 first recomputes that block's summary from K (the summaries kernel's
// arithmetic, same bits), stores it into summ and scores with it.  With
// dec_cnt non-null it also zeroes dec_cnt[row] for every (sequence, group)
// row (the arrival counts of the fused decode step's merge).
sas_status launch_select_decode_chunks(const sas_dims& d, const void* q, const int32_t* seq_lens,
                                       const float* Wq, const float* summ, const void* K,
                                       const float* Wk, KvPages pg, int32_t* idx,
                                       float* log_gate, float* score_lse, void* ws,
                                       hipStream_t st, int* dec_cnt = nullptr);
// Its second stage: merges the per-chunk state into idx/log_gate/score_lse
// (nothing to do when a row fits one chunk).
sas_status launch_select_decode_merge(const sas_dims& d, const int32_t* seq_lens, int32_t* idx,
                                      float* log_gate, float* score_lse, void* ws,
                                      hipStream_t st);

size_t decode_ws_bytes(const sas_dims& d);
sas_status launch_decode_fwd(const sas_dims& d, const void* q, const void* K, const void* V,
                             const int32_t* seq_lens, const int32_t* idx, const float* log_gate,
                             float scale, void* o, float* lse, void* ws, hipStream_t st);

size_t decode_step_ws_bytes(const sas_dims& d);
sas_status launch_decode_step(const sas_dims& d, const void* q, const void* K, const void* V,
                              const int32_t* seq_lens, const float* Wq, const float* summ,
                              const float* Wk, KvPages pg, int gated, float scale, int32_t* idx, float* log_gate,
                              float* score_lse, void* o, float* lse, void* ws, hipStream_t st);

size_t selector_bwd_ws_bytes(const sas_dims& d, int q_len);
sas_status launch_selector_bwd(const sas_dims& d, const void* Q, int q_len, const void* K,
                               const float* Wq, const float* summ, const int32_t* idx,
                               const float* score_lse, const float* dlg, float* ds, float* dWq,
                               float* dWk, void* ws, hipStream_t st);
// The same for per-query rows (idx/score_lse/dlog_gate [B,Hkv,q_len,...]).
size_t selector_bwd_queries_ws_bytes(const sas_dims& d, int q_len);
sas_status launch_selector_bwd_queries(const sas_dims& d, const void* Q, int q_len,
                                       const void* K, const float* Wq, const float* Wk,
                                       const float* summ, const int32_t* idx,
                                       const float* score_lse, const float* dlg, float* ds,
                                       float* dWq, float* dWk, void* ws, hipStream_t st);

size_t prefill_ws_bytes(const sas_dims& d, int seq_len);
sas_status launch_prefill_fwd(const sas_dims& d, const void* Q, const void* K, const void* V,
                              int seq_len, const int32_t* idx, const float* log_gate,
                              float scale, void* O, float* lse, void* ws, hipStream_t st);
// The same with one selection per query: idx/log_gate [B,Hkv,seq_len,k].
sas_status launch_prefill_fwd_queries(const sas_dims& d, const void* Q, const void* K,
                                      const void* V, int seq_len, const int32_t* idx,
                                      const float* log_gate, float scale, void* O, float* lse,
                                      hipStream_t st);

size_t bwd_ws_bytes(const sas_dims& d, int seq_len);
sas_status launch_bwd(const sas_dims& d, const void* Q, const void* K, const void* V,
                      const void* O, const void* dO, const float* lse, int seq_len,
                      const int32_t* idx, const float* log_gate, float scale, void* dQ,
                      void* dK, void* dV, float* dlog_gate, void* ws, hipStream_t st);
// The same with one selection per query: idx/log_gate/dlog_gate [B,Hkv,seq_len,k].
size_t bwd_queries_ws_bytes(const sas_dims& d, int seq_len);
sas_status launch_bwd_queries(const sas_dims& d, const void* Q, const void* K, const void* V,
                              const void* O, const void* dO, const float* lse, int seq_len,
                              const int32_t* idx, const float* log_gate, float scale, void* dQ,
                              void* dK, void* dV, float* dlog_gate, void* ws, hipStream_t st);

}  // namespace sas
