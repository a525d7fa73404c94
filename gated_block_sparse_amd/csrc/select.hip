// Selector score, softmax gate and Top-K (SAS close reading 2.1-2.2; SAS
// summary, Method; MSA notes 4.1 for ranking the raw scores).
//
//   s_m       = qbar . summ_m,  qbar = Wq_sel . mean(q over the row) / sqrt(d_sel)
//   score_lse = LSE over the row's C history blocks
//   idx       = the min(k, C) largest s (ties -> lower m), ascending
//   log_gate  = s_idx - score_lse
//
// The score is linear in q, so the row's queries are pooled before the
// projection.  Top-K works on 64-bit keys (order-preserving score bits, then
// ~m), a strict total order, so the sort is exact and deterministic.
//
// Decode: C can reach thousands of blocks and the summary scan is the HBM
// traffic, so the row is cut into chunks of 64-256 blocks, one workgroup
// each: score (half a wave per 128-float summary row), chunk max/sum-exp, and
// the chunk's own top-k by an LDS bitonic sort.  A second small kernel per row
// merges the chunk LSE states and the chunk candidates.
// Tiles (prefill): one workgroup per (tile, group) does everything.
#include "sas_device.h"
#include "sas_internal.h"
#include "sas_select_dev.h"
#include "sas_summary_dev.h"

namespace sas {


// ------------------------------------------------------------- decode ---
// Chunk kernel: grid (chunk, group, sequence), 8R blocks per chunk (half
// wave hw owns blocks hw + 8j, j < R).  Every load the workgroup needs (the
// lane's channels of the group's query heads, its slices of d_sel/8 Wq_sel
// rows and of R summary rows) is issued before any arithmetic, so the kernel
// pays about one memory round trip; both the projection and the scores read
// whole rows per half wave (coalesced) and finish with a transposing
// butterfly sum.  Each wave then sorts its 64 scores with a shuffle bitonic
// network, the four sorted lists are merged by rank (a key's rank is its
// position in its own list plus the number of larger keys in the others,
// found by binary search), and the chunk's top-k keys plus its (max, sum-exp)
// go to the workspace.  A row that fits one chunk is finished right here.
template <typename T, int D, int DS, int G, int R>
__global__ void __launch_bounds__(kSelThreads)
select_decode_chunk_kernel(const T* __restrict__ q, const int32_t* __restrict__ seq_lens,
                           const float* __restrict__ Wq, const float* summ,
                           const T* __restrict__ K, const float* __restrict__ Wk,
                           float* summ_out, KvPages pg, int Hkv, int t_max, int c_max, int k,
                           int kc, int nchunk,
                           float* __restrict__ scores, float2* __restrict__ part,
                           uint64_t* __restrict__ cand, int32_t* __restrict__ idx,
                           float* __restrict__ log_gate, float* __restrict__ score_lse,
                           int* __restrict__ dec_cnt) {
  constexpr int PL = DS / 32;                 // summary floats per lane
  constexpr int PD = D / 32;                  // query channels per lane
  constexpr int RW = DS / 8;                  // Wq_sel rows per half wave
  constexpr int NW = kSelThreads / 64;
  constexpr int kChunk = 8 * R;
  static_assert(PL == 2 || PL == 4, "d_sel");
  static_assert(PD == 2 || PD == 4, "d");
  __shared__ float qs[DS];
  __shared__ uint64_t lists[NW][64];
  __shared__ uint64_t best[kMaxTopK];
  __shared__ float red[2][NW];
  __shared__ float rmean[D];   // fused refresh: pooled keys, then the new summary
  __shared__ float rsumm[DS];
  static_assert(kSelThreads == kSumThreads, "the refresh uses the summaries' thread mapping");

  const int b = blockIdx.z, r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, hw = tid >> 5, l32 = tid & 31;
  const int len = clamp_len(seq_lens[b], t_max);
  const int C = (len - 1) / kBlock;
  const int m0 = chunk * kChunk;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  const size_t p = row * nchunk + chunk;
  const int n = max(0, min(kChunk, C - m0));
  if (dec_cnt && chunk == 0 && tid == 0) dec_cnt[row] = 0;
  // fused refresh (Wk given): this workgroup holds the newest complete block
  const int mnew = C - 1;
  const bool refresh = Wk != nullptr && n > 0 && mnew >= m0 && mnew < m0 + n;

  // ---- all loads up front (the refresh's K block and Wk_sel slice first:
  // they start the longest chain of this workgroup)
  WkSlice<D, DS> wsl;
  BlockMean<T, D> bm;
  if (refresh) {
    wsl.load(Wk, tid);
    if (wave == 0) bm.load(K + kv_block_row(pg, b, r, mnew, Hkv, t_max) * D, lane);
  }
  float qraw[G][PD];
  {
    const T* qb = q + (row * G) * static_cast<size_t>(D) + PD * l32;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < PD; ++e) qraw[h][e] = load_scalar<T>(qb + h * D + e);
  }
  float wv[RW][PD];
  {
    const float* wr = Wq + static_cast<size_t>(hw) * D + PD * l32;
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      const float* w = wr + static_cast<size_t>(8 * j) * D;
      if constexpr (PD == 4) {
        const float4 x = *reinterpret_cast<const float4*>(w);
        wv[j][0] = x.x; wv[j][1] = x.y; wv[j][2] = x.z; wv[j][3] = x.w;
      } else {
        const float2 x = *reinterpret_cast<const float2*>(w);
        wv[j][0] = x.x; wv[j][1] = x.y;
      }
    }
  }
  float xs[R][PL];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = hw + 8 * j;
#pragma unroll
    for (int e = 0; e < PL; ++e) xs[j][e] = 0.f;
    if (i < n) {
      const float* sp = summ + ((row * c_max) + m0 + i) * static_cast<size_t>(DS) + l32 * PL;
      if constexpr (PL == 4) {
        const float4 x = *reinterpret_cast<const float4*>(sp);
        xs[j][0] = x.x; xs[j][1] = x.y; xs[j][2] = x.z; xs[j][3] = x.w;
      } else {
        const float2 x = *reinterpret_cast<const float2*>(sp);
        xs[j][0] = x.x; xs[j][1] = x.y;
      }
    }
  }
  // ---- fused refresh of block mnew: its summary is recomputed from K with
  // the summaries kernel's own arithmetic, stored, and replaces the (stale)
  // slice of row mnew loaded above
  if (refresh) {
    if (wave == 0) bm.reduce(lane, rmean);
    __syncthreads();
    const float a = wsl.project(rmean, tid);
    if (tid % WkSlice<D, DS>::SPLIT == 0) {
      const int jo = tid / WkSlice<D, DS>::SPLIT;
      rsumm[jo] = a;
      summ_out[(row * c_max + mnew) * static_cast<size_t>(DS) + jo] = a;
    }
    __syncthreads();
    const int i = mnew - m0;
    if (hw == (i & 7)) {
#pragma unroll
      for (int j = 0; j < R; ++j)
        if (j == (i >> 3)) {
#pragma unroll
          for (int e = 0; e < PL; ++e) xs[j][e] = rsumm[l32 * PL + e];
        }
    }
  }
  // ---- pooled query, projected: half wave hw owns Wq_sel rows hw + 8j
  {
    float qm[PD];
#pragma unroll
    for (int e = 0; e < PD; ++e) {
      float a = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) a += qraw[h][e];
      qm[e] = a / G;
    }
    float pv[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < PD; ++e) a += wv[j][e] * qm[e];
      pv[j] = a;
    }
    const float proj = transpose_sum<RW>(pv, l32);
    if (l32 < RW) qs[hw + 8 * l32] = proj * (1.0f / sqrtf(static_cast<float>(DS)));
  }
  __syncthreads();
  // ---- scores: the transposed butterfly leaves row hw + 8 * (l32 % R) in
  // lane l32 (lanes l32 >= R hold copies and stand aside)
  float v[R];
  {
    float qv[PL];
#pragma unroll
    for (int e = 0; e < PL; ++e) qv[e] = qs[l32 * PL + e];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < PL; ++e) a += xs[j][e] * qv[e];
      v[j] = a;
    }
  }
  const float sdot = transpose_sum<R>(v, l32);
  const int i_row = hw + 8 * (l32 & (R - 1));
  const bool valid = l32 < R && i_row < n;
  const float sc = valid ? sdot : -INFINITY;
  if (scores && valid) scores[row * c_max + m0 + i_row] = sc;

  // ---- chunk (max, sum exp)
  float mx = group_max(sc, 64);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[0][w]);
  float se = group_sum(valid ? expf(sc - M) : 0.f, 64);
  if (lane == 0) red[1][wave] = se;

  // ---- chunk top-k
  const uint64_t key = wave_sort_desc(valid ? topk_key(sc, m0 + i_row) : 0ull);
  lists[wave][lane] = key;
  __syncthreads();
  float Ssum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) Ssum += red[1][w];
  {
    int rank = lane;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w != wave) rank += count_greater_desc(lists[w], 64, key);
    if (rank < kc && key != 0ull) best[rank] = key;
  }
  __syncthreads();
  const int nk = min(kc, n);  // valid keys among the chunk's best
  if (nchunk == 1) {
    const float lse = C > 0 ? M + logf(Ssum) : -INFINITY;
    write_selection(best, min(k, C), k, lse, idx + row * k, log_gate + row * k);
    if (tid == 0) score_lse[row] = lse;
    return;
  }
  if (tid < kc) cand[p * kc + tid] = tid < nk ? best[tid] : 0ull;
  if (tid == 0) part[p] = n > 0 ? make_float2(M, Ssum) : make_float2(-INFINITY, 0.f);
}

// Merge kernel: one workgroup per (group, sequence) combines the chunk
// (max, sum-exp) pairs into LSE(s) and merges the chunks' sorted candidate
// lists pairwise, log2(#chunks) levels: an element's place in the merged list
// is its own position plus the number of larger keys in the partner list
// (binary search), and each merged list keeps its top kc.
__global__ void __launch_bounds__(kSelThreads)
select_decode_merge_kernel(const int32_t* __restrict__ seq_lens, int Hkv, int t_max, int k,
                           int kc, int nchunk, int nlist, const float2* __restrict__ part,
                           const uint64_t* __restrict__ cand, int32_t* __restrict__ idx,
                           float* __restrict__ log_gate, float* __restrict__ score_lse) {
  extern __shared__ uint64_t lds[];          // two buffers of nlist * kc keys
  __shared__ float red[kSelThreads / 64];
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int len = clamp_len(seq_lens[b], t_max);
  const int C = (len - 1) / kBlock;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  uint64_t* src = lds;
  uint64_t* dst = lds + nlist * kc;
  const float lse = load_chunk_states(cand + row * static_cast<size_t>(nchunk * kc),
                                      part + row * nchunk, nchunk, nlist, kc, C, src, red);
  src = merge_sorted_lists(src, dst, nlist, kc);
  write_selection(src, min(k, C), k, lse, idx + row * k, log_gate + row * k);
  if (tid == 0) score_lse[row] = lse;
}

// Blocks per decode chunk, 8R with R rows per half wave: the smallest chunk
// that keeps the grid within one workgroup per CU and the merged candidate
// lists short (more, smaller chunks mean more loads in flight at batch 1),
// else 256.
static int chunk_count(int c_max, int R) {
  const int n = cdiv(c_max, 8 * R);
  return n > 0 ? n : 1;
}
static int decode_chunk_rows(const sas_dims& d) {
  const long rows = static_cast<long>(d.batch) * d.n_kv_heads;
  const int kc = d.top_k > 0 ? d.top_k : 1;
  for (int R = 8; R < 32; R <<= 1) {
    const int nc = chunk_count(d.t_max / kBlock, R);
    int nl = 1;
    while (nl < nc) nl <<= 1;
    if (rows * nc <= kChunkGridCap && nl * kc <= kChunkKeysCap) return R;
  }
  return 32;
}
static int decode_nchunk(const sas_dims& d) {
  return chunk_count(d.t_max / kBlock, decode_chunk_rows(d));
}
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: part[rows*nchunk] | cand[rows*nchunk*max(k,1)]
size_t select_decode_ws_bytes(const sas_dims& d) {
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  const size_t nc = decode_nchunk(d);
  return align256(rows * nc * sizeof(float2)) +
         rows * nc * static_cast<size_t>(d.top_k > 0 ? d.top_k : 1) * sizeof(uint64_t);
}

SelectDecodeLayout select_decode_layout(const sas_dims& d, void* ws) {
  SelectDecodeLayout L;
  L.nchunk = decode_nchunk(d);
  L.kc = d.top_k > 0 ? d.top_k : 1;
  L.nlist = 1;
  while (L.nlist < L.nchunk) L.nlist <<= 1;
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  char* w = static_cast<char*>(ws);
  L.part = reinterpret_cast<float2*>(w);
  L.cand = reinterpret_cast<uint64_t*>(w + align256(rows * L.nchunk * sizeof(float2)));
  return L;
}

template <typename T, int D, int DS, int G>
static sas_status launch_sd_chunks(const sas_dims& d, const void* q, const int32_t* seq_lens,
                                   const float* Wq, const float* summ, const void* K,
                                   const float* Wk, KvPages pg, int32_t* idx, float* log_gate,
                                   float* score_lse, float* scores, void* ws, hipStream_t st,
                                   int* dec_cnt) {
  const SelectDecodeLayout L = select_decode_layout(d, ws);
  if (L.nlist * L.kc > kMaxMergeKeys)
    return fail(SAS_ERR_UNSUPPORTED, "select: %d chunk candidates exceed the merge buffer",
                L.nlist * L.kc);
#define SAS_SD_CHUNK(R)                                                                       \
  hipLaunchKernelGGL((select_decode_chunk_kernel<T, D, DS, G, R>),                              \
                     dim3(L.nchunk, d.n_kv_heads, d.batch), dim3(kSelThreads), 0, st,           \
                     static_cast<const T*>(q), seq_lens, Wq, summ, static_cast<const T*>(K),    \
                     Wk, const_cast<float*>(summ), pg, d.n_kv_heads, d.t_max, d.t_max / kBlock, \
                     d.top_k, L.kc, L.nchunk, scores, L.part, L.cand, idx, log_gate, score_lse, \
                     dec_cnt)
  switch (decode_chunk_rows(d)) {
    case 8: SAS_SD_CHUNK(8); break;
    case 16: SAS_SD_CHUNK(16); break;
    default: SAS_SD_CHUNK(32); break;
  }
#undef SAS_SD_CHUNK
  return check_launch("select_decode_chunk");
}

sas_status launch_select_decode_merge(const sas_dims& d, const int32_t* seq_lens, int32_t* idx,
                                      float* log_gate, float* score_lse, void* ws,
                                      hipStream_t st) {
  const SelectDecodeLayout L = select_decode_layout(d, ws);
  if (L.nchunk == 1) return SAS_OK;
  hipLaunchKernelGGL(select_decode_merge_kernel, dim3(d.n_kv_heads, d.batch), dim3(kSelThreads),
                     2 * L.nlist * L.kc * sizeof(uint64_t), st, seq_lens, d.n_kv_heads, d.t_max,
                     d.top_k, L.kc, L.nchunk, L.nlist, L.part, L.cand, idx, log_gate, score_lse);
  return check_launch("select_decode_merge");
}

template <typename T, int D, int DS, int G>
static sas_status launch_sd(const sas_dims& d, const void* q, const int32_t* seq_lens,
                            const float* Wq, const float* summ, int32_t* idx, float* log_gate,
                            float* score_lse, float* scores, void* ws, hipStream_t st) {
  sas_status s = launch_sd_chunks<T, D, DS, G>(d, q, seq_lens, Wq, summ, nullptr, nullptr,
                                               KvPages{nullptr, 0}, idx, log_gate, score_lse,
                                               scores, ws, st, nullptr);
  if (s != SAS_OK) return s;
  return launch_select_decode_merge(d, seq_lens, idx, log_gate, score_lse, ws, st);
}

// -------------------------------------------------------------- tiles ---
template <typename T, int D, int DS, int G>
__global__ void __launch_bounds__(kSelThreads)
select_tiles_kernel(const T* __restrict__ Q, int q_len, const float* __restrict__ Wq,
                    const float* __restrict__ summ, int Hkv, int c_max, int rows, int k,
                    int32_t* __restrict__ idx, float* __restrict__ log_gate,
                    float* __restrict__ score_lse, float* __restrict__ scores) {
  __shared__ float qpart[kSelThreads / (D / Vec16<T>::N)][D];
  __shared__ float qm[D];
  __shared__ float qs[DS];
  __shared__ float sc[kMaxTileRows];
  __shared__ uint64_t keys[kMaxTileRows];
  __shared__ float red[kSelThreads / 64];

  const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int C = t;
  const int i0 = t * kBlock;
  const int nq = min(kBlock, q_len - i0);
  const size_t row = (static_cast<size_t>(b) * Hkv + r) * rows + t;

  tile_pooled_query<T, D, G>(Q, q_len, Hkv, b, r, i0, nq, &qpart[0][0], qm);
  project_query<D, DS>(Wq, qm, qs);
  __syncthreads();

  const float* srow = summ + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(c_max) * DS;
  score_rows<DS>(srow, qs, C, sc);
  __syncthreads();

  float mloc = -INFINITY;
  for (int m = tid; m < C; m += kSelThreads) mloc = fmaxf(mloc, sc[m]);
  const float M = block_max(mloc, red);
  float sloc = 0.f;
  for (int m = tid; m < C; m += kSelThreads) sloc += expf(sc[m] - M);
  const float L = block_sum(sloc, red);
  const float lse = C > 0 ? M + logf(L) : -INFINITY;
  if (scores)
    for (int m = tid; m < C; m += kSelThreads) scores[row * c_max + m] = sc[m];

  const int npow = C <= 2 ? 2 : (1 << (32 - __clz(C - 1)));
  for (int m = tid; m < npow; m += kSelThreads) keys[m] = m < C ? topk_key(sc[m], m) : 0ull;
  bitonic_sort_desc(keys, npow);
  const int kk = min(k, C);
  write_selection(keys, kk, k, lse, idx + row * k, log_gate + row * k);
  if (tid == 0) score_lse[row] = lse;
}

// ------------------------------------------------------------ queries ---
// One selection per query (SAS close reading 2.4: the training kernel masks
// every query by its own gate threshold).  Query i has the C = i / 64
// complete blocks before its own block as history, and its score of block m
// is the decode score of a query at position i: the mean over the group's G
// heads of (Wq_sel q_h) . summ_m / sqrt(d_sel).  The GPU pools the G heads
// first and projects once (linear; fp32 rounding only).
//
// One workgroup per 32 queries (half a tile), group and sequence; all its
// queries share C.  The pooled queries and then their projections u (32 x
// d_sel) sit in LDS; the summaries are scored in chunks of 64 blocks staged
// in LDS (rows padded by 4 floats: the 16-byte reads of 16 consecutive rows
// hit distinct banks), each thread forming 2 queries x 4 blocks.  Each wave
// then keeps, for 8 queries, a running (max, sum-exp) and a running Top-K
// list (descending composite keys, as in the decode selection): it sorts the
// chunk's 64 keys across its lanes and merges them with the list by rank (a
// key's place in the merged list is its own position plus the number of
// larger keys in the other list).
constexpr int kQsRows = 32;   // queries per workgroup
constexpr int kQsChunk = 64;  // blocks scored per pass

template <typename T, int D, int DS, int G>
__global__ void __launch_bounds__(kSelThreads, 2)   // two workgroups per CU (LDS allows it)
select_queries_kernel(const T* __restrict__ Q, int q_len, const float* __restrict__ Wq,
                      const float* __restrict__ summ, int Hkv, int c_max, int k,
                      int32_t* __restrict__ idx, float* __restrict__ log_gate,
                      float* __restrict__ score_lse, float* __restrict__ scores) {
  constexpr int NW = kSelThreads / 64;          // waves
  constexpr int QPW = kQsRows / NW;             // queries per wave in the Top-K phase
  constexpr int QS = D + 4, US = DS + 4;        // padded LDS row strides (floats)
  constexpr int BUF = (kQsRows * QS > kQsChunk * US) ? kQsRows * QS : kQsChunk * US;
  __shared__ __attribute__((aligned(16))) float buf[BUF];        // pooled queries, then summaries
  __shared__ __attribute__((aligned(16))) float u[kQsRows * US];  // projected queries
  __shared__ float sc[kQsRows][kQsChunk + 1];
  __shared__ uint64_t top[kQsRows][kMaxTopK];

  const int t = blockIdx.x >> 1, r = blockIdx.y, b = blockIdx.z;
  const int i0 = t * kBlock + (blockIdx.x & 1) * kQsRows;
  const int nq = min(kQsRows, q_len - i0);
  if (nq <= 0) return;   // second half of a short last tile (workgroup-uniform)
  const int C = t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- pooled queries qbar[q] = (1/G) sum_h Q[b, rG+h, i0+q, :]
  {
    constexpr int EPL = Vec16<T>::N, LPR = D / EPL;
    for (int x = tid; x < kQsRows * LPR; x += kSelThreads) {
      const int q = x / LPR, col = x % LPR;
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
      if (q < nq) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const T* src = Q + ((static_cast<size_t>(b) * Hkv * G + r * G + h) * q_len + i0 + q) * D +
                         col * EPL;
          float f[EPL];
          Vec16<T>::unpack(*reinterpret_cast<const uint4*>(src), f);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] += f[e];
        }
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) buf[q * QS + col * EPL + e] = acc[e] * (1.0f / G);
    }
  }
  __syncthreads();
  // ---- u[q][c] = (Wq[c,:] . qbar[q]) / sqrt(DS); thread: channel c, every
  // NQG-th query (a wave shares its query rows: broadcast LDS reads)
  {
    constexpr int NQG = kSelThreads / DS, NE = kQsRows / NQG;
    const int c = tid % DS, qg = tid / DS;
    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
    const float4* w = reinterpret_cast<const float4*>(Wq + static_cast<size_t>(c) * D);
#pragma unroll 4
    for (int j4 = 0; j4 < D / 4; ++j4) {
      const float4 x = w[j4];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float4 a = *reinterpret_cast<const float4*>(&buf[(qg + NQG * e) * QS + 4 * j4]);
        acc[e] += x.x * a.x + x.y * a.y + x.z * a.z + x.w * a.w;
      }
    }
    const float inv = 1.0f / sqrtf(static_cast<float>(DS));
#pragma unroll
    for (int e = 0; e < NE; ++e) u[(qg + NQG * e) * US + c] = acc[e] * inv;
  }

  float run_m[QPW], run_s[QPW];
#pragma unroll
  for (int e = 0; e < QPW; ++e) {
    run_m[e] = -INFINITY;
    run_s[e] = 0.f;
  }
  const float* srow = summ + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(c_max) * DS;
  const size_t row0 = (static_cast<size_t>(b) * Hkv + r) * q_len + i0;   // row of query i0

  for (int c0 = 0; c0 < C; c0 += kQsChunk) {
    const int nb = min(kQsChunk, C - c0);
    __syncthreads();   // the previous chunk's readers of buf/sc are done (and u is written)
    // ---- stage the chunk's summaries
    for (int x = tid; x < kQsChunk * (DS / 4); x += kSelThreads) {
      const int m = x / (DS / 4), c4 = x % (DS / 4);
      const float4 v = m < nb ? *reinterpret_cast<const float4*>(srow + static_cast<size_t>(c0 + m) * DS + 4 * c4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&buf[m * US + 4 * c4]) = v;
    }
    __syncthreads();
    // ---- scores: thread (tq, tm) takes queries 2tq, 2tq+1 and blocks tm + 16x
    {
      const int tq = tid >> 4, tm = tid & 15;
      float acc[2][4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[a][x] = 0.f;
#pragma unroll 2
      for (int j4 = 0; j4 < DS / 4; ++j4) {
        float4 uq[2], sv[4];
#pragma unroll
        for (int a = 0; a < 2; ++a) uq[a] = *reinterpret_cast<const float4*>(&u[(2 * tq + a) * US + 4 * j4]);
#pragma unroll
        for (int x = 0; x < 4; ++x) sv[x] = *reinterpret_cast<const float4*>(&buf[(tm + 16 * x) * US + 4 * j4]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            acc[a][x] += uq[a].x * sv[x].x + uq[a].y * sv[x].y + uq[a].z * sv[x].z + uq[a].w * sv[x].w;
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int q = 2 * tq + a, m = tm + 16 * x;
          sc[q][m] = acc[a][x];
          if (scores && q < nq && m < nb)
            scores[(row0 + q) * c_max + c0 + m] = acc[a][x];
        }
    }
    __syncthreads();
    // ---- per query: softmax state and Top-K list.  A wave's QPW queries go
    // through every step in lockstep (each cross-lane step is issued for all
    // of them before the next), so the latencies of the lane shuffles and of
    // the LDS reads of the searches overlap instead of adding up.  Rows of
    // queries past nq are processed too (finite zeros) and never output.
    {
      const bool ok = lane < nb;
      float sv[QPW], cm[QPW], ex[QPW];
#pragma unroll
      for (int e = 0; e < QPW; ++e) {
        sv[e] = sc[wave * QPW + e][lane];
        cm[e] = ok ? sv[e] : -INFINITY;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < QPW; ++e) cm[e] = fmaxf(cm[e], __shfl_xor(cm[e], o, 64));
#pragma unroll
      for (int e = 0; e < QPW; ++e) {
        cm[e] = fmaxf(run_m[e], cm[e]);   // the new running max
        ex[e] = ok ? expf(sv[e] - cm[e]) : 0.f;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < QPW; ++e) ex[e] += __shfl_xor(ex[e], o, 64);
#pragma unroll
      for (int e = 0; e < QPW; ++e) {
        run_s[e] = run_s[e] * expf(run_m[e] - cm[e]) + ex[e];
        run_m[e] = cm[e];
      }
      if (k > 0) {
        // bitonic sort of each query's 64 chunk keys across the lanes
        // (descending: lane 0 holds the largest)
        uint64_t key[QPW];
#pragma unroll
        for (int e = 0; e < QPW; ++e) key[e] = ok ? topk_key(sv[e], c0 + lane) : 0ull;
#pragma unroll
        for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
#pragma unroll
            for (int e = 0; e < QPW; ++e) {
              const uint64_t other = shfl_xor_u64(key[e], stride);
              key[e] = keep_max ? (key[e] > other ? key[e] : other)
                                : (key[e] < other ? key[e] : other);
            }
          }
        // merge with the running list by rank: a key's place is its own
        // position plus the number of larger keys in the other list (a
        // binary search of at most 7 steps, n <= 64)
        const int n_old = min(k, c0);   // kept so far (every earlier block is a candidate)
        const int n_new = min(k, c0 + nb);
        uint64_t lk[QPW];
        int lo[QPW], hi[QPW], lo2[QPW], hi2[QPW];
#pragma unroll
        for (int e = 0; e < QPW; ++e) {
          lk[e] = lane < n_old ? top[wave * QPW + e][lane] : 0ull;
          lo[e] = 0;
          hi[e] = n_old;
          lo2[e] = 0;
          hi2[e] = nb;
        }
#pragma unroll
        for (int step = 0; step < 7; ++step)
#pragma unroll
          for (int e = 0; e < QPW; ++e) {
            // place of this lane's chunk key in the list (LDS)
            const int mid = (lo[e] + hi[e]) >> 1;
            if (lo[e] < hi[e]) {
              if (top[wave * QPW + e][mid] > key[e]) lo[e] = mid + 1;
              else hi[e] = mid;
            }
            // place of this lane's list key among the chunk keys (lanes)
            const int mid2 = (lo2[e] + hi2[e]) >> 1;
            const uint32_t src = static_cast<uint32_t>(min(mid2, 63));
            const uint64_t v = (static_cast<uint64_t>(__shfl(static_cast<uint32_t>(key[e] >> 32), src, 64)) << 32) |
                               __shfl(static_cast<uint32_t>(key[e]), src, 64);
            if (lo2[e] < hi2[e]) {
              if (v > lk[e]) lo2[e] = mid2 + 1;
              else hi2[e] = mid2;
            }
          }
        // every read of the lists is done before any lane writes them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int e = 0; e < QPW; ++e) {
          const int pc = ok ? lane + lo[e] : kMaxTopK;
          const int pl = lane < n_old ? lane + lo2[e] : kMaxTopK;
          if (pc < n_new) top[wave * QPW + e][pc] = key[e];
          if (pl < n_new) top[wave * QPW + e][pl] = lk[e];
        }
      }
    }
  }
  // ---- outputs: ascending idx, log g = s - LSE(s), LSE
  __syncthreads();
#pragma unroll
  for (int e = 0; e < QPW; ++e) {
    const int q = wave * QPW + e;
    if (q >= nq) continue;
    const float lse = C > 0 ? run_m[e] + logf(run_s[e]) : -INFINITY;
    const int kk = min(k, C);
    const size_t row = row0 + q;
    if (lane < kk) {
      const uint64_t key = top[q][lane];
      const int mb = key_block(key);
      int rank = 0;
      for (int j = 0; j < kk; ++j) rank += key_block(top[q][j]) < mb;
      idx[row * k + rank] = mb;
      log_gate[row * k + rank] = key_score(key) - lse;
    } else if (lane < k) {
      idx[row * k + lane] = -1;
      log_gate[row * k + lane] = -INFINITY;
    }
    if (lane == 0) score_lse[row] = lse;
  }
}

// ---------------------------------------------------------- dispatch ---
template <typename T, int D, int DS, int G>
struct SelDecode {
  static sas_status run(const sas_dims& d, const void* q, const int32_t* seq_lens, const float* Wq,
                        const float* summ, int32_t* idx, float* log_gate, float* score_lse,
                        float* scores, void* ws, hipStream_t st) {
    return launch_sd<T, D, DS, G>(d, q, seq_lens, Wq, summ, idx, log_gate, score_lse, scores,
                                  ws, st);
  }
};

template <typename T, int D, int DS, int G>
struct SelDecodeChunks {
  static sas_status run(const sas_dims& d, const void* q, const int32_t* seq_lens, const float* Wq,
                        const float* summ, const void* K, const float* Wk, KvPages pg,
                        int32_t* idx, float* log_gate, float* score_lse, float* scores, void* ws,
                        hipStream_t st, int* dec_cnt) {
    return launch_sd_chunks<T, D, DS, G>(d, q, seq_lens, Wq, summ, K, Wk, pg, idx, log_gate,
                                         score_lse, scores, ws, st, dec_cnt);
  }
};

template <typename T, int D, int DS, int G>
struct SelTiles {
  static sas_status run(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                        const float* summ, int32_t* idx, float* log_gate, float* score_lse,
                        float* scores, hipStream_t st) {
    const int rows = cdiv(q_len, kBlock);
    hipLaunchKernelGGL((select_tiles_kernel<T, D, DS, G>), dim3(rows, d.n_kv_heads, d.batch),
                       dim3(kSelThreads), 0, st, static_cast<const T*>(Q), q_len, Wq, summ,
                       d.n_kv_heads, d.t_max / kBlock, rows, d.top_k, idx, log_gate, score_lse,
                       scores);
    return check_launch("select_tiles");
  }
};

template <typename T, int D, int DS, int G>
struct SelQueries {
  static sas_status run(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                        const float* summ, int32_t* idx, float* log_gate, float* score_lse,
                        float* scores, hipStream_t st) {
    const int n_tiles = cdiv(q_len, kBlock);
    hipLaunchKernelGGL((select_queries_kernel<T, D, DS, G>), dim3(2 * n_tiles, d.n_kv_heads,
                       d.batch), dim3(kSelThreads), 0, st, static_cast<const T*>(Q), q_len, Wq,
                       summ, d.n_kv_heads, d.t_max / kBlock, d.top_k, idx, log_gate, score_lse,
                       scores);
    return check_launch("select_queries");
  }
};

template <template <typename, int, int, int> class F, typename T, int D, int DS, typename... A>
static sas_status by_group(const sas_dims& d, A... a) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return F<T, D, DS, 1>::run(d, a...);
    case 2: return F<T, D, DS, 2>::run(d, a...);
    case 4: return F<T, D, DS, 4>::run(d, a...);
    case 8: return F<T, D, DS, 8>::run(d, a...);
  }
  return fail(SAS_ERR_UNSUPPORTED, "select: group size");
}

template <template <typename, int, int, int> class F, typename T, typename... A>
static sas_status by_dims(const sas_dims& d, A... a) {
  if (d.head_dim == 64 && d.sel_dim == 64) return by_group<F, T, 64, 64>(d, a...);
  if (d.head_dim == 64 && d.sel_dim == 128) return by_group<F, T, 64, 128>(d, a...);
  if (d.head_dim == 128 && d.sel_dim == 64) return by_group<F, T, 128, 64>(d, a...);
  if (d.head_dim == 128 && d.sel_dim == 128) return by_group<F, T, 128, 128>(d, a...);
  return fail(SAS_ERR_UNSUPPORTED, "select: d=%d d_sel=%d", d.head_dim, d.sel_dim);
}

template <template <typename, int, int, int> class F, typename... A>
static sas_status by_type(const sas_dims& d, A... a) {
  if (d.dtype == SAS_BF16) return by_dims<F, uint16_t>(d, a...);
  return by_dims<F, float>(d, a...);
}

sas_status launch_select_decode(const sas_dims& d, const void* q, const int32_t* seq_lens,
                                const float* Wq, const float* summ, int32_t* idx, float* log_gate,
                                float* score_lse, float* scores, void* ws, hipStream_t st) {
  return by_type<SelDecode>(d, q, seq_lens, Wq, summ, idx, log_gate, score_lse, scores, ws, st);
}

sas_status launch_select_decode_chunks(const sas_dims& d, const void* q, const int32_t* seq_lens,
                                       const float* Wq, const float* summ, const void* K,
                                       const float* Wk, KvPages pg, int32_t* idx,
                                       float* log_gate, float* score_lse, void* ws,
                                       hipStream_t st, int* dec_cnt) {
  return by_type<SelDecodeChunks>(d, q, seq_lens, Wq, summ, K, Wk, pg, idx, log_gate, score_lse,
                                  static_cast<float*>(nullptr), ws, st, dec_cnt);
}

sas_status launch_select_tiles(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                               const float* summ, int32_t* idx, float* log_gate,
                               float* score_lse, float* scores, hipStream_t st) {
  return by_type<SelTiles>(d, Q, q_len, Wq, summ, idx, log_gate, score_lse, scores, st);
}

sas_status launch_select_queries(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                                 const float* summ, int32_t* idx, float* log_gate,
                                 float* score_lse, float* scores, hipStream_t st) {
  return by_type<SelQueries>(d, Q, q_len, Wq, summ, idx, log_gate, score_lse, scores, st);
}

}  // namespace sas
