// Backward of the selector into its own weights (SAS close reading 2.2, gate
// equation; 2.3, eq. 8 for the sparse training scope; 2.4 and the training
// description after it: the loss reaches the selector through the log-gate).
//
// For one tile row t of group r, with C = t history blocks, the scores
//   s_m = u . summ_m,   u = Wq_sel qbar / sqrt(d_sel),   summ_m = Wk_sel kbar_m
// (qbar: mean of the tile's queries over the group's heads; kbar_m: mean key
// of block m) and the gate log g = s - LSE(s), the gradients of the selected
// slots' log-gates give, over every history block,
//   ds_m = dlog g_m [m selected] - g_m * sum_slots dlog g,
// and then
//   dWq_sel = sum_rows a_row qbar_row^T / sqrt(d_sel),  a_row = sum_m ds_m summ_m,
//   dWk_sel = sum_(group, m) e_m kbar_m^T,              e_m = sum_rows ds_(row, m) u_row.
// Three kernels, no atomics, fixed summation orders (bitwise reproducible):
//   1. one workgroup per row: pooled query, scores (the selection's own code),
//      ds, a_row;
//   2. one workgroup per history block: kbar_m and e_m (a sum over the rows
//      that see the block);
//   3. the two sums above: chunk partials of the outer products, then their
//      sum in chunk order.
#include "sas_device.h"
#include "sas_internal.h"
#include "sas_select_dev.h"

namespace sas {

// Per-row state kept in the workspace: a_row [DS], qbar [D], u [DS].
template <int D, int DS> struct SelRow { static constexpr int kFloats = 2 * DS + D; };
// Per-block state: e_m [DS], kbar_m [D].
template <int D, int DS> struct SelBlk { static constexpr int kFloats = DS + D; };

template <typename T, int D, int DS, int G>
__global__ void __launch_bounds__(kSelThreads)
selector_bwd_rows_kernel(const T* __restrict__ Q, int q_len, const float* __restrict__ Wq,
                         const float* __restrict__ summ, const int32_t* __restrict__ idx,
                         const float* __restrict__ score_lse, const float* __restrict__ dlg,
                         int Hkv, int c_max, int rows, int k, float* __restrict__ ds_ws,
                         float* __restrict__ ds_out, float* __restrict__ rowdat) {
  __shared__ float qpart[kSelThreads / (D / Vec16<T>::N)][D];
  __shared__ float qm[D];
  __shared__ float qs[DS];
  __shared__ float sc[kMaxTileRows];
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

  // ds_m = -g_m * (sum of the row's log-gate gradients), then the selected
  // blocks' own terms (block indices are distinct within a row)
  float tot = 0.f;
  for (int slot = 0; slot < k; ++slot)
    if (idx[row * k + slot] >= 0) tot += dlg[row * k + slot];
  const float lse = score_lse[row];
  for (int m = tid; m < C; m += kSelThreads) sc[m] = -expf(sc[m] - lse) * tot;
  __syncthreads();
  if (tid < k) {
    const int m = idx[row * k + tid];
    if (m >= 0) sc[m] += dlg[row * k + tid];
  }
  __syncthreads();
  for (int m = tid; m < C; m += kSelThreads) {
    ds_ws[row * c_max + m] = sc[m];
    if (ds_out) ds_out[row * c_max + m] = sc[m];
  }
  // a_row = sum_m ds_m summ_m; qbar and u for the weight sums
  float* rd = rowdat + row * SelRow<D, DS>::kFloats;
  if (tid < DS) {
    // 8 independent accumulators: eight summary loads in flight at a time
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int m = 0;
    for (; m + 7 < C; m += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        a[u] = fmaf(sc[m + u], srow[static_cast<size_t>(m + u) * DS + tid], a[u]);
    }
    for (; m < C; ++m) a[0] = fmaf(sc[m], srow[static_cast<size_t>(m) * DS + tid], a[0]);
    rd[tid] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    rd[DS + D + tid] = qs[tid];
  }
  if (tid < D) rd[DS + tid] = qm[tid];
}

template <typename T, int D, int DS>
__global__ void __launch_bounds__(kSelThreads)
selector_bwd_blocks_kernel(const T* __restrict__ K, int Hkv, int t_max, int c_max, int rows,
                           const float* __restrict__ ds_ws, const float* __restrict__ rowdat,
                           float* __restrict__ blkdat) {
  __shared__ float part[kSelThreads / D > 0 ? kSelThreads / D : 1][D];
  const int m = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const size_t grp = static_cast<size_t>(b) * Hkv + r;
  float* bd = blkdat + (grp * rows + m) * SelBlk<D, DS>::kFloats;
  // kbar_m: thread (c, q) sums tokens q, q + NQ, ... of column c
  constexpr int NQ = kSelThreads / D;
  {
    const int c = tid % D, q = tid / D;
    const T* kb = K + (grp * t_max + static_cast<size_t>(m) * kBlock) * D + c;
    float a = 0.f;
    for (int j = q; j < kBlock; j += NQ) a += load_scalar<T>(kb + static_cast<size_t>(j) * D);
    part[q][c] = a;
  }
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
    for (int q = 0; q < NQ; ++q) a += part[q][tid];
    bd[DS + tid] = a * (1.0f / kBlock);
  }
  // e_m = sum over the rows that see block m (tiles t > m) of ds_(t, m) u_t
  if (tid < DS) {
    // 8 independent accumulators: eight rows' loads in flight at a time
    float e[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    constexpr int F = SelRow<D, DS>::kFloats;
    int t = m + 1;
    for (; t + 7 < rows; t += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const size_t r0 = grp * rows + t + u;
        e[u] = fmaf(ds_ws[r0 * c_max + m], rowdat[r0 * F + DS + D + tid], e[u]);
      }
    }
    for (; t < rows; ++t) {
      const size_t r0 = grp * rows + t;
      e[0] = fmaf(ds_ws[r0 * c_max + m], rowdat[r0 * F + DS + D + tid], e[0]);
    }
    bd[tid] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }
}

// The weight sums, in two fixed-order stages.  Stage 1: workgroup (chunk,
// which) adds the outer products of up to kSbChunk entries (rows for dWq,
// history blocks for dWk) into a partial [DS][D] in the workspace; thread
// (c, half) keeps the DS/2 rows j of column c in registers, and the entries'
// vectors are staged in LDS.  Stage 2: one thread per weight adds the
// chunk partials in chunk order.
constexpr int kSbChunk = 16;

template <int D, int DS>
__global__ void __launch_bounds__(2 * D)
selector_bwd_partial_kernel(int n_groups, int rows, const float* __restrict__ rowdat,
                            const float* __restrict__ blkdat, float* __restrict__ partial) {
  constexpr int JH = DS / 2;
  __shared__ float left[kSbChunk][DS];
  __shared__ float right[kSbChunk][D];
  const int which = blockIdx.y, chunk = blockIdx.x;
  const int c = threadIdx.x % D, half = threadIdx.x / D;
  // entries of this chunk: rows (dWq) or history blocks m < rows - 1 (dWk)
  const int per_group = which == 0 ? rows : rows - 1;
  const int n_entries = n_groups * per_group;
  const int e0 = chunk * kSbChunk, ne = min(kSbChunk, n_entries - e0);
  auto entry_ptr = [&](int e) -> const float* {
    const int g = e / per_group, i = e % per_group;
    return which == 0 ? rowdat + (static_cast<size_t>(g) * rows + i) * SelRow<D, DS>::kFloats
                      : blkdat + (static_cast<size_t>(g) * rows + i) * SelBlk<D, DS>::kFloats;
  };
  for (int x = threadIdx.x; x < ne * DS; x += 2 * D) left[x / DS][x % DS] = entry_ptr(e0 + x / DS)[x % DS];
  for (int x = threadIdx.x; x < ne * D; x += 2 * D) right[x / D][x % D] = entry_ptr(e0 + x / D)[DS + x % D];
  __syncthreads();
  float acc[JH];
#pragma unroll
  for (int j = 0; j < JH; ++j) acc[j] = 0.f;
  for (int e = 0; e < ne; ++e) {
    const float rv = right[e][c];   // qbar (dWq) or kbar (dWk)
#pragma unroll
    for (int j = 0; j < JH; ++j) acc[j] = fmaf(left[e][half * JH + j], rv, acc[j]);
  }
  float* out = partial + ((static_cast<size_t>(which) * gridDim.x + chunk) * DS + half * JH) * D + c;
#pragma unroll
  for (int j = 0; j < JH; ++j) out[static_cast<size_t>(j) * D] = acc[j];
}

template <int D, int DS>
__global__ void __launch_bounds__(D)
selector_bwd_weights_kernel(int n_chunks, const float* __restrict__ partial,
                            float* __restrict__ dWq, float* __restrict__ dWk) {
  const int which = blockIdx.y, j = blockIdx.x, c = threadIdx.x;
  const float* src = partial + (static_cast<size_t>(which) * n_chunks * DS + j) * D + c;
  float a = 0.f;
  // chunk order; unrolled so that 16 chunks' loads are in flight at a time
#pragma unroll 16
  for (int ch = 0; ch < n_chunks; ++ch) a += src[static_cast<size_t>(ch) * DS * D];
  if (which == 0) dWq[j * D + c] = a * (1.0f / sqrtf(static_cast<float>(DS)));
  else dWk[j * D + c] = a;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int sb_chunks(const sas_dims& d, int rows) {
  return cdiv(d.batch * d.n_kv_heads * rows, kSbChunk);
}

// workspace: ds [B*Hkv*rows*c_max] | rowdat [B*Hkv*rows*(2DS+D)] |
//            blkdat [B*Hkv*rows*(DS+D)] | partial [2][chunks][DS][D]
size_t selector_bwd_ws_bytes(const sas_dims& d, int q_len) {
  const int rows = cdiv(q_len, kBlock);
  const size_t grp = static_cast<size_t>(d.batch) * d.n_kv_heads;
  const size_t c_max = d.t_max / kBlock;
  return align256(grp * rows * c_max * sizeof(float)) +
         align256(grp * rows * (2 * d.sel_dim + d.head_dim) * sizeof(float)) +
         align256(grp * rows * (d.sel_dim + d.head_dim) * sizeof(float)) +
         2 * static_cast<size_t>(sb_chunks(d, rows)) * d.sel_dim * d.head_dim * sizeof(float);
}

template <typename T, int D, int DS, int G>
static sas_status launch_sbwd(const sas_dims& d, const void* Q, int q_len, const void* K,
                              const float* Wq, const float* summ, const int32_t* idx,
                              const float* score_lse, const float* dlg, float* ds,
                              float* dWq, float* dWk, void* ws, hipStream_t st) {
  const int rows = cdiv(q_len, kBlock);
  const size_t grp = static_cast<size_t>(d.batch) * d.n_kv_heads;
  const int c_max = d.t_max / kBlock;
  char* w = static_cast<char*>(ws);
  float* ds_ws = reinterpret_cast<float*>(w);
  w += align256(grp * rows * c_max * sizeof(float));
  float* rowdat = reinterpret_cast<float*>(w);
  w += align256(grp * rows * SelRow<D, DS>::kFloats * sizeof(float));
  float* blkdat = reinterpret_cast<float*>(w);
  w += align256(grp * rows * SelBlk<D, DS>::kFloats * sizeof(float));
  float* partial = reinterpret_cast<float*>(w);
  const int n_chunks = sb_chunks(d, rows);
  hipLaunchKernelGGL((selector_bwd_rows_kernel<T, D, DS, G>), dim3(rows, d.n_kv_heads, d.batch),
                     dim3(kSelThreads), 0, st, static_cast<const T*>(Q), q_len, Wq, summ, idx,
                     score_lse, dlg, d.n_kv_heads, c_max, rows, d.top_k, ds_ws, ds, rowdat);
  sas_status s = check_launch("selector_bwd_rows");
  if (s != SAS_OK) return s;
  if (rows > 1) {
    hipLaunchKernelGGL((selector_bwd_blocks_kernel<T, D, DS>),
                       dim3(rows - 1, d.n_kv_heads, d.batch), dim3(kSelThreads), 0, st,
                       static_cast<const T*>(K), d.n_kv_heads, d.t_max, c_max, rows, ds_ws,
                       rowdat, blkdat);
    s = check_launch("selector_bwd_blocks");
    if (s != SAS_OK) return s;
  }
  // dWk's chunks beyond its entries (grp * (rows - 1) of them) hold zeros
  hipLaunchKernelGGL((selector_bwd_partial_kernel<D, DS>), dim3(n_chunks, 2), dim3(2 * D), 0, st,
                     static_cast<int>(grp), rows, rowdat, blkdat, partial);
  s = check_launch("selector_bwd_partial");
  if (s != SAS_OK) return s;
  hipLaunchKernelGGL((selector_bwd_weights_kernel<D, DS>), dim3(DS, 2), dim3(D), 0, st, n_chunks,
                     partial, dWq, dWk);
  return check_launch("selector_bwd_weights");
}

template <typename T, int D, int DS>
static sas_status sbwd_by_group(const sas_dims& d, const void* Q, int q_len, const void* K,
                                const float* Wq, const float* summ, const int32_t* idx,
                                const float* score_lse, const float* dlg, float* ds, float* dWq,
                                float* dWk, void* ws, hipStream_t st) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_sbwd<T, D, DS, 1>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
    case 2: return launch_sbwd<T, D, DS, 2>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
    case 4: return launch_sbwd<T, D, DS, 4>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
    case 8: return launch_sbwd<T, D, DS, 8>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  }
  return fail(SAS_ERR_UNSUPPORTED, "selector backward: group size");
}

template <typename T>
static sas_status sbwd_by_dims(const sas_dims& d, const void* Q, int q_len, const void* K,
                               const float* Wq, const float* summ, const int32_t* idx,
                               const float* score_lse, const float* dlg, float* ds, float* dWq,
                               float* dWk, void* ws, hipStream_t st) {
  if (d.head_dim == 128 && d.sel_dim == 128)
    return sbwd_by_group<T, 128, 128>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  if (d.head_dim == 128)
    return sbwd_by_group<T, 128, 64>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  if (d.sel_dim == 128)
    return sbwd_by_group<T, 64, 128>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  return sbwd_by_group<T, 64, 64>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
}

// ---------------------------------------------------------- query rows ---
// Per-query rows (one selection per query): row (i, r) has C = i / 64 blocks
// and the pooled query qbar_i (mean of query i over the group's heads).  A
// block is seen by up to S rows, so instead of forming e_m = sum_rows ds u
// per block the gradients go through one D x D matrix:
//   h_i = sum_m ds_(i,m) kbar_m,   H = sum_rows h_i qbar_i^T,
//   dWq_sel = Wk_sel H / sqrt(d_sel)      (= sum_rows a_i qbar_i^T / sqrt(d_sel),
//                                          a_i = sum_m ds_(i,m) Wk_sel kbar_m),
//   dWk_sel = Wq_sel H^T / sqrt(d_sel)    (= sum_m e_m kbar_m^T,
//                                          e_m = sum_rows ds_(i,m) Wq_sel qbar_i / sqrt(d_sel)).
// Four kernels, fixed summation orders (bitwise reproducible): mean keys;
// one workgroup per 32 rows (scores, ds, h); chunked outer-product partials
// of H; H and the two small products.
constexpr int kQsbRows = 32;      // rows per workgroup of the row kernel
constexpr int kQsbChunk = 64;     // blocks per scoring pass
constexpr int kQsbPartRows = 512;   // rows per H partial

template <typename T, int D>
__global__ void __launch_bounds__(kSelThreads)
qsb_kbar_kernel(const T* __restrict__ K, int Hkv, int t_max, int c_max, int n_blk,
                float* __restrict__ kbar) {
  __shared__ float part[kSelThreads / D][D];
  const int m = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const size_t grp = static_cast<size_t>(b) * Hkv + r;
  constexpr int NQ = kSelThreads / D;
  const int c = tid % D, q = tid / D;
  const T* kb = K + (grp * t_max + static_cast<size_t>(m) * kBlock) * D + c;
  float a = 0.f;
  for (int j = q; j < kBlock; j += NQ) a += load_scalar<T>(kb + static_cast<size_t>(j) * D);
  part[q][c] = a;
  __syncthreads();
  if (tid < D) {
    float x = 0.f;
    for (int qq = 0; qq < NQ; ++qq) x += part[qq][tid];
    kbar[(grp * c_max + m) * D + tid] = x * (1.0f / kBlock);
  }
  (void)n_blk;
}

template <typename T, int D, int DS, int G>
__global__ void __launch_bounds__(kSelThreads)
qsb_rows_kernel(const T* __restrict__ Q, int q_len, const float* __restrict__ Wq,
                const float* __restrict__ summ, const float* __restrict__ kbar,
                const int32_t* __restrict__ idx, const float* __restrict__ score_lse,
                const float* __restrict__ dlg, int Hkv, int c_max, int k,
                float* __restrict__ ds_out, float* __restrict__ rowdat) {
  constexpr int QS = D + 4, US = DS + 4;
  constexpr int MS = (D > DS ? D : DS) + 4;   // staging row stride (summaries, then mean keys)
  __shared__ __attribute__((aligned(16))) float qb[kQsbRows * QS];    // pooled queries
  __shared__ __attribute__((aligned(16))) float u[kQsbRows * US];     // their projections
  __shared__ __attribute__((aligned(16))) float stg[kQsbChunk * MS];
  __shared__ float sc[kQsbRows][kQsbChunk + 1];                        // ds of the chunk
  __shared__ float s_lse[kQsbRows], s_tot[kQsbRows];

  const int t = blockIdx.x >> 1, r = blockIdx.y, b = blockIdx.z;
  const int i0 = t * kBlock + (blockIdx.x & 1) * kQsbRows;
  const int nq = min(kQsbRows, q_len - i0);
  if (nq <= 0) return;   // second half of a short last tile (workgroup-uniform)
  const int C = t;
  const int tid = threadIdx.x;
  const size_t grp = static_cast<size_t>(b) * Hkv + r;
  const size_t row0 = grp * q_len + i0;

  // pooled queries (G heads summed in head order, times 1/G)
  {
    constexpr int EPL = Vec16<T>::N, LPR = D / EPL;
    for (int x = tid; x < kQsbRows * LPR; x += kSelThreads) {
      const int q = x / LPR, col = x % LPR;
      float acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
      if (q < nq) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const T* src = Q + ((grp * G + h) * q_len + i0 + q) * D + col * EPL;
          float f[EPL];
          Vec16<T>::unpack(*reinterpret_cast<const uint4*>(src), f);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] += f[e];
        }
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) qb[q * QS + col * EPL + e] = acc[e] * (1.0f / G);
    }
  }
  if (tid < kQsbRows) {
    float tot = 0.f;
    if (tid < nq)
      for (int slot = 0; slot < k; ++slot)
        if (idx[(row0 + tid) * k + slot] >= 0) tot += dlg[(row0 + tid) * k + slot];
    s_tot[tid] = tot;
    s_lse[tid] = tid < nq ? score_lse[row0 + tid] : 0.f;
  }
  __syncthreads();
  // u = Wq qbar / sqrt(DS)
  {
    constexpr int NQG = kSelThreads / DS, NE = kQsbRows / NQG;
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
        const float4 a = *reinterpret_cast<const float4*>(&qb[(qg + NQG * e) * QS + 4 * j4]);
        acc[e] += x.x * a.x + x.y * a.y + x.z * a.z + x.w * a.w;
      }
    }
    const float inv = 1.0f / sqrtf(static_cast<float>(DS));
#pragma unroll
    for (int e = 0; e < NE; ++e) u[(qg + NQG * e) * US + c] = acc[e] * inv;
  }
  // h: thread (hq, hc) keeps row hq's channels 16 hc .. 16 hc + 15 (D = 128)
  // or 8 hc .. 8 hc + 7 (D = 64)
  constexpr int HC = D / 8;   // channels per thread
  const int hq = tid >> 3, hc = tid & 7;
  float h[HC];
#pragma unroll
  for (int e = 0; e < HC; ++e) h[e] = 0.f;

  const float* srow = summ + grp * static_cast<size_t>(c_max) * DS;
  const float* krow = kbar + grp * static_cast<size_t>(c_max) * D;
  for (int c0 = 0; c0 < C; c0 += kQsbChunk) {
    const int nb = min(kQsbChunk, C - c0);
    __syncthreads();   // u written / the previous chunk's readers of stg and sc are done
    for (int x = tid; x < kQsbChunk * (DS / 4); x += kSelThreads) {
      const int m = x / (DS / 4), c4 = x % (DS / 4);
      const float4 v = m < nb ? *reinterpret_cast<const float4*>(srow + static_cast<size_t>(c0 + m) * DS + 4 * c4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&stg[m * MS + 4 * c4]) = v;
    }
    __syncthreads();
    // ds = -g * (sum of the row's log-gate gradients) over the chunk's blocks
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
        for (int x = 0; x < 4; ++x) sv[x] = *reinterpret_cast<const float4*>(&stg[(tm + 16 * x) * MS + 4 * j4]);
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
          sc[q][m] = (q < nq && m < nb) ? -expf(acc[a][x] - s_lse[q]) * s_tot[q] : 0.f;
        }
    }
    __syncthreads();
    // the selected blocks' own terms (block indices are distinct within a row)
    for (int x = tid; x < nq * k; x += kSelThreads) {
      const int q = x / k;
      const int m = idx[row0 * k + x];
      if (m >= c0 && m < c0 + nb) sc[q][m - c0] += dlg[row0 * k + x];
    }
    __syncthreads();
    if (ds_out)
      for (int x = tid; x < nq * nb; x += kSelThreads) {
        const int q = x / nb, m = x % nb;
        ds_out[(row0 + q) * c_max + c0 + m] = sc[q][m];
      }
    // stage the chunk's mean keys (the scores are done with the summaries)
    for (int x = tid; x < kQsbChunk * (D / 4); x += kSelThreads) {
      const int m = x / (D / 4), c4 = x % (D / 4);
      const float4 v = m < nb ? *reinterpret_cast<const float4*>(krow + static_cast<size_t>(c0 + m) * D + 4 * c4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(&stg[m * MS + 4 * c4]) = v;
    }
    __syncthreads();
    // h += ds kbar, blocks in order
#pragma unroll 2
    for (int m = 0; m < nb; ++m) {
      const float w = sc[hq][m];
#pragma unroll
      for (int e4 = 0; e4 < HC / 4; ++e4) {
        const float4 kv = *reinterpret_cast<const float4*>(&stg[m * MS + HC * hc + 4 * e4]);
        h[4 * e4 + 0] = fmaf(w, kv.x, h[4 * e4 + 0]);
        h[4 * e4 + 1] = fmaf(w, kv.y, h[4 * e4 + 1]);
        h[4 * e4 + 2] = fmaf(w, kv.z, h[4 * e4 + 2]);
        h[4 * e4 + 3] = fmaf(w, kv.w, h[4 * e4 + 3]);
      }
    }
  }
  // rowdat: h [D], qbar [D] per row (rows past q_len are not stored)
  if (hq < nq) {
    float* rd = rowdat + (row0 + hq) * (2 * D);
#pragma unroll
    for (int e = 0; e < HC; ++e) rd[HC * hc + e] = h[e];
    for (int e = 0; e < HC; ++e) rd[D + HC * hc + e] = qb[hq * QS + HC * hc + e];
  }
}

// Partial of H = sum_rows h qbar^T over kQsbPartRows rows, staged 64 at a
// time; thread (ti, tj) of a 16 x 16 grid keeps the TR x TR block of H at
// rows TR ti.., columns TR tj.. in registers, so each staged value feeds TR
// multiply-adds.
template <int D>
__global__ void __launch_bounds__(256)
qsb_partial_kernel(size_t n_rows, const float* __restrict__ rowdat, float* __restrict__ partial) {
  constexpr int TR = D / 16;
  __shared__ __attribute__((aligned(16))) float left[64][D];
  __shared__ __attribute__((aligned(16))) float right[64][D];
  const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
  const size_t e_begin = static_cast<size_t>(blockIdx.x) * kQsbPartRows;
  const size_t e_end = e_begin + kQsbPartRows < n_rows ? e_begin + kQsbPartRows : n_rows;
  float acc[TR][TR];
#pragma unroll
  for (int a = 0; a < TR; ++a)
#pragma unroll
    for (int c = 0; c < TR; ++c) acc[a][c] = 0.f;
  for (size_t e0 = e_begin; e0 < e_end; e0 += 64) {
    const int ne = static_cast<int>(e_end - e0 < 64 ? e_end - e0 : 64);
    __syncthreads();
    for (int x = tid; x < ne * (D / 4); x += 256) {
      const int e = x / (D / 4), c4 = x % (D / 4);
      const float* rd = rowdat + (e0 + e) * (2 * D);
      *reinterpret_cast<float4*>(&left[e][4 * c4]) = *reinterpret_cast<const float4*>(rd + 4 * c4);
      *reinterpret_cast<float4*>(&right[e][4 * c4]) = *reinterpret_cast<const float4*>(rd + D + 4 * c4);
    }
    __syncthreads();
    for (int e = 0; e < ne; ++e) {
      float l[TR], rr[TR];
#pragma unroll
      for (int a4 = 0; a4 < TR / 4; ++a4) {
        const float4 x = *reinterpret_cast<const float4*>(&left[e][TR * ti + 4 * a4]);
        const float4 y = *reinterpret_cast<const float4*>(&right[e][TR * tj + 4 * a4]);
        l[4 * a4] = x.x; l[4 * a4 + 1] = x.y; l[4 * a4 + 2] = x.z; l[4 * a4 + 3] = x.w;
        rr[4 * a4] = y.x; rr[4 * a4 + 1] = y.y; rr[4 * a4 + 2] = y.z; rr[4 * a4 + 3] = y.w;
      }
#pragma unroll
      for (int a = 0; a < TR; ++a)
#pragma unroll
        for (int c = 0; c < TR; ++c) acc[a][c] = fmaf(l[a], rr[c], acc[a][c]);
    }
  }
  float* out = partial + static_cast<size_t>(blockIdx.x) * D * D;
#pragma unroll
  for (int a = 0; a < TR; ++a)
#pragma unroll
    for (int c = 0; c < TR; ++c) out[(TR * ti + a) * D + TR * tj + c] = acc[a][c];
}

// H = sum of the partials in chunk order.
template <int D>
__global__ void __launch_bounds__(D)
qsb_sum_kernel(int n_chunks, const float* __restrict__ partial, float* __restrict__ H) {
  const int x = blockIdx.x, c = threadIdx.x;
  float a = 0.f;
  // chunk order; unrolled so that 16 chunks' loads are in flight at a time
#pragma unroll 16
  for (int ch = 0; ch < n_chunks; ++ch) a += partial[(static_cast<size_t>(ch) * D + x) * D + c];
  H[x * D + c] = a;
}

// dWq[j][c] = sum_x Wk[j][x] H[x][c] / sqrt(DS); dWk[j][c] = sum_x Wq[j][x] H[c][x] / sqrt(DS).
template <int D, int DS>
__global__ void __launch_bounds__(D)
qsb_weights_kernel(const float* __restrict__ Wq, const float* __restrict__ Wk,
                   const float* __restrict__ H, float* __restrict__ dWq, float* __restrict__ dWk) {
  const int which = blockIdx.y, j = blockIdx.x, c = threadIdx.x;
  const float inv = 1.0f / sqrtf(static_cast<float>(DS));
  float a = 0.f;
  if (which == 0) {
    for (int x = 0; x < D; ++x) a = fmaf(Wk[j * D + x], H[x * D + c], a);
    dWq[j * D + c] = a * inv;
  } else {
    for (int x = 0; x < D; ++x) a = fmaf(Wq[j * D + x], H[c * D + x], a);
    dWk[j * D + c] = a * inv;
  }
}

// workspace: kbar [grp * c_max * D] | rowdat [grp * q_len * 2D] |
//            partial [chunks * D * D] | H [D * D]
static size_t qsb_chunks(const sas_dims& d, int q_len) {
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads * q_len;
  return (rows + kQsbPartRows - 1) / kQsbPartRows;
}
size_t selector_bwd_queries_ws_bytes(const sas_dims& d, int q_len) {
  const size_t grp = static_cast<size_t>(d.batch) * d.n_kv_heads;
  const size_t c_max = d.t_max / kBlock, D = d.head_dim;
  return align256(grp * c_max * D * sizeof(float)) +
         align256(grp * q_len * 2 * D * sizeof(float)) +
         align256(qsb_chunks(d, q_len) * D * D * sizeof(float)) + D * D * sizeof(float);
}

template <typename T, int D, int DS, int G>
static sas_status launch_qsb(const sas_dims& d, const void* Q, int q_len, const void* K,
                             const float* Wq, const float* Wk, const float* summ,
                             const int32_t* idx, const float* score_lse, const float* dlg,
                             float* ds, float* dWq, float* dWk, void* ws, hipStream_t st) {
  const size_t grp = static_cast<size_t>(d.batch) * d.n_kv_heads;
  const int c_max = d.t_max / kBlock;
  const int n_tiles = cdiv(q_len, kBlock);
  char* w = static_cast<char*>(ws);
  float* kbar = reinterpret_cast<float*>(w);
  w += align256(grp * c_max * D * sizeof(float));
  float* rowdat = reinterpret_cast<float*>(w);
  w += align256(grp * q_len * 2 * D * sizeof(float));
  float* partial = reinterpret_cast<float*>(w);
  const int n_chunks = static_cast<int>(qsb_chunks(d, q_len));
  w += align256(static_cast<size_t>(n_chunks) * D * D * sizeof(float));
  float* H = reinterpret_cast<float*>(w);
  if (n_tiles > 1) {   // history blocks 0 .. n_tiles - 2
    hipLaunchKernelGGL((qsb_kbar_kernel<T, D>), dim3(n_tiles - 1, d.n_kv_heads, d.batch),
                       dim3(kSelThreads), 0, st, static_cast<const T*>(K), d.n_kv_heads, d.t_max,
                       c_max, n_tiles - 1, kbar);
    sas_status s = check_launch("selector_bwd_queries_kbar");
    if (s != SAS_OK) return s;
  }
  hipLaunchKernelGGL((qsb_rows_kernel<T, D, DS, G>), dim3(2 * n_tiles, d.n_kv_heads, d.batch),
                     dim3(kSelThreads), 0, st, static_cast<const T*>(Q), q_len, Wq, summ, kbar,
                     idx, score_lse, dlg, d.n_kv_heads, c_max, d.top_k, ds, rowdat);
  sas_status s = check_launch("selector_bwd_queries_rows");
  if (s != SAS_OK) return s;
  hipLaunchKernelGGL((qsb_partial_kernel<D>), dim3(n_chunks), dim3(256), 0, st,
                     grp * static_cast<size_t>(q_len), rowdat, partial);
  s = check_launch("selector_bwd_queries_partial");
  if (s != SAS_OK) return s;
  hipLaunchKernelGGL((qsb_sum_kernel<D>), dim3(D), dim3(D), 0, st, n_chunks, partial, H);
  s = check_launch("selector_bwd_queries_sum");
  if (s != SAS_OK) return s;
  hipLaunchKernelGGL((qsb_weights_kernel<D, DS>), dim3(DS, 2), dim3(D), 0, st, Wq, Wk, H, dWq,
                     dWk);
  return check_launch("selector_bwd_queries_weights");
}

template <typename T, int D, int DS>
static sas_status qsb_by_group(const sas_dims& d, const void* Q, int q_len, const void* K,
                               const float* Wq, const float* Wk, const float* summ,
                               const int32_t* idx, const float* score_lse, const float* dlg,
                               float* ds, float* dWq, float* dWk, void* ws, hipStream_t st) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_qsb<T, D, DS, 1>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
    case 2: return launch_qsb<T, D, DS, 2>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
    case 4: return launch_qsb<T, D, DS, 4>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
    case 8: return launch_qsb<T, D, DS, 8>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  }
  return fail(SAS_ERR_UNSUPPORTED, "selector backward: group size");
}

template <typename T>
static sas_status qsb_by_dims(const sas_dims& d, const void* Q, int q_len, const void* K,
                              const float* Wq, const float* Wk, const float* summ,
                              const int32_t* idx, const float* score_lse, const float* dlg,
                              float* ds, float* dWq, float* dWk, void* ws, hipStream_t st) {
  if (d.head_dim == 128 && d.sel_dim == 128)
    return qsb_by_group<T, 128, 128>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  if (d.head_dim == 128)
    return qsb_by_group<T, 128, 64>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  if (d.sel_dim == 128)
    return qsb_by_group<T, 64, 128>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  return qsb_by_group<T, 64, 64>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
}

sas_status launch_selector_bwd_queries(const sas_dims& d, const void* Q, int q_len,
                                       const void* K, const float* Wq, const float* Wk,
                                       const float* summ, const int32_t* idx,
                                       const float* score_lse, const float* dlg, float* ds,
                                       float* dWq, float* dWk, void* ws, hipStream_t st) {
  if (d.dtype == SAS_BF16)
    return qsb_by_dims<uint16_t>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  return qsb_by_dims<float>(d, Q, q_len, K, Wq, Wk, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
}

sas_status launch_selector_bwd(const sas_dims& d, const void* Q, int q_len, const void* K,
                               const float* Wq, const float* summ, const int32_t* idx,
                               const float* score_lse, const float* dlg, float* ds, float* dWq,
                               float* dWk, void* ws, hipStream_t st) {
  if (d.dtype == SAS_BF16)
    return sbwd_by_dims<uint16_t>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  return sbwd_by_dims<float>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
}

}  // namespace sas
