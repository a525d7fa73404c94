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
//   3. one thread per weight: the two sums above.
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
    float a0 = 0.f, a1 = 0.f;
    int m = 0;
    for (; m + 1 < C; m += 2) {
      a0 = fmaf(sc[m], srow[static_cast<size_t>(m) * DS + tid], a0);
      a1 = fmaf(sc[m + 1], srow[static_cast<size_t>(m + 1) * DS + tid], a1);
    }
    if (m < C) a0 = fmaf(sc[m], srow[static_cast<size_t>(m) * DS + tid], a0);
    rd[tid] = a0 + a1;
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
    float e0 = 0.f, e1 = 0.f;
    int t = m + 1;
    for (; t + 1 < rows; t += 2) {
      const size_t r0 = grp * rows + t;
      e0 = fmaf(ds_ws[r0 * c_max + m], rowdat[r0 * SelRow<D, DS>::kFloats + DS + D + tid], e0);
      e1 = fmaf(ds_ws[(r0 + 1) * c_max + m],
                rowdat[(r0 + 1) * SelRow<D, DS>::kFloats + DS + D + tid], e1);
    }
    if (t < rows) {
      const size_t r0 = grp * rows + t;
      e0 = fmaf(ds_ws[r0 * c_max + m], rowdat[r0 * SelRow<D, DS>::kFloats + DS + D + tid], e0);
    }
    bd[tid] = e0 + e1;
  }
}

// dWq[j][c] (blockIdx.y == 0) or dWk[j][c] (blockIdx.y == 1), row j =
// blockIdx.x, column c = threadIdx.x.
template <int D, int DS>
__global__ void __launch_bounds__(D)
selector_bwd_weights_kernel(int n_groups, int rows, const float* __restrict__ rowdat,
                            const float* __restrict__ blkdat, float* __restrict__ dWq,
                            float* __restrict__ dWk) {
  const int j = blockIdx.x, c = threadIdx.x;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  if (blockIdx.y == 0) {
    constexpr int F = SelRow<D, DS>::kFloats;
    const int n = n_groups * rows;
    for (int x = 0; x < n; ++x) a[x & 3] = fmaf(rowdat[x * F + j], rowdat[x * F + DS + c], a[x & 3]);
    dWq[j * D + c] = ((a[0] + a[1]) + (a[2] + a[3])) * (1.0f / sqrtf(static_cast<float>(DS)));
  } else {
    constexpr int F = SelBlk<D, DS>::kFloats;
    for (int g = 0; g < n_groups; ++g)
      for (int m = 0; m + 1 < rows; ++m) {
        const int x = g * rows + m;
        a[m & 3] = fmaf(blkdat[x * F + j], blkdat[x * F + DS + c], a[m & 3]);
      }
    dWk[j * D + c] = (a[0] + a[1]) + (a[2] + a[3]);
  }
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: ds [B*Hkv*rows*c_max] | rowdat [B*Hkv*rows*(2DS+D)] | blkdat [B*Hkv*rows*(DS+D)]
size_t selector_bwd_ws_bytes(const sas_dims& d, int q_len) {
  const size_t rows = cdiv(q_len, kBlock);
  const size_t grp = static_cast<size_t>(d.batch) * d.n_kv_heads;
  const size_t c_max = d.t_max / kBlock;
  return align256(grp * rows * c_max * sizeof(float)) +
         align256(grp * rows * (2 * d.sel_dim + d.head_dim) * sizeof(float)) +
         grp * rows * (d.sel_dim + d.head_dim) * sizeof(float);
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
  hipLaunchKernelGGL((selector_bwd_weights_kernel<D, DS>), dim3(DS, 2), dim3(D), 0, st,
                     static_cast<int>(grp), rows, rowdat, blkdat, dWq, dWk);
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

sas_status launch_selector_bwd(const sas_dims& d, const void* Q, int q_len, const void* K,
                               const float* Wq, const float* summ, const int32_t* idx,
                               const float* score_lse, const float* dlg, float* ds, float* dWq,
                               float* dWk, void* ws, hipStream_t st) {
  if (d.dtype == SAS_BF16)
    return sbwd_by_dims<uint16_t>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
  return sbwd_by_dims<float>(d, Q, q_len, K, Wq, summ, idx, score_lse, dlg, ds, dWq, dWk, ws, st);
}

}  // namespace sas
