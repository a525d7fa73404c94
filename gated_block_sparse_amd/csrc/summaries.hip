// Block summaries (SAS close reading 2.1, block summary, mean-pooled):
//   summ[b,r,m,:] = Wk_sel . mean_{j in block m} K[b,r,j,:]
// Pooling first and projecting once per block is the same linear map as
// projecting every key and pooling, at 1/64 of the arithmetic.
//
// HBM-bound: every key of a summarised block is read once.  One workgroup
// (4 waves) handles kSumBlocks consecutive blocks of one (b, r): each wave
// streams whole 64-token blocks with 16-byte loads (a row is LPR lanes, so a
// load instruction covers 64/LPR full rows, fully coalesced), sums its rows
// in registers and finishes the column sums with a butterfly inside the wave.
// For the projection each thread keeps a slice of one row of Wk_sel in
// registers (loaded while the key loads are in flight) and SPLIT adjacent
// lanes combine their slices of one output with a butterfly.
#include "sas_device.h"
#include "sas_internal.h"
#include "sas_summary_dev.h"

namespace sas {

constexpr int kSumBlocks = 16;   // blocks per workgroup

template <typename T, int D, int DS>
__global__ void __launch_bounds__(kSumThreads)
block_summaries_kernel(const T* __restrict__ K, const int32_t* __restrict__ seq_lens,
                       const float* __restrict__ Wk, int blk_begin, int blk_end, int Hkv,
                       int t_max, int c_max, KvPages pg, float* __restrict__ summ) {
  using WS = WkSlice<D, DS>;
  __shared__ float mean[kSumBlocks][D];

  const int b = blockIdx.z, r = blockIdx.y;
  const int first = blk_begin + blockIdx.x * kSumBlocks;
  const int len = clamp_len(seq_lens[b], t_max);
  const int C = (len - 1) / kBlock;
  const int last = min(min(blk_end, C), first + kSumBlocks);  // exclusive
  if (first >= last) return;
  const int nblk = last - first;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  WS ws;
  ws.load(Wk, tid);

  for (int jb = wave; jb < nblk; jb += 4) {
    BlockMean<T, D> bm;
    bm.load(K + kv_block_row(pg, b, r, first + jb, Hkv, t_max) * D, lane);
    bm.reduce(lane, mean[jb]);
  }
  __syncthreads();

  float* dst = summ + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(c_max) * DS;
  const int j = tid / WS::SPLIT, part = tid % WS::SPLIT;
  for (int jb = 0; jb < nblk; ++jb) {
    const float a = ws.project(mean[jb], tid);
    if (part == 0) dst[static_cast<size_t>(first + jb) * DS + j] = a;
  }
}

template <typename T, int D, int DS>
static void launch_sum(const sas_dims& d, const void* K, const int32_t* seq_lens, const float* Wk,
                       int blk_begin, int blk_end, float* summ, hipStream_t st, KvPages pg) {
  dim3 grid(cdiv(blk_end - blk_begin, kSumBlocks), d.n_kv_heads, d.batch);
  hipLaunchKernelGGL((block_summaries_kernel<T, D, DS>), grid, dim3(kSumThreads), 0, st,
                     static_cast<const T*>(K), seq_lens, Wk, blk_begin, blk_end, d.n_kv_heads,
                     d.t_max, d.t_max / kBlock, pg, summ);
}

static sas_status sum_any(const sas_dims& d, const void* K, KvPages pg, const int32_t* seq_lens,
                          const float* Wk, int blk_begin, int blk_end, float* summ,
                          hipStream_t st) {
  const bool bf = d.dtype == SAS_BF16;
#define SAS_SUM_CASE(TT, DD, SS)                                                      \
  if (d.head_dim == DD && d.sel_dim == SS) {                                          \
    launch_sum<TT, DD, SS>(d, K, seq_lens, Wk, blk_begin, blk_end, summ, st, pg);     \
    return check_launch("block_summaries");                                           \
  }
  if (bf) {
    SAS_SUM_CASE(uint16_t, 64, 64)
    SAS_SUM_CASE(uint16_t, 64, 128)
    SAS_SUM_CASE(uint16_t, 128, 64)
    SAS_SUM_CASE(uint16_t, 128, 128)
  } else {
    SAS_SUM_CASE(float, 64, 64)
    SAS_SUM_CASE(float, 64, 128)
    SAS_SUM_CASE(float, 128, 64)
    SAS_SUM_CASE(float, 128, 128)
  }
#undef SAS_SUM_CASE
  return fail(SAS_ERR_UNSUPPORTED, "block_summaries: d=%d d_sel=%d", d.head_dim, d.sel_dim);
}

sas_status launch_block_summaries(const sas_dims& d, const void* K, const int32_t* seq_lens,
                                  const float* Wk, int blk_begin, int blk_end, float* summ,
                                  hipStream_t st) {
  return sum_any(d, K, KvPages{nullptr, 0}, seq_lens, Wk, blk_begin, blk_end, summ, st);
}

sas_status launch_block_summaries_paged(const sas_dims& d, const void* K, KvPages pg,
                                        const int32_t* seq_lens, const float* Wk, int blk_begin,
                                        int blk_end, float* summ, hipStream_t st) {
  return sum_any(d, K, pg, seq_lens, Wk, blk_begin, blk_end, summ, st);
}

}  // namespace sas
