// Device helpers of the decode selection that the selection kernels and the
// fused select + attention kernel share (the merge of per-chunk Top-K
// candidate lists and of per-chunk softmax states).
#pragma once

#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

__device__ __forceinline__ float block_max(float v, float* red) {
  v = group_max(v, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = group_sum(v, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r += red[i];
  return r;
}

// Loads a row's chunk candidates (nchunk sorted lists of kc keys, padded to
// nlist lists with zero keys) into src and merges the chunks' (max, sum-exp)
// states into the row's LSE of the scores (-inf when C == 0).  Every thread
// of the workgroup calls it; it ends with a barrier.
__device__ __forceinline__ float load_chunk_states(const uint64_t* __restrict__ cr,
                                                   const float2* __restrict__ pr, int nchunk,
                                                   int nlist, int kc, int C, uint64_t* src,
                                                   float* red) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int ncand = nchunk * kc, ntot = nlist * kc;
  for (int i = tid; i < ntot; i += nt) src[i] = i < ncand ? cr[i] : 0ull;
  float mloc = -INFINITY;
  for (int i = tid; i < nchunk; i += nt) mloc = fmaxf(mloc, pr[i].x);
  const float M = block_max(mloc, red);
  float sloc = 0.f;
  for (int i = tid; i < nchunk; i += nt) {
    const float2 v = pr[i];
    if (v.x != -INFINITY) sloc += v.y * expf(v.x - M);
  }
  const float L = block_sum(sloc, red);  // ends with a barrier: src is complete
  return C > 0 ? M + logf(L) : -INFINITY;
}

// Pairwise merge of nlist (a power of two) descending lists of kc keys held in
// src, log2(nlist) levels: a key's place in the merged list is its own
// position plus the number of larger keys in the partner list (binary
// search); each merged list keeps its top kc.  Returns the buffer (src or
// dst) holding the final list.  All threads call it; ends with a barrier.
__device__ __forceinline__ uint64_t* merge_sorted_lists(uint64_t* src, uint64_t* dst, int nlist,
                                                        int kc) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int nl = nlist; nl > 1; nl >>= 1) {
    const int half = nl >> 1;
    for (int i = tid; i < half * kc; i += nt) dst[i] = 0ull;
    __syncthreads();
    for (int i = tid; i < nl * kc; i += nt) {
      const int li = i / kc, pos = i % kc;
      const uint64_t key = src[i];
      if (key == 0ull) continue;
      const int partner = li ^ 1;
      const int rank = pos + count_greater_desc(src + partner * kc, kc, key);
      if (rank < kc) dst[(li >> 1) * kc + rank] = key;
    }
    __syncthreads();
    uint64_t* t = src;
    src = dst;
    dst = t;
  }
  return src;
}

// Writes the row's final outputs from the (descending-sorted) keys[0..kk).
__device__ __forceinline__ void write_selection(const uint64_t* keys, int kk, int k, float lse,
                                                int32_t* idx, float* log_gate) {
  const int tid = threadIdx.x;
  if (tid < kk) {
    const uint64_t key = keys[tid];
    const int mb = key_block(key);
    int rank = 0;
    for (int j = 0; j < kk; ++j) rank += key_block(keys[j]) < mb;
    idx[rank] = mb;
    log_gate[rank] = key_score(key) - lse;
  } else if (tid < k) {
    idx[tid] = -1;
    log_gate[tid] = -INFINITY;
  }
}

}  // namespace sas
