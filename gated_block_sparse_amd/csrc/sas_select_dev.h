// Device helpers of the selection shared by the selection kernels, the fused
// select + attention kernel and the selector backward: block reductions, the
// projected pooled query, score rows, the merge of per-chunk Top-K candidate
// lists and of per-chunk softmax states.
#pragma once

#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

constexpr int kSelThreads = 256;

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

// qs[j] = (Wq[j,:] . qm) / sqrt(DS), for j < DS (threads tid < DS).
template <int D, int DS>
__device__ __forceinline__ void project_query(const float* __restrict__ Wq, const float* qm,
                                              float* qs) {
  const int tid = threadIdx.x;
  if (tid < DS) {
    const float4* w = reinterpret_cast<const float4*>(Wq + static_cast<size_t>(tid) * D);
    float acc = 0.f;
#pragma unroll 8
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const float4 x = w[c4];
      acc += x.x * qm[4 * c4 + 0];
      acc += x.y * qm[4 * c4 + 1];
      acc += x.z * qm[4 * c4 + 2];
      acc += x.w * qm[4 * c4 + 3];
    }
    qs[tid] = acc * (1.0f / sqrtf(static_cast<float>(DS)));
  }
}

// Mean of the query rows of one tile over the group's G heads and the tile's
// nq queries (qm[0..D), written by threads tid < D); qpart is LDS scratch of
// (kSelThreads / (D / 16-byte elements)) x D floats.  Ends with a barrier.
template <typename T, int D, int G>
__device__ __forceinline__ void tile_pooled_query(const T* __restrict__ Q, int q_len, int Hkv,
                                                  int b, int r, int i0, int nq, float* qpart,
                                                  float* qm) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  constexpr int RG = kSelThreads / LPR;  // row groups
  const int tid = threadIdx.x;
  {
    const int col = tid % LPR, rg = tid / LPR;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    const int nrows = G * nq;
    for (int x = rg; x < nrows; x += RG) {
      const int h = r * G + x / nq, i = i0 + x % nq;
      const T* src = Q + ((static_cast<size_t>(b) * Hkv * G + h) * q_len + i) * D + col * EPL;
      float f[EPL];
      Vec16<T>::unpack(*reinterpret_cast<const uint4*>(src), f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) qpart[rg * D + col * EPL + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
    for (int g = 0; g < RG; ++g) a += qpart[g * D + tid];
    qm[tid] = a / static_cast<float>(G * nq);
  }
  __syncthreads();
}

// Scores of blocks [0, n) of one (b, r) (rows of summ_row0) into sc[0..n).
// Each half wave owns 32 rows per round (rows hw + 8j, j < 32): all 32
// 16-byte loads are issued before any arithmetic, then a transposed butterfly
// (16+8+4+2+1 shuffles) leaves the full dot of row j in lane j.
template <int DS>
__device__ __forceinline__ void score_rows(const float* __restrict__ summ_row0, const float* qs,
                                           int n, float* sc) {
  constexpr int PL = DS / 32;  // floats per lane (2 or 4)
  const int tid = threadIdx.x, hw = tid >> 5, l32 = tid & 31;
  float qv[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) qv[e] = qs[l32 * PL + e];
  for (int base = 0; base < n; base += 32 * (kSelThreads / 32)) {
    float v[32];
    if constexpr (PL == 4) {
      float4 x[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int i = base + hw + 8 * j;
        x[j] = i < n ? *reinterpret_cast<const float4*>(summ_row0 + static_cast<size_t>(i) * DS + l32 * PL)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = x[j].x * qv[0] + x[j].y * qv[1] + x[j].z * qv[2] + x[j].w * qv[3];
    } else {
      float2 x[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int i = base + hw + 8 * j;
        x[j] = i < n ? *reinterpret_cast<const float2*>(summ_row0 + static_cast<size_t>(i) * DS + l32 * PL)
                     : make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = x[j].x * qv[0] + x[j].y * qv[1];
    }
    transpose_sum32(v, l32);
    const int i = base + hw + 8 * l32;
    if (i < n) sc[i] = v[0];
  }
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
