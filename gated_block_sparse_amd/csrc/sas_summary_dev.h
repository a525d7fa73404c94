// Device pieces of the block summary (SAS close reading 2.1, block summary,
// mean-pooled): summ_m = Wk_sel . mean_{j in block m} k_j.  Shared by the
// summaries kernel and the decode step's fused refresh of the newest block,
// which must produce the same bits: both run these functions with the same
// 256-thread mapping, so every sum is taken in the same order.
#pragma once

#include "sas_device.h"

namespace sas {

constexpr int kSumThreads = 256;   // threads of a workgroup that summarises

template <typename T, int D>
struct BlockMean {
  static constexpr int EPL = Vec16<T>::N;   // elements per 16-byte load
  static constexpr int LPR = D / EPL;       // lanes per K row
  static constexpr int RPI = 64 / LPR;      // rows per load instruction (per wave)
  static constexpr int NI = kBlock / RPI;   // load instructions per block
  uint4 raw[NI];

  // The wave's loads of one 64-token block (lane: row lane / LPR + RPI i,
  // 16-byte column slice lane % LPR).
  __device__ __forceinline__ void load(const T* blk, int lane) {
    const int col = lane % LPR, row0 = lane / LPR;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(blk + (row0 + i * RPI) * D + col * EPL);
  }
  // Column sums (rows in load order, then a butterfly over the row groups);
  // lanes < LPR write the mean of their EPL columns to mean[].
  __device__ __forceinline__ void reduce(int lane, float* mean) const {
    const int col = lane % LPR;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float f[EPL];
      Vec16<T>::unpack(raw[i], f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += f[e];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = wave_sum_from(acc[e], LPR);
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) mean[col * EPL + e] = acc[e] * (1.0f / kBlock);
    }
  }
};

// Projection by Wk_sel: thread tid owns output j = tid / SPLIT and input
// channels part * CW .. + CW (part = tid % SPLIT); SPLIT adjacent lanes
// combine their partial sums.
template <int D, int DS>
struct WkSlice {
  static constexpr int SPLIT = kSumThreads / DS;
  static constexpr int CW = D / SPLIT;
  float w[CW];

  __device__ __forceinline__ void load(const float* Wk, int tid) {
    const int j = tid / SPLIT, part = tid % SPLIT;
    const float4* wr = reinterpret_cast<const float4*>(Wk + static_cast<size_t>(j) * D + part * CW);
#pragma unroll
    for (int c4 = 0; c4 < CW / 4; ++c4) {
      const float4 x = wr[c4];
      w[4 * c4 + 0] = x.x;
      w[4 * c4 + 1] = x.y;
      w[4 * c4 + 2] = x.z;
      w[4 * c4 + 3] = x.w;
    }
  }
  // Output tid / SPLIT of the projected mean (valid on every lane of its group).
  __device__ __forceinline__ float project(const float* mean, int tid) const {
    const int part = tid % SPLIT;
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < CW; ++c) a += w[c] * mean[part * CW + c];
    return group_sum(a, SPLIT);
  }
};

}  // namespace sas
