// Causal prefill / training forward with one selection per 64-query tile
// (SAS summary, Method, fused kernel; SAS close reading 2.1-2.4):
//   query i of tile t, head h of group r attends to
//     - every token of the selected history blocks idx[b,r,t,:], bias log g,
//     - tokens 64t..i of its own block (causal), bias 0,
//   o = softmax(q K^T * scale + beta) V,  lse = LSE of the logits.
//
// gfx950 MFMA design (bf16 in, fp32 accumulate, v_mfma_f32_32x32x16_bf16):
//  * one workgroup per (tile, group, sequence), heaviest tiles first; it
//    packs up to 4 query heads of the group (2 waves per head, 32 queries per
//    wave), so every K/V block staged in LDS feeds all of them;
//  * each wave computes S^T = K Q^T (token rows x query columns): a lane then
//    owns one query column, so the row max / sum of the online softmax is a
//    register reduction plus one cross-half swap, and the accumulator rescale
//    is one multiply per lane;
//  * O^T += V^T P^T: P^T comes straight from the S^T accumulators of the lane
//    (the 16 tokens of a k-step are taken in the order the accumulator layout
//    holds them, and V^T is read in that same order), V is transposed while
//    it is staged into LDS;
//  * the log-gate is added per block; the diagonal block is masked j > i.
#include "sas_device.h"
#include "sas_internal.h"
#include "sas_mfma.h"

namespace sas {

template <int D, int HPW>
__global__ void __launch_bounds__(128 * HPW)
prefill_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, int S, int Hkv, int G, int t_max,
                   int n_tiles, int k, const int32_t* __restrict__ idx,
                   const float* __restrict__ log_gate, float scale2, uint16_t* __restrict__ O,
                   float* __restrict__ lse) {
  constexpr int NT = 128 * HPW;      // threads
  constexpr int KS = D / 16;         // k-steps of S^T = K Q^T
  constexpr int CT = D / 32;         // channel tiles of O^T
  constexpr int KSTR = D + 8;        // K row stride in LDS (bf16), +16 bytes
  constexpr int VSTR = 64 + 8;       // V^T row stride in LDS (bf16), +16 bytes
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];

  const int nhc = G / HPW;                       // head chunks per group
  const int t = n_tiles - 1 - static_cast<int>(blockIdx.x) / nhc;
  const int hc = static_cast<int>(blockIdx.x) % nhc;
  const int r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int Hq = Hkv * G, h = r * G + hc * HPW + (wave >> 1);
  const int qloc = (wave & 1) * 32 + l32;        // query within the tile
  const int qi = t * 64 + qloc;
  const bool qvalid = qi < S;

  bf16x8_t qb[KS];  // B operand of S^T = K Q^T: Q[qi][16ks + 8hi .. +8]
  {
    const uint16_t* qrow = Q + ((static_cast<size_t>(b) * Hq + h) * S + (qvalid ? qi : 0)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4*>(qrow + 16 * ks)
                                : make_uint4(0, 0, 0, 0));
  }
  f32x16_t acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[ct][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const size_t srow = (static_cast<size_t>(b) * Hkv + r) * n_tiles + t;
  const uint16_t* Kg = K + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;
  const uint16_t* Vg = V + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;

  for (int it = 0; it <= k; ++it) {
    const bool diag = it == k;
    int blk = t;
    float beta2 = 0.f;
    if (!diag) {
      blk = idx[srow * k + it];
      if (blk < 0) continue;  // uniform across the workgroup
      if (log_gate) beta2 = log_gate[srow * k + it] * kLog2eF;
    }
    const int tok0 = blk * 64;
    __syncthreads();  // the previous block's LDS reads are done
    stage_rows<D, NT>(Kg + static_cast<size_t>(tok0) * D, S - tok0, Ks, nullptr, tid);
    stage_rows<D, NT>(Vg + static_cast<size_t>(tok0) * D, S - tok0, nullptr, Vt, tid);
    __syncthreads();

    // S^T (64 tokens x 32 queries) = K Q^T
    f32x16_t s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[tt][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(&Ks[(32 * tt + l32) * KSTR + 16 * ks + 8 * hi]));
        s[tt] = mfma32x32x16(a, qb[ks], s[tt]);
      }
    }
    // online softmax on the lane's query column (base-2 domain)
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tok = 32 * tt + 8 * (v >> 2) + 4 * hi + (v & 3);
        float z = s[tt][v] * scale2 + beta2;
        if (diag && tok > qloc) z = -INFINITY;
        s[tt][v] = z;
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2f(s[tt][v] - m_new);
        s[tt][v] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ct][v] *= alpha;

    // O^T (D channels x 32 queries) += V^T P^T, k-step j = tokens 16j..16j+15
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t pb = acc_to_bop(s, j);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        acc[ct] = mfma32x32x16(lds_aop_perm(&Vt[(32 * ct + l32) * VSTR], j, hi), pb, acc[ct]);
    }
  }

  if (qvalid) {
    store_acc_col<CT>(acc, 1.f / l_run, O + ((static_cast<size_t>(b) * Hq + h) * S + qi) * D, hi);
    if (hi == 0) lse[(static_cast<size_t>(b) * Hq + h) * S + qi] = (m_run + log2f(l_run)) * kLn2F;
  }
}

size_t prefill_ws_bytes(const sas_dims&, int) { return 0; }

template <int D>
static sas_status launch_pf(const sas_dims& d, const void* Q, const void* K, const void* V,
                            int S, const int32_t* idx, const float* log_gate, float scale,
                            void* O, float* lse, hipStream_t st) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const int n_tiles = cdiv(S, kBlock);
  const float scale2 = scale * kLog2eF;
#define SAS_PF_CASE(HPW)                                                                   \
  hipLaunchKernelGGL((prefill_fwd_kernel<D, HPW>), dim3(n_tiles * (G / HPW), d.n_kv_heads, \
                     d.batch), dim3(128 * HPW), 0, st, static_cast<const uint16_t*>(Q),   \
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), S,   \
                     d.n_kv_heads, G, d.t_max, n_tiles, d.top_k, idx, log_gate, scale2,     \
                     static_cast<uint16_t*>(O), lse)
  switch (G) {
    case 1: SAS_PF_CASE(1); break;
    case 2: SAS_PF_CASE(2); break;
    default: SAS_PF_CASE(4); break;  // G = 4 or 8 (two head chunks)
  }
#undef SAS_PF_CASE
  return check_launch("prefill_fwd");
}

sas_status launch_prefill_fwd(const sas_dims& d, const void* Q, const void* K, const void* V,
                              int seq_len, const int32_t* idx, const float* log_gate,
                              float scale, void* O, float* lse, void* ws, hipStream_t st) {
  (void)ws;
  if (d.head_dim == 128)
    return launch_pf<128>(d, Q, K, V, seq_len, idx, log_gate, scale, O, lse, st);
  return launch_pf<64>(d, Q, K, V, seq_len, idx, log_gate, scale, O, lse, st);
}

}  // namespace sas
