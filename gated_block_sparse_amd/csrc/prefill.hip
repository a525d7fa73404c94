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
//    holds them), and V^T is read in that same order from the row-major V
//    tile with the LDS transpose read;
//  * the log-gate is added per block; the diagonal block is masked j > i;
//  * the block loop is software-pipelined (see the kernel) so each wave always
//    has matrix and vector work that do not depend on each other.
#include "sas_device.h"
#include "sas_internal.h"
#include "sas_mfma.h"

namespace sas {

// Per-thread share of staging one 64-token block: K and V rows, as 16-byte
// chunks copied row-major into LDS (V, at the transpose-read stride, is read
// back transposed by the LDS transpose read, so no shuffling on the way in).
template <int D, int NT>
struct BlockStage {
  static constexpr int TOT = 64 * (D / 8);           // 16-byte chunks per tensor
  static constexpr int CH = (TOT + NT - 1) / NT;     // per thread
  uint4 k[CH], v[CH];

  __device__ __forceinline__ void load(const uint16_t* Kb, const uint16_t* Vb, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * NT, row = c / (D / 8), cc = c % (D / 8);
      const bool ok = c < TOT && row < valid;
      k[i] = ok ? *reinterpret_cast<const uint4*>(Kb + static_cast<size_t>(row) * D + cc * 8)
                : make_uint4(0, 0, 0, 0);
      v[i] = ok ? *reinterpret_cast<const uint4*>(Vb + static_cast<size_t>(row) * D + cc * 8)
                : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* Ks, uint16_t* Vs, int tid) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * NT, row = c / (D / 8), cc = c % (D / 8);
      if (c < TOT) {
        lds_store_row8<kRowStride<D>>(Ks, row, cc * 8, k[i]);
        lds_store_row8<kTrStride<D>>(Vs, row, cc * 8, v[i]);
      }
    }
  }
};

// S^T (64 tokens x 32 queries) = K Q^T for one staged block.
template <int D>
__device__ __forceinline__ void block_scores(const uint16_t* Kc, const bf16x8_t* qb, f32x16_t* s,
                                             int l32, int hi) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    zero16(s[tt]);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      s[tt] = mfma32x32x16(lds_row8<kRowStride<D>>(Kc, 32 * tt + l32, 16 * ks + 8 * hi), qb[ks],
                           s[tt]);
  }
}

// O^T (D channels x 32 queries) += V^T P^T for one staged block; k-step j =
// tokens 16j..16j+15 in accumulator order.
template <int D>
__device__ __forceinline__ void block_pv(const uint16_t* Vc, const bf16x8_t* pb, f32x16_t* acc,
                                         int hi) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
      acc[ct] = mfma32x32x16(lds_aop_tr_perm<kTrStride<D>>(Vc, 32 * ct, j, hi), pb[j], acc[ct]);
}

// Software pipeline over the block list: in iteration i a wave
//   A: adds block i-1's P V into O^T (MFMA) while it takes block i's max (VALU),
//   B: computes block i+1's scores (MFMA) while it exponentiates block i (VALU),
// so the matrix cores and the vector ALUs of a wave have independent work at
// every point.  Staged blocks live in a ring of four LDS buffers (block i in
// buffer i % 4); block i+2 is written while blocks i-1 and i+1 are read, so
// one barrier per iteration suffices.
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
  constexpr int NBUF = 4;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NBUF][64 * kRowStride<D>];  // row reads
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NBUF][64 * kTrStride<D>];   // transpose reads
  __shared__ int s_blk[kMaxTopK + 1];
  __shared__ float s_beta[kMaxTopK + 1];
  __shared__ int s_nblk;

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

  // block list: the valid selected blocks (in slot order), then the diagonal
  const size_t srow = (static_cast<size_t>(b) * Hkv + r) * n_tiles + t;
  if (wave == 0) {
    const bool ok = lane < k && idx[srow * k + lane] >= 0;
    const unsigned long long mask = __ballot(ok);
    if (ok) {
      const int pos = __popcll(mask & ((1ull << lane) - 1ull));
      s_blk[pos] = idx[srow * k + lane];
      s_beta[pos] = log_gate ? log_gate[srow * k + lane] * kLog2eF : 0.f;
    }
    if (lane == 0) {
      const int nv = __popcll(mask);
      s_blk[nv] = t;
      s_beta[nv] = 0.f;
      s_nblk = nv + 1;
    }
  }

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
  for (int ct = 0; ct < CT; ++ct) zero16(acc[ct]);
  float m_run = -INFINITY, l_run = 0.f;

  const uint16_t* Kg = K + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;
  const uint16_t* Vg = V + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;
  __syncthreads();
  const int nblk = s_nblk;

  // History blocks are 0..nh-1, the diagonal block is nh.  The loop body
  // has no branch apart from the (rare) rescale, so each half of it is one
  // basic block in which the matrix and vector work can interleave: indices
  // of blocks beyond the list are clamped (their staging writes land in a
  // buffer nobody reads again), and the first iteration's P V runs on a
  // zeroed buffer with P = 0.
  const int nh = nblk - 1;
  BlockStage<D, NT> stg;
  auto load_block = [&](int i) {
    const int tok = s_blk[min(i, nh)] * 64;
    stg.load(Kg + static_cast<size_t>(tok) * D, Vg + static_cast<size_t>(tok) * D, S - tok, tid);
  };
  load_block(0);
  stg.store(Ks[0], Vs[0], tid);
  load_block(1);
  stg.store(Ks[1], Vs[1], tid);
  for (int c = tid; c < 64 * kTrStride<D> / 8; c += NT)
    *reinterpret_cast<uint4*>(&Vs[3][8 * c]) = make_uint4(0, 0, 0, 0);
  load_block(2);
  __syncthreads();

  f32x16_t s_cur[2];
  block_scores<D>(Ks[0], qb, s_cur, l32, hi);
  bf16x8_t p_prev[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) p_prev[j] = as_bf16x8(make_uint4(0, 0, 0, 0));

  // Lazy rescaling: the running max only moves (and the accumulators are
  // only rescaled) when some lane's max grew by more than 2^8; otherwise the
  // probabilities are taken against the stale max, which bounds them by 256.
  auto update_max = [&](float beta2) {
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s_cur[tt][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_cand = fmaxf(m_run, mx * scale2 + beta2);
    if (__any(!(m_cand - m_run <= 8.f))) {
      const float alpha = exp2f(m_run - m_cand);
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ct][v] *= alpha;
      m_run = m_cand;
    }
  };
  auto probabilities = [&](float beta2) {
    const float off = beta2 - m_run;
    float ls = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(fmaf(s_cur[tt][v], scale2, off));
        s_cur[tt][v] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l_run += ls;
#pragma unroll
    for (int j = 0; j < 4; ++j) p_prev[j] = acc_to_bop(s_cur, j);
  };

  for (int it = 0; it < nh; ++it) {
    const float beta2 = s_beta[it];
    // A: the previous block's P V, this block's max
    block_pv<D>(Vs[(it + 3) & 3], p_prev, acc, hi);
    update_max(beta2);
    // B: the next block's scores, this block's probabilities, staging of
    // block it+2 and the loads of block it+3
    f32x16_t s_next[2];
    block_scores<D>(Ks[(it + 1) & 3], qb, s_next, l32, hi);
    probabilities(beta2);
    stg.store(Ks[(it + 2) & 3], Vs[(it + 2) & 3], tid);
    load_block(it + 3);
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) s_cur[tt] = s_next[tt];
  }
  // the diagonal block: causal mask j > i
  block_pv<D>(Vs[(nh + 3) & 3], p_prev, acc, hi);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (32 * tt + acc_row(v, hi) > qloc) s_cur[tt][v] = -INFINITY;
  update_max(0.f);
  probabilities(0.f);
  block_pv<D>(Vs[nh & 3], p_prev, acc, hi);

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
