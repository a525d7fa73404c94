// Backward of the causal gated block-sparse prefill (SAS close reading 2.4
// and 2.2 eq. 5; SAS summary, Method):
//   P = exp(q K^T * scale + beta - lse),  D = rowsum(dO * O),
//   dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
//   dlog_gate[t, slot] = sum of dS over the heads of the group, the queries
//                        of tile t and the tokens of block idx[t, slot].
// The log-gate is an independent input (its chain into the selector is not
// part of this call); B0 carries no gate.
//
// Three kernels, no atomics (bitwise reproducible):
//  1. pre-pass: D per query row; zero dlog_gate.
//  2. Q-outer (one workgroup per tile x group, heads packed like the
//     forward): recompute S^T = K Q^T, dP^T = V dO^T, dS^T; dQ^T += K^T dS^T.
//  3. KV-outer (one workgroup per key block x group): the workgroup finds the
//     tiles that selected its block (binary search in each later tile's
//     ascending idx row) plus the diagonal tile, then for every such tile and
//     head recomputes S = Q K^T (a lane owns one token column), dP = dO V^T,
//     dS, and accumulates dV^T += dO^T P and dK^T += Q^T dS in registers.  It
//     is the only writer of dK/dV for its block and of the dlog_gate entries
//     that point at it, which it sums over heads in a fixed order.
#include "sas_device.h"
#include "sas_internal.h"
#include "sas_mfma.h"

namespace sas {

// ------------------------------------------------------------ pre-pass ---
template <int D>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, size_t n_rows,
               float* __restrict__ Dq, float* __restrict__ dlg, size_t n_dlg) {
  constexpr int LPR = D / 8;
  const size_t g = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t row = g / LPR;
  const int col = static_cast<int>(g % LPR);
  float acc = 0.f;
  if (row < n_rows) {
    float a[8], c[8];
    Vec16<uint16_t>::unpack(*reinterpret_cast<const uint4*>(O + row * D + col * 8), a);
    Vec16<uint16_t>::unpack(*reinterpret_cast<const uint4*>(dO + row * D + col * 8), c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += a[e] * c[e];
  }
  acc = group_sum(acc, LPR);
  if (row < n_rows && col == 0) Dq[row] = acc;
  for (size_t i = g; i < n_dlg; i += static_cast<size_t>(gridDim.x) * blockDim.x) dlg[i] = 0.f;
}

// ------------------------------------------------------------ dQ pass ---
template <int D, int HPW>
__global__ void __launch_bounds__(128 * HPW)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ lse, const float* __restrict__ Dq, int S, int Hkv, int G,
              int t_max, int n_tiles, int k, const int32_t* __restrict__ idx,
              const float* __restrict__ log_gate, float scale2, float scale,
              uint16_t* __restrict__ dQ) {
  constexpr int NT = 128 * HPW;
  constexpr int KS = D / 16, CT = D / 32;
  constexpr int RSTR = D + 8, TSTR = 64 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[64 * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * TSTR];

  const int nhc = G / HPW;
  const int t = n_tiles - 1 - static_cast<int>(blockIdx.x) / nhc;
  const int hc = static_cast<int>(blockIdx.x) % nhc;
  const int r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int Hq = Hkv * G, h = r * G + hc * HPW + (wave >> 1);
  const int qloc = (wave & 1) * 32 + l32;
  const int qi = t * 64 + qloc;
  const bool qvalid = qi < S;
  const size_t qrow_i = (static_cast<size_t>(b) * Hq + h) * S + (qvalid ? qi : 0);

  bf16x8_t qb[KS], db[KS];  // B operands: Q[qi][..], dO[qi][..]
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qb[ks] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4*>(Q + qrow_i * D + 16 * ks + 8 * hi)
                              : make_uint4(0, 0, 0, 0));
    db[ks] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4*>(dO + qrow_i * D + 16 * ks + 8 * hi)
                              : make_uint4(0, 0, 0, 0));
  }
  const float lse2 = qvalid ? lse[qrow_i] * kLog2eF : 0.f;
  const float Dv = qvalid ? Dq[qrow_i] : 0.f;
  f32x16_t dq[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) zero16(dq[ct]);

  const size_t srow = (static_cast<size_t>(b) * Hkv + r) * n_tiles + t;
  const uint16_t* Kg = K + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;
  const uint16_t* Vg = V + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;

  for (int it = 0; it <= k; ++it) {
    const bool diag = it == k;
    int blk = t;
    float beta2 = 0.f;
    if (!diag) {
      blk = idx[srow * k + it];
      if (blk < 0) continue;
      if (log_gate) beta2 = log_gate[srow * k + it] * kLog2eF;
    }
    const int tok0 = blk * 64;
    __syncthreads();
    stage_rows<D, NT>(Kg + static_cast<size_t>(tok0) * D, S - tok0, Ks, Kt, tid);
    stage_rows<D, NT>(Vg + static_cast<size_t>(tok0) * D, S - tok0, Vs, nullptr, tid);
    __syncthreads();

    f32x16_t s[2], dp[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      zero16(s[tt]);
      zero16(dp[tt]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = (32 * tt + l32) * RSTR + 16 * ks + 8 * hi;
        s[tt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(&Ks[off])), qb[ks], s[tt]);
        dp[tt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(&Vs[off])), db[ks], dp[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tok = 32 * tt + acc_row(v, hi);
        const bool ok = qvalid && !(diag && tok > qloc);
        const float p = ok ? exp2f(s[tt][v] * scale2 + beta2 - lse2) : 0.f;
        s[tt][v] = p * (dp[tt][v] - Dv);  // dS^T
      }
    // dQ^T (D x 32 queries) += K^T dS^T, k-step j = tokens 16j..16j+15
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t bop = acc_to_bop(s, j);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        dq[ct] = mfma32x32x16(lds_aop_perm(&Kt[(32 * ct + l32) * TSTR], j, hi), bop, dq[ct]);
    }
  }
  if (qvalid) store_acc_col<CT>(dq, scale, dQ + qrow_i * D, hi);
}

// --------------------------------------------------------- dK/dV pass ---
template <int D>
__global__ void __launch_bounds__(128)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ lse, const float* __restrict__ Dq, int S, int Hkv,
                int G, int t_max, int n_tiles, int k, const int32_t* __restrict__ idx,
                const float* __restrict__ log_gate, float scale2, float scale,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ dlg) {
  constexpr int NT = 128;
  constexpr int KS = D / 16, CT = D / 32;
  constexpr int RSTR = D + 8, TSTR = 64 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[64 * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[64 * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[D * TSTR];
  __shared__ float lse_s[64];
  __shared__ float D_s[64];
  __shared__ int list_t[kMaxTileRows];
  __shared__ int list_slot[kMaxTileRows];
  __shared__ int s_count;
  __shared__ int s_wcount[2];
  __shared__ float s_red[2];

  const int m = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int Hq = Hkv * G;
  const size_t grow = static_cast<size_t>(b) * Hkv + r;

  // ---- the tiles that read this block: the diagonal one, then every later
  // tile whose ascending idx row contains m (in ascending tile order)
  if (tid == 0) {
    list_t[0] = m;
    list_slot[0] = -1;
    s_count = 1;
  }
  __syncthreads();
  for (int base = m + 1; base < n_tiles; base += NT) {
    const int t = base + tid;
    int slot = -1;
    if (t < n_tiles && k > 0) {
      const int32_t* row = idx + (grow * n_tiles + t) * k;
      int lo = 0, hi2 = k;
      while (lo < hi2) {
        const int mid = (lo + hi2) >> 1;
        const int v = row[mid];
        if (v >= 0 && v < m) lo = mid + 1;
        else hi2 = mid;
      }
      if (lo < k && row[lo] == m) slot = lo;
    }
    const unsigned long long mask = __ballot(slot >= 0);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) s_wcount[wave] = __popcll(mask);
    __syncthreads();
    const int off = s_count + (wave == 1 ? s_wcount[0] : 0);
    if (slot >= 0) {
      list_t[off + before] = t;
      list_slot[off + before] = slot;
    }
    __syncthreads();
    if (tid == 0) s_count += s_wcount[0] + s_wcount[1];
    __syncthreads();
  }
  const int n_list = s_count;

  // ---- this lane's token column: K/V rows as B operands
  const int tokloc = 32 * wave + l32;
  const int tok = 64 * m + tokloc;
  const bool tvalid = tok < S;
  const uint16_t* Krow = K + (grow * t_max + (tvalid ? tok : 0)) * D;
  const uint16_t* Vrow = V + (grow * t_max + (tvalid ? tok : 0)) * D;
  bf16x8_t kb[KS], vb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kb[ks] = as_bf16x8(tvalid ? *reinterpret_cast<const uint4*>(Krow + 16 * ks + 8 * hi) : make_uint4(0, 0, 0, 0));
    vb[ks] = as_bf16x8(tvalid ? *reinterpret_cast<const uint4*>(Vrow + 16 * ks + 8 * hi) : make_uint4(0, 0, 0, 0));
  }
  f32x16_t dk[CT], dv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    zero16(dk[ct]);
    zero16(dv[ct]);
  }

  for (int e = 0; e < n_list; ++e) {
    const int t = list_t[e], slot = list_slot[e];
    const bool diag = slot < 0;
    const float beta2 = (!diag && log_gate) ? log_gate[(grow * n_tiles + t) * k + slot] * kLog2eF : 0.f;
    const int q0 = 64 * t;
    const int nq = min(64, S - q0);
    float dsum = 0.f;
    for (int g = 0; g < G; ++g) {
      const size_t hrow = (static_cast<size_t>(b) * Hq + r * G + g) * S + q0;
      __syncthreads();
      stage_rows<D, NT>(Q + hrow * D, nq, Qs, Qt, tid);
      stage_rows<D, NT>(dO + hrow * D, nq, dOs, dOt, tid);
      if (tid < 64) {
        lse_s[tid] = tid < nq ? lse[hrow + tid] * kLog2eF : 0.f;
        D_s[tid] = tid < nq ? Dq[hrow + tid] : 0.f;
      }
      __syncthreads();

      // S and dP (64 queries x this wave's 32 tokens)
      f32x16_t s[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        zero16(s[qt]);
        zero16(dp[qt]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = (32 * qt + l32) * RSTR + 16 * ks + 8 * hi;
          s[qt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(&Qs[off])), kb[ks], s[qt]);
          dp[qt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(&dOs[off])), vb[ks], dp[qt]);
        }
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int q = 32 * qt + acc_row(v, hi);
          const bool ok = tvalid && q < nq && !(diag && tokloc > q);
          const float p = ok ? exp2f(s[qt][v] * scale2 + beta2 - lse_s[q]) : 0.f;
          const float ds = p * (dp[qt][v] - D_s[q]);
          s[qt][v] = p;
          dp[qt][v] = ds;
          dsum += ds;
        }
      // dV^T += dO^T P and dK^T += Q^T dS; k-step j = queries 16j..16j+15
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t pb = acc_to_bop(s, j);
        const bf16x8_t sb = acc_to_bop(dp, j);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          dv[ct] = mfma32x32x16(lds_aop_perm(&dOt[(32 * ct + l32) * TSTR], j, hi), pb, dv[ct]);
          dk[ct] = mfma32x32x16(lds_aop_perm(&Qt[(32 * ct + l32) * TSTR], j, hi), sb, dk[ct]);
        }
      }
    }
    if (!diag) {  // dlog_gate entry (t, slot): sum over both token halves
      dsum = wave_sum_from(dsum, 1);
      if (lane == 0) s_red[wave] = dsum;
      __syncthreads();
      if (tid == 0) dlg[(grow * n_tiles + t) * k + slot] = s_red[0] + s_red[1];
    }
  }
  if (tvalid) {
    store_acc_col<CT>(dk, scale, dK + (grow * t_max + tok) * D, hi);
    store_acc_col<CT>(dv, 1.f, dV + (grow * t_max + tok) * D, hi);
  }
}

// ------------------------------------------------------------ launcher ---
size_t bwd_ws_bytes(const sas_dims& d, int seq_len) {
  return static_cast<size_t>(d.batch) * d.n_q_heads * seq_len * sizeof(float);
}

template <int D>
static sas_status launch_bwd_d(const sas_dims& d, const void* Q, const void* K, const void* V,
                               const void* O, const void* dO, const float* lse, int S,
                               const int32_t* idx, const float* log_gate, float scale, void* dQ,
                               void* dK, void* dV, float* dlg, void* ws, hipStream_t st) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const int n_tiles = cdiv(S, kBlock);
  const float scale2 = scale * kLog2eF;
  float* Dq = static_cast<float*>(ws);
  const size_t n_rows = static_cast<size_t>(d.batch) * d.n_q_heads * S;
  const size_t n_dlg = (d.top_k > 0 && dlg) ? static_cast<size_t>(d.batch) * d.n_kv_heads * n_tiles * d.top_k : 0;
  const size_t thr = n_rows * (D / 8);
  const int pre_blocks = static_cast<int>((thr + 255) / 256);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(pre_blocks), dim3(256), 0, st,
                     static_cast<const uint16_t*>(O), static_cast<const uint16_t*>(dO), n_rows,
                     Dq, dlg, n_dlg);
  sas_status s = check_launch("bwd_pre");
  if (s != SAS_OK) return s;
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* kk = static_cast<const uint16_t*>(K);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  const uint16_t* dop = static_cast<const uint16_t*>(dO);
#define SAS_DQ_CASE(HPW)                                                                        \
  hipLaunchKernelGGL((bwd_dq_kernel<D, HPW>), dim3(n_tiles * (G / HPW), d.n_kv_heads, d.batch), \
                     dim3(128 * HPW), 0, st, q, kk, v, dop, lse, Dq, S, d.n_kv_heads, G,        \
                     d.t_max, n_tiles, d.top_k, idx, log_gate, scale2, scale,                   \
                     static_cast<uint16_t*>(dQ))
  switch (G) {
    case 1: SAS_DQ_CASE(1); break;
    case 2: SAS_DQ_CASE(2); break;
    default: SAS_DQ_CASE(4); break;
  }
#undef SAS_DQ_CASE
  s = check_launch("bwd_dq");
  if (s != SAS_OK) return s;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(n_tiles, d.n_kv_heads, d.batch), dim3(128), 0, st,
                     q, kk, v, dop, lse, Dq, S, d.n_kv_heads, G, d.t_max, n_tiles, d.top_k, idx,
                     log_gate, scale2, scale, static_cast<uint16_t*>(dK),
                     static_cast<uint16_t*>(dV), dlg);
  return check_launch("bwd_dkdv");
}

sas_status launch_bwd(const sas_dims& d, const void* Q, const void* K, const void* V,
                      const void* O, const void* dO, const float* lse, int seq_len,
                      const int32_t* idx, const float* log_gate, float scale, void* dQ,
                      void* dK, void* dV, float* dlog_gate, void* ws, hipStream_t st) {
  if (cdiv(seq_len, kBlock) > kMaxTileRows)
    return fail(SAS_ERR_UNSUPPORTED, "backward: seq_len=%d gives more than %d tiles", seq_len,
                kMaxTileRows);
  if (d.head_dim == 128)
    return launch_bwd_d<128>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK, dV,
                             dlog_gate, ws, st);
  return launch_bwd_d<64>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK, dV,
                          dlog_gate, ws, st);
}

}  // namespace sas
