// One decode step of gated sparse attention (SAS reproduction note, core
// formula; SAS summary, Method, fused kernel; SAS close reading 2.1-2.2):
//   z_j = q_h . k_j * scale + beta_j,   beta = log g_m on selected history
//         block m, 0 on the current block B0 (beta = 0 everywhere when the
//         gate is not passed: the inference rule of SAS close reading 2.1/2.3)
//   o_h = softmax(z) V,  lse_h = LSE(z)
//
// Split-KV: the unit of work is one 64-token block of one (sequence, group):
// the k selected history blocks plus B0.  A workgroup streams its block's K
// and V once (16-byte loads, every load instruction covers whole 256-byte
// rows), applies it to all G query heads of the group (each K/V byte serves G
// heads), and leaves an unnormalised partial softmax state (max, sum, acc) in
// the workspace.  The last workgroup of a (sequence, group) to finish -- found
// with one arrival counter per group -- merges the k+1 partials of each head
// in slot order:  o = sum_u e^{m_u-M} acc_u / sum_u e^{m_u-M} l_u,  so the
// result does not depend on arrival order and is bitwise reproducible.  That
// workgroup also resets the counter, leaving the workspace ready for the next
// call (the counters must be zero before the first one).
#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

constexpr int kDecThreads = 256;  // 4 waves x 16 tokens = one 64-token block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int G, int D> struct DecPartial {
  // acc[G][D], then m[G] (base-2 max of z*log2e), then l[G]
  static constexpr int kFloats = G * (D + 2);
};

template <typename T, int D, int G>
__global__ void __launch_bounds__(kDecThreads)
decode_fwd_kernel(const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V,
                  const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ idx,
                  const float* __restrict__ log_gate, float scale2, int Hkv, int t_max, int k,
                  unsigned* __restrict__ counters, float* __restrict__ part, T* __restrict__ o,
                  float* __restrict__ lse) {
  constexpr int EPL = Vec16<T>::N;      // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per wave load instruction
  constexpr int NI = 16 / RPI;          // loads per wave per tensor (16 tokens per wave)
  constexpr int PF = DecPartial<G, D>::kFloats;
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ float red_acc[4][G][D];
  __shared__ float mrg_w[kMaxTopK + 1][G];  // per-slot max, then merge weight
  __shared__ float mrg_l[kMaxTopK + 1][G];
  __shared__ float mrg_L[G];
  __shared__ int s_last;

  const int u = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int len = clamp_len(seq_lens[b], t_max);
  const int C = (len - 1) / kBlock;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  float* out = part + (row * (k + 1) + u) * static_cast<size_t>(PF);

  int start = 0, ntok = 0;
  float beta2 = 0.f;  // bias, already multiplied by log2(e)
  if (u < k) {
    const int m = idx[row * k + u];
    if (m >= 0) {
      start = m * kBlock;
      ntok = kBlock;
      if (log_gate) beta2 = log_gate[row * k + u] * kLog2e;
    }
  } else {
    start = C * kBlock;
    ntok = len - start;
  }

  if (ntok == 0) {  // empty slot: a neutral partial
    for (int x = tid; x < PF; x += kDecThreads) out[x] = (x >= G * D && x < G * D + G) ? -INFINITY : 0.f;
  } else {
    const int col = lane % LPR, rsub = lane / LPR;
    const T* Kb = K + (row * t_max + start) * static_cast<size_t>(D) + col * EPL;
    const T* Vb = V + (row * t_max + start) * static_cast<size_t>(D) + col * EPL;
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = wave * 16 + i * RPI + rsub;
      if (j < ntok) {
        kr[i] = *reinterpret_cast<const uint4*>(Kb + static_cast<size_t>(j) * D);
        vr[i] = *reinterpret_cast<const uint4*>(Vb + static_cast<size_t>(j) * D);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
    float qv[G][EPL];
    {
      const T* qb = q + (row * G) * static_cast<size_t>(D) + col * EPL;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        uint4 raw = *reinterpret_cast<const uint4*>(qb + h * D);
        Vec16<T>::unpack(raw, qv[h]);
      }
    }
    // logits (base-2 domain)
    float z[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPL];
      Vec16<T>::unpack(kr[i], kf);
      const int j = wave * 16 + i * RPI + rsub;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot += qv[h][e] * kf[e];
        dot = group_sum(dot, LPR);
        z[i][h] = (j < ntok) ? dot * scale2 + beta2 : -INFINITY;
      }
    }
    float mh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float v = z[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) v = fmaxf(v, z[i][h]);
      mh[h] = wave_max_from(v, LPR);
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) red_m[wave][h] = mh[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h)
      mh[h] = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));

    float acc[G][EPL];
    float lh[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lh[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      Vec16<T>::unpack(vr[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = exp2f(z[i][h] - mh[h]);  // 0 for masked rows
        lh[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[e];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lh[h] = wave_sum_from(lh[h], LPR);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = wave_sum_from(acc[h][e], LPR);
    }
    if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) red_acc[wave][h][col * EPL + e] = acc[h][e];
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) red_l[wave][h] = lh[h];
    }
    __syncthreads();
    for (int x = tid; x < G * D; x += kDecThreads) {
      const int h = x / D, c = x % D;
      out[x] = red_acc[0][h][c] + red_acc[1][h][c] + red_acc[2][h][c] + red_acc[3][h][c];
    }
    if (tid < G) {
      out[G * D + tid] = mh[tid];
      out[G * D + G + tid] = red_l[0][tid] + red_l[1][tid] + red_l[2][tid] + red_l[3][tid];
    }
  }

  // ---- arrival; the last workgroup of the row merges
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(counters + row, 1u) == static_cast<unsigned>(k);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const float* base = part + row * (k + 1) * static_cast<size_t>(PF);
  for (int x = tid; x < (k + 1) * G; x += kDecThreads) {  // all (max, sum) loads at once
    const int uu = x / G, g = x % G;
    mrg_w[uu][g] = base[uu * PF + G * D + g];
    mrg_l[uu][g] = base[uu * PF + G * D + G + g];
  }
  __syncthreads();
  if (tid < G) {
    const int g = tid;
    float M = -INFINITY;
    for (int uu = 0; uu <= k; ++uu) M = fmaxf(M, mrg_w[uu][g]);
    float L = 0.f;
    for (int uu = 0; uu <= k; ++uu) {
      const float w = exp2f(mrg_w[uu][g] - M);
      mrg_w[uu][g] = w;
      L += w * mrg_l[uu][g];
    }
    mrg_L[g] = L;
    if (lse) lse[row * G + g] = M * kLn2 + logf(L);
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += kDecThreads) {
    const int g = x / D;
    float a = 0.f;
#pragma unroll 8
    for (int uu = 0; uu <= k; ++uu) a += mrg_w[uu][g] * base[uu * PF + x];
    store_scalar<T>(o + (row * G) * static_cast<size_t>(D) + x, a / mrg_L[g]);
  }
  if (tid == 0) counters[row] = 0u;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: counters[B*Hkv] | partials[B*Hkv*(k+1)*G*(d+2)] fp32
size_t decode_ws_bytes(const sas_dims& d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  return align256(rows * sizeof(unsigned)) +
         rows * (d.top_k + 1) * G * (d.head_dim + 2) * sizeof(float);
}

template <typename T, int D, int G>
static sas_status launch_dec(const sas_dims& d, const void* q, const void* K, const void* V,
                             const int32_t* seq_lens, const int32_t* idx, const float* log_gate,
                             float scale, void* o, float* lse, void* ws, hipStream_t st) {
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  unsigned* counters = static_cast<unsigned*>(ws);
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(rows * sizeof(unsigned)));
  hipLaunchKernelGGL((decode_fwd_kernel<T, D, G>), dim3(d.top_k + 1, d.n_kv_heads, d.batch),
                     dim3(kDecThreads), 0, st, static_cast<const T*>(q),
                     static_cast<const T*>(K), static_cast<const T*>(V), seq_lens, idx, log_gate,
                     scale * kLog2e, d.n_kv_heads, d.t_max, d.top_k, counters, part,
                     static_cast<T*>(o), lse);
  return check_launch("decode_fwd");
}

template <typename T, int D>
static sas_status dec_by_group(const sas_dims& d, const void* q, const void* K, const void* V,
                               const int32_t* seq_lens, const int32_t* idx,
                               const float* log_gate, float scale, void* o, float* lse,
                               void* ws, hipStream_t st) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_dec<T, D, 1>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
    case 2: return launch_dec<T, D, 2>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
    case 4: return launch_dec<T, D, 4>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
    case 8: return launch_dec<T, D, 8>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
  }
  return fail(SAS_ERR_UNSUPPORTED, "decode: group size");
}

sas_status launch_decode_fwd(const sas_dims& d, const void* q, const void* K, const void* V,
                             const int32_t* seq_lens, const int32_t* idx, const float* log_gate,
                             float scale, void* o, float* lse, void* ws, hipStream_t st) {
  if (d.dtype == SAS_BF16) {
    if (d.head_dim == 128)
      return dec_by_group<uint16_t, 128>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
    return dec_by_group<uint16_t, 64>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
  }
  if (d.head_dim == 128)
    return dec_by_group<float, 128>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
  return dec_by_group<float, 64>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
}

}  // namespace sas
