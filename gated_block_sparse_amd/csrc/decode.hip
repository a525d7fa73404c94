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
// the workspace.  A second, small kernel merges the k+1 partials of each head
// in slot order:  o = sum_u e^{m_u-M} acc_u / sum_u e^{m_u-M} l_u,  issuing
// all of its loads at once; the kernel boundary orders the two, so no
// device-wide fences or atomics are needed and results are bitwise
// reproducible.
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
decode_split_kernel(const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V,
                  const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ idx,
                  const float* __restrict__ log_gate, float scale2, int Hkv, int t_max, int k,
                  float* __restrict__ part) {
  constexpr int EPL = Vec16<T>::N;      // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per wave load instruction
  constexpr int NI = 16 / RPI;          // loads per wave per tensor (16 tokens per wave)
  constexpr int PF = DecPartial<G, D>::kFloats;
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ float red_acc[4][G][D];

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
      mh[h] = wave_max_from(v, LPR);  // across the row groups
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
        const float p = fast_exp2(z[i][h] - mh[h]);  // 0 for masked rows
        lh[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[e];
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) lh[h] = wave_sum_from(lh[h], LPR);
    // Sum acc over the RG = 64/LPR row groups of the wave with a transposed
    // butterfly: each step halves the values a lane keeps, so lane group q
    // ends up owning NV/RG distinct (head, element) sums.
    constexpr int NV = G * EPL, RG = 64 / LPR;
    float av[NV];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) av[h * EPL + e] = acc[h][e];
    int kept = NV;
#pragma unroll
    for (int sft = 32; sft >= LPR; sft >>= 1) {
      const uint32_t up = (lane & sft) ? 0xFFFFFFFFu : 0u;
      const int half = kept / 2;
#pragma unroll
      for (int j = 0; j < NV / 2; ++j) {
        if (j < half) {
          const uint32_t a = __float_as_uint(av[j]), bb = __float_as_uint(av[j + half]);
          const float keep = __uint_as_float((bb & up) | (a & ~up));
          const float send = __uint_as_float((a & up) | (bb & ~up));
          av[j] = keep + __shfl_xor(send, sft, 64);
        }
      }
      kept = half;
    }
    {
      // lane's row group q = lane / LPR selects which block of NV/RG values it owns
      const int q = lane / LPR;
      int owner = 0;
#pragma unroll
      for (int bit = RG / 2, sft = 32; bit >= 1; bit >>= 1, sft >>= 1)
        if (lane & sft) owner += bit;
      (void)q;
#pragma unroll
      for (int j = 0; j < NV / RG; ++j) {
        const int vi = owner * (NV / RG) + j;
        red_acc[wave][vi / EPL][col * EPL + (vi % EPL)] = av[j];
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

}

// One workgroup per (sequence, group): thread x handles outputs x, x + 256 of
// the group's G*D.  The partials are folded in slot order with the usual
// online rescaling, loading BATCH slots at a time before using any of them.
template <typename T, int D, int G>
__global__ void __launch_bounds__(kDecThreads)
decode_merge_kernel(int Hkv, int k, const float* __restrict__ part, T* __restrict__ o,
                    float* __restrict__ lse) {
  constexpr int PF = DecPartial<G, D>::kFloats;
  constexpr int PER = (G * D + kDecThreads - 1) / kDecThreads;
  constexpr int BATCH = 24;  // k = 16 or 23: one round trip of loads
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  const float* base = part + row * (k + 1) * static_cast<size_t>(PF);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int x = tid + e * kDecThreads;
    if (x >= G * D) break;
    const int g = x / D;
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int u0 = 0; u0 <= k; u0 += BATCH) {
      float mv[BATCH], lv[BATCH], av[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int u = u0 + j;
        mv[j] = -INFINITY;
        lv[j] = 0.f;
        av[j] = 0.f;
        if (u <= k) {
          const float* pu = base + static_cast<size_t>(u) * PF;
          mv[j] = pu[G * D + g];
          lv[j] = pu[G * D + G + g];
          av[j] = pu[x];
        }
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        if (mv[j] == -INFINITY) continue;  // empty slot
        const float mn = fmaxf(M, mv[j]);
        const float so = exp2f(M - mn), w = exp2f(mv[j] - mn);
        L = L * so + w * lv[j];
        A = A * so + w * av[j];
        M = mn;
      }
    }
    store_scalar<T>(o + (row * G) * static_cast<size_t>(D) + x, A / L);
    if (lse && (x % D) == 0) lse[row * G + g] = M * kLn2 + logf(L);
  }
}

// workspace: partials[B*Hkv*(k+1)*G*(d+2)] fp32
size_t decode_ws_bytes(const sas_dims& d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  return rows * (d.top_k + 1) * G * (d.head_dim + 2) * sizeof(float);
}

template <typename T, int D, int G>
static sas_status launch_dec(const sas_dims& d, const void* q, const void* K, const void* V,
                             const int32_t* seq_lens, const int32_t* idx, const float* log_gate,
                             float scale, void* o, float* lse, void* ws, hipStream_t st) {
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL((decode_split_kernel<T, D, G>), dim3(d.top_k + 1, d.n_kv_heads, d.batch),
                     dim3(kDecThreads), 0, st, static_cast<const T*>(q),
                     static_cast<const T*>(K), static_cast<const T*>(V), seq_lens, idx, log_gate,
                     scale * kLog2e, d.n_kv_heads, d.t_max, d.top_k, part);
  sas_status s = check_launch("decode_split");
  if (s != SAS_OK) return s;
  hipLaunchKernelGGL((decode_merge_kernel<T, D, G>), dim3(d.n_kv_heads, d.batch),
                     dim3(kDecThreads), 0, st, d.n_kv_heads, d.top_k, part, static_cast<T*>(o),
                     lse);
  return check_launch("decode_merge");
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
