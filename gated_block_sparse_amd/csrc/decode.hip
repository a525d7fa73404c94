// One decode step of gated sparse attention (SAS reproduction note, core
// formula; SAS summary, Method, fused kernel; SAS close reading 2.1-2.2):
//   z_j = q_h . k_j * scale + beta_j,   beta = log g_m on selected history
//         block m, 0 on the current block B0 (beta = 0 everywhere when the
//         gate is not passed: the inference rule of SAS close reading 2.1/2.3)
//   o_h = softmax(z) V,  lse_h = LSE(z)
//
// Split-KV: the unit of work is one or two 64-token blocks of one (sequence,
// group), taken from the k selected history blocks plus B0 (slot k).  A
// workgroup issues every K and V load of its unit at once (16-byte loads,
// every load instruction covers whole 256-byte rows), applies them to all G
// query heads of the group (each K/V byte serves G heads), and leaves an
// unnormalised partial softmax state (max, sum, acc) in the workspace.  Two
// blocks per unit are used once the grid has enough units to fill the chip:
// twice the bytes in flight per thread and half the partials to merge.  The
// partials of each head (one per unit) are merged in unit order:
//   o = sum_u e^{m_u-M} acc_u / sum_u e^{m_u-M} l_u.
// sas_decode_fwd does it in a second, small kernel that issues all of its
// loads at once (the kernel boundary orders the two).  The fused decode step
// does it in the split kernel: each unit publishes its partial (stores at
// device scope, then one atomic count per row) and the unit that arrives
// last merges the row, which saves the merge launch.  Both merges run the same
// arithmetic in slot order, so every path gives the same bits, whichever
// unit arrives last.
#include "sas_device.h"
#include "sas_internal.h"
#include "sas_select_dev.h"

namespace sas {

constexpr int kDecThreads = 256;  // 4 waves x 16 tokens = one 64-token block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int G, int D> struct DecPartial {
  // acc[G][D], then m[G] (base-2 max of z*log2e), then l[G]
  static constexpr int kFloats = G * (D + 2);
};

// Shared memory of one split unit: cross-wave max, sum and accumulators.
template <int G, int D> struct SplitLds {
  float m[4][G];
  float l[4][G];
  float acc[4][G][D];
};

// Partial states are stored and, by the fused merge, loaded at device scope
// (relaxed atomics: written through to, and read from, the level where all
// XCDs see the same data), so publishing a partial needs only the wait for
// its stores, no write-back or invalidation of a whole L2.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent2(const float* p) {   // 8-byte aligned
  const unsigned long long v = __hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)),
                     __uint_as_float(static_cast<uint32_t>(v >> 32)));
}

// Attention over the (up to NB) blocks of one unit, all G heads of group
// `row`: writes the unit's partial state to `out`.  Every thread of the
// workgroup calls it.
template <typename T, int D, int G, int NB>
__device__ __forceinline__ void split_unit(const T* __restrict__ q, const T* __restrict__ K,
                                           const T* __restrict__ V, size_t row,
                                           const size_t* brow, const int* ntok, const float* beta2,
                                           float scale2, float* __restrict__ out,
                                           SplitLds<G, D>& sh) {
  constexpr int EPL = Vec16<T>::N;      // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per wave load instruction
  constexpr int NI = 16 / RPI;          // loads per wave per tensor per block (16 tokens per wave)
  constexpr int PF = DecPartial<G, D>::kFloats;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tot = 0;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) tot += ntok[bb];
  if (tot == 0) {  // only empty slots: a neutral partial
    for (int x = tid; x < PF; x += kDecThreads)
      store_coherent(out + x, (x >= G * D && x < G * D + G) ? -INFINITY : 0.f);
    return;
  }
  const int col = lane % LPR, rsub = lane / LPR;
  uint4 kr[NB][NI], vr[NB][NI];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const T* Kb = K + brow[bb] * static_cast<size_t>(D) + col * EPL;
    const T* Vb = V + brow[bb] * static_cast<size_t>(D) + col * EPL;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = wave * 16 + i * RPI + rsub;
      if (j < ntok[bb]) {
        kr[bb][i] = *reinterpret_cast<const uint4*>(Kb + static_cast<size_t>(j) * D);
        vr[bb][i] = *reinterpret_cast<const uint4*>(Vb + static_cast<size_t>(j) * D);
      } else {
        kr[bb][i] = make_uint4(0, 0, 0, 0);
        vr[bb][i] = make_uint4(0, 0, 0, 0);
      }
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
  float z[NB][NI][G];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPL];
      Vec16<T>::unpack(kr[bb][i], kf);
      const int j = wave * 16 + i * RPI + rsub;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot += qv[h][e] * kf[e];
        dot = group_sum(dot, LPR);
        z[bb][i][h] = (j < ntok[bb]) ? dot * scale2 + beta2[bb] : -INFINITY;
      }
    }
  float mh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int i = 0; i < NI; ++i) v = fmaxf(v, z[bb][i][h]);
    mh[h] = wave_max_from(v, LPR);  // across the row groups
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) sh.m[wave][h] = mh[h];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h)
    mh[h] = fmaxf(fmaxf(sh.m[0][h], sh.m[1][h]), fmaxf(sh.m[2][h], sh.m[3][h]));

  float acc[G][EPL];
  float lh[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lh[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
#pragma unroll
  for (int bb = 0; bb < NB; ++bb)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      Vec16<T>::unpack(vr[bb][i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = fast_exp2(z[bb][i][h] - mh[h]);  // 0 for masked rows
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
    // the lane's row group selects which block of NV/RG values it owns
    int owner = 0;
#pragma unroll
    for (int bit = RG / 2, sft = 32; bit >= 1; bit >>= 1, sft >>= 1)
      if (lane & sft) owner += bit;
#pragma unroll
    for (int j = 0; j < NV / RG; ++j) {
      const int vi = owner * (NV / RG) + j;
      sh.acc[wave][vi / EPL][col * EPL + (vi % EPL)] = av[j];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) sh.l[wave][h] = lh[h];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += kDecThreads) {
    const int h = x / D, c = x % D;
    store_coherent(out + x, sh.acc[0][h][c] + sh.acc[1][h][c] + sh.acc[2][h][c] + sh.acc[3][h][c]);
  }
  if (tid < G) {
    store_coherent(out + G * D + tid, mh[tid]);
    store_coherent(out + G * D + G + tid, sh.l[0][tid] + sh.l[1][tid] + sh.l[2][tid] + sh.l[3][tid]);
  }
}

// The merge's arithmetic for one output pair (x, x+1) of head g, in slot
// order, shared by the merge kernel and the fused merge:
//   M = max_u m_u,  w_u = 2^(m_u - M),  o = sum_u w_u acc_u / sum_u w_u l_u,
// with w_u = 0 for an empty slot (m_u = -inf).
__device__ __forceinline__ void merge_fold(float mu, float lu, float2 a, float M, float& L,
                                           float& A0, float& A1) {
  const float w = fast_exp2(mu - M);
  L = fmaf(w, lu, L);
  A0 = fmaf(w, a.x, A0);
  A1 = fmaf(w, a.y, A1);
}
template <typename T>
__device__ __forceinline__ void merge_store(float M, float L, float A0, float A1, T* op,
                                            float* lse_g) {
  const float inv = 1.f / L;
  store_scalar<T>(op, A0 * inv);
  store_scalar<T>(op + 1, A1 * inv);
  if (lse_g) *lse_g = fmaf(M, kLn2, logf(L));
}

constexpr int kMergeMaxSlots = kMaxTopK + 1;
constexpr int kFusedMergeSlots = 17;  // accumulator slots per round trip in the fused merge

// Fused merge: called by every thread of the unit that arrived last, once
// the other units' partials are visible.  The (max, sum) pairs of all slots
// go to LDS (ml), the accumulators come kFusedMergeSlots slots per round trip
// (the first batch together with the pairs), which bounds the registers the
// split kernel needs for it.
template <typename T, int D, int G>
__device__ __forceinline__ void fused_merge(int ns, const float* __restrict__ base,
                                            T* __restrict__ o_row, float* __restrict__ lse_row,
                                            float (*ml)[2 * G]) {
  constexpr int PF = DecPartial<G, D>::kFloats;
  constexpr int SB = kFusedMergeSlots;
  const int tid = threadIdx.x;
  float2 av[SB];
  auto load_batch = [&](int x, int u0) {
#pragma unroll
    for (int j = 0; j < SB; ++j)
      if (u0 + j < ns) av[j] = load_coherent2(base + static_cast<size_t>(u0 + j) * PF + x);
  };
  if (2 * tid < G * D) load_batch(2 * tid, 0);
  for (int i = tid; i < ns * 2 * G; i += kDecThreads) {
    const int u = i / (2 * G), j = i % (2 * G);
    ml[u][j] = load_coherent(base + static_cast<size_t>(u) * PF + G * D + j);
  }
  __syncthreads();
  for (int x = 2 * tid; x < G * D; x += 2 * kDecThreads) {
    if (x != 2 * tid) load_batch(x, 0);
    const int g = x / D;
    float M = -INFINITY;
    for (int u = 0; u < ns; ++u) M = fmaxf(M, ml[u][g]);
    float L = 0.f, A0 = 0.f, A1 = 0.f;
    for (int u0 = 0; u0 < ns; u0 += SB) {
      if (u0 > 0) load_batch(x, u0);
#pragma unroll
      for (int j = 0; j < SB; ++j)
        if (u0 + j < ns) merge_fold(ml[u0 + j][g], ml[u0 + j][G + g], av[j], M, L, A0, A1);
    }
    merge_store<T>(M, L, A0, A1, o_row + x, (lse_row && (x % D) == 0) ? lse_row + g : nullptr);
  }
}

// The end of a split unit with a fused merge (cnt non-null; the row's count
// starts at zero): publish this unit's partial (its device-scope stores have
// completed once every wave has waited for them), count it with one atomic
// add, and merge the row in the unit that arrives last, reading the
// partials at device scope.  No unit waits for another.
template <typename T, int D, int G>
__device__ __forceinline__ void publish_and_merge(int* __restrict__ cnt, size_t row, int n_units,
                                                  const float* __restrict__ part,
                                                  T* __restrict__ o, float* __restrict__ lse,
                                                  SplitLds<G, D>& sh, int& s_last) {
  constexpr int PF = DecPartial<G, D>::kFloats;
  static_assert(sizeof(sh.acc) >= sizeof(float) * kMergeMaxSlots * 2 * G, "merge pairs fit");
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cnt + row, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             n_units - 1;
  __syncthreads();
  if (!s_last) return;   // workgroup-uniform
  fused_merge<T, D, G>(n_units, part + row * n_units * static_cast<size_t>(PF),
                       o + (row * G) * static_cast<size_t>(D), lse ? lse + row * G : nullptr,
                       reinterpret_cast<float (*)[2 * G]>(&sh.acc[0][0][0]));
}

// Split kernel of sas_decode_fwd: the unit's blocks come from idx/log_gate.
template <typename T, int D, int G, int NB>
__global__ void __launch_bounds__(kDecThreads)
decode_split_kernel(const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V,
                    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ idx,
                    const float* __restrict__ log_gate, int gated, float scale2, int Hkv,
                    int t_max, int k, KvPages pg, float* __restrict__ part,
                    int* __restrict__ cnt, T* __restrict__ o, float* __restrict__ lse) {
  constexpr int PF = DecPartial<G, D>::kFloats;
  __shared__ SplitLds<G, D> sh;
  __shared__ int s_last;
  const int unit = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  const int n_units = (k + NB) / NB;   // ceil((k + 1) / NB)
  // All the small loads of the unit are issued together, with no branch
  // between them (slot indices clamped into range; idx and log_gate always
  // point at readable memory, see the launcher), so they cost one memory
  // round trip before the K/V loads instead of a chain of them.
  int mi[NB];
  float lgi[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const size_t at = row * k + min(unit * NB + bb, k > 0 ? k - 1 : 0);
    mi[bb] = idx[at];
    lgi[bb] = log_gate[at];
  }
  const int len = clamp_len(seq_lens[b], t_max);
  const int C = (len - 1) / kBlock;
  // the NB slots of this unit: history slots u < k, then B0 as slot k
  size_t brow[NB];
  int ntok[NB];
  float beta2[NB];  // bias, already multiplied by log2(e)
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int u = unit * NB + bb;
    const bool hist = u < k && mi[bb] >= 0, cur = u == k;
    brow[bb] = (hist || cur) ? kv_block_row(pg, b, r, hist ? mi[bb] : C, Hkv, t_max) : 0;
    ntok[bb] = hist ? kBlock : (cur ? len - C * kBlock : 0);
    beta2[bb] = (hist && gated) ? lgi[bb] * kLog2e : 0.f;
  }
  split_unit<T, D, G, NB>(q, K, V, row, brow, ntok, beta2, scale2,
                          part + (row * n_units + unit) * static_cast<size_t>(PF), sh);
  if (cnt) publish_and_merge<T, D, G>(cnt, row, n_units, part, o, lse, sh, s_last);
}

// Split kernel of sas_decode_step: the selection of the row is finished here
// from the per-chunk state of the selection's first stage (the same merge of
// chunk (max, sum-exp) states and candidate lists as the selection's own
// merge kernel, so the outputs are identical), then the unit attends its
// blocks.  Unit 0 also stores the row's idx, log_gate and score_lse.
template <typename T, int D, int G, int NB>
__global__ void __launch_bounds__(kDecThreads)
decode_select_split_kernel(const T* __restrict__ q, const T* __restrict__ K,
                           const T* __restrict__ V, const int32_t* __restrict__ seq_lens,
                           const float2* __restrict__ cpart, const uint64_t* __restrict__ cand,
                           int nchunk, int nlist, int kc, int gated, float scale2, int Hkv,
                           int t_max, int k, KvPages pg, int32_t* __restrict__ idx,
                           float* __restrict__ log_gate, float* __restrict__ score_lse,
                           float* __restrict__ part, int* __restrict__ cnt, T* __restrict__ o,
                           float* __restrict__ lse) {
  constexpr int PF = DecPartial<G, D>::kFloats;
  extern __shared__ uint64_t keys[];   // two buffers of nlist * kc keys
  __shared__ SplitLds<G, D> sh;
  __shared__ int s_last;
  __shared__ float red[kDecThreads / 64];
  __shared__ int32_t sel_blk[kMaxTopK];
  __shared__ float sel_lg[kMaxTopK];
  const int unit = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int len = clamp_len(seq_lens[b], t_max);
  const int C = (len - 1) / kBlock;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  const int n_units = (k + NB) / NB;

  uint64_t* src = keys;
  const float lse_s = load_chunk_states(cand + row * static_cast<size_t>(nchunk * kc),
                                        cpart + row * nchunk, nchunk, nlist, kc, C, src, red);
  src = merge_sorted_lists(src, keys + nlist * kc, nlist, kc);
  write_selection(src, min(k, C), k, lse_s, sel_blk, sel_lg);
  __syncthreads();
  if (unit == 0) {
    if (tid < k) {
      idx[row * k + tid] = sel_blk[tid];
      log_gate[row * k + tid] = sel_lg[tid];
    }
    if (tid == 0) score_lse[row] = lse_s;
  }
  size_t brow[NB];
  int ntok[NB];
  float beta2[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int u = unit * NB + bb;
    brow[bb] = 0;
    ntok[bb] = 0;
    beta2[bb] = 0.f;
    if (u < k) {
      const int m = sel_blk[u];
      if (m >= 0) {
        brow[bb] = kv_block_row(pg, b, r, m, Hkv, t_max);
        ntok[bb] = kBlock;
        if (gated) beta2[bb] = sel_lg[u] * kLog2e;
      }
    } else if (u == k) {
      brow[bb] = kv_block_row(pg, b, r, C, Hkv, t_max);
      ntok[bb] = len - C * kBlock;
    }
  }
  split_unit<T, D, G, NB>(q, K, V, row, brow, ntok, beta2, scale2,
                          part + (row * n_units + unit) * static_cast<size_t>(PF), sh);
  publish_and_merge<T, D, G>(cnt, row, n_units, part, o, lse, sh, s_last);
}

// One workgroup per (sequence, group), one thread per pair of outputs (a
// wave per head at d = 128).  Every load of the kernel is issued before any
// is used: the (max, sum) pairs of all slots go to LDS, each thread's
// accumulator pairs of all slots to registers, so the merge costs a single
// round trip to memory.  Then, in slot order,
//   M = max_u m_u,  w_u = 2^(m_u - M),  o = sum_u w_u acc_u / sum_u w_u l_u.
template <typename T, int D, int G>
__global__ void __launch_bounds__(G * D / 2 < 64 ? 64 : G * D / 2)
decode_merge_kernel(int Hkv, int ns, const float* __restrict__ part, T* __restrict__ o,
                    float* __restrict__ lse) {
  constexpr int PF = DecPartial<G, D>::kFloats;
  constexpr int NT = G * D / 2 < 64 ? 64 : G * D / 2;
  __shared__ float ml[kMergeMaxSlots][2 * G];
  const int r = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  const float* base = part + row * ns * static_cast<size_t>(PF);
  const int x = 2 * tid;  // outputs x, x + 1 of head x / D
  const bool act = x < G * D;
  float2 av[kMergeMaxSlots];
#pragma unroll
  for (int u = 0; u < kMergeMaxSlots; ++u) {
    if (u < ns && act) av[u] = *reinterpret_cast<const float2*>(base + static_cast<size_t>(u) * PF + x);
  }
  for (int i = tid; i < ns * 2 * G; i += NT) {
    const int u = i / (2 * G), j = i % (2 * G);
    ml[u][j] = base[static_cast<size_t>(u) * PF + G * D + j];
  }
  __syncthreads();
  if (!act) return;
  const int g = x / D;
  float M = -INFINITY;
  for (int u = 0; u < ns; ++u) M = fmaxf(M, ml[u][g]);
  float L = 0.f, A0 = 0.f, A1 = 0.f;
#pragma unroll
  for (int u = 0; u < kMergeMaxSlots; ++u)
    if (u < ns) merge_fold(ml[u][g], ml[u][G + g], av[u], M, L, A0, A1);
  merge_store<T>(M, L, A0, A1, o + (row * G) * static_cast<size_t>(D) + x,
                 (lse && (x % D) == 0) ? lse + row * G + g : nullptr);
}

// workspace: partials[B*Hkv*(k+1)*G*(d+2)] fp32
size_t decode_ws_bytes(const sas_dims& d) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  return rows * (d.top_k + 1) * G * (d.head_dim + 2) * sizeof(float);
}

// Blocks per split workgroup: one while that leaves the grid too small to
// fill the chip, else two (more bytes in flight per thread, half the partials).
static int decode_blocks_per_unit(const sas_dims& d) {
  const long units = static_cast<long>(d.batch) * d.n_kv_heads * (d.top_k + 1);
  return units >= 1024 ? 2 : 1;
}

template <typename T, int D, int G, int NB>
static sas_status launch_dec_nb(const sas_dims& d, const void* q, const void* K, const void* V,
                                const int32_t* seq_lens, const int32_t* idx,
                                const float* log_gate, float scale, void* o, float* lse,
                                void* ws, hipStream_t st, KvPages pg = KvPages{nullptr, 0},
                                int* cnt = nullptr) {
  float* part = static_cast<float*>(ws);
  const int n_units = (d.top_k + NB) / NB;
  // k = 0 or the ungated rule may pass NULL idx / log_gate: the kernel then
  // reads (and ignores) seq_lens in their place, so its loads need no branch
  const int32_t* idx_r = d.top_k > 0 ? idx : seq_lens;
  const float* lg_r = (d.top_k > 0 && log_gate) ? log_gate : reinterpret_cast<const float*>(idx_r);
  hipLaunchKernelGGL((decode_split_kernel<T, D, G, NB>), dim3(n_units, d.n_kv_heads, d.batch),
                     dim3(kDecThreads), 0, st, static_cast<const T*>(q),
                     static_cast<const T*>(K), static_cast<const T*>(V), seq_lens, idx_r, lg_r,
                     log_gate != nullptr ? 1 : 0, scale * kLog2e, d.n_kv_heads, d.t_max,
                     d.top_k, pg, part, cnt, static_cast<T*>(o), lse);
  sas_status s = check_launch("decode_split");
  if (s != SAS_OK || cnt) return s;   // with counts, the last unit of each row merged it
  constexpr int kMergeThreads = G * D / 2 < 64 ? 64 : G * D / 2;
  hipLaunchKernelGGL((decode_merge_kernel<T, D, G>), dim3(d.n_kv_heads, d.batch),
                     dim3(kMergeThreads), 0, st, d.n_kv_heads, n_units, part, static_cast<T*>(o),
                     lse);
  return check_launch("decode_merge");
}

template <typename T, int D, int G>
static sas_status launch_dec(const sas_dims& d, const void* q, const void* K, const void* V,
                             const int32_t* seq_lens, const int32_t* idx, const float* log_gate,
                             float scale, void* o, float* lse, void* ws, hipStream_t st) {
  if (decode_blocks_per_unit(d) == 2)
    return launch_dec_nb<T, D, G, 2>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
  return launch_dec_nb<T, D, G, 1>(d, q, K, V, seq_lens, idx, log_gate, scale, o, lse, ws, st);
}

// Fused decode step: the selection's chunk stage, then (rows of more than
// one chunk) the select-merge + split kernel, whose last unit per row merges
// the row.  Large grids (two blocks per unit) run the selection's own merge
// kernel and then the plain split kernel (also merging in its last unit).
template <typename T, int D, int G, int NB>
static sas_status launch_step_nb(const sas_dims& d, const void* q, const void* K, const void* V,
                                 const int32_t* seq_lens, const float* Wq, const float* summ,
                                 const float* Wk, KvPages pg, int gated, float scale,
                                 int32_t* idx, float* log_gate, float* score_lse, void* o,
                                 float* lse, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws) + ((select_decode_ws_bytes(d) + 255) & ~size_t(255));
  float* part = reinterpret_cast<float*>(w);
  int* cnt = reinterpret_cast<int*>(w + ((decode_ws_bytes(d) + 255) & ~size_t(255)));
  // the chunk stage also zeroes the arrival counts of the split kernel's merge
  sas_status s = launch_select_decode_chunks(d, q, seq_lens, Wq, summ, K, Wk, pg, idx, log_gate,
                                             score_lse, ws, st, cnt);
  if (s != SAS_OK) return s;
  const SelectDecodeLayout L = select_decode_layout(d, ws);
  if (L.nchunk == 1)  // the chunk stage already wrote the selection
    return launch_dec_nb<T, D, G, NB>(d, q, K, V, seq_lens, idx, gated ? log_gate : nullptr,
                                      scale, o, lse, part, st, pg, cnt);
  if constexpr (NB > 1) {
    // Grids this large keep the chip busy on their own; there the redundant
    // per-workgroup merge costs more than the launch it saves, so the
    // selection's own merge kernel runs first (same outputs).
    s = launch_select_decode_merge(d, seq_lens, idx, log_gate, score_lse, ws, st);
    if (s != SAS_OK) return s;
    return launch_dec_nb<T, D, G, NB>(d, q, K, V, seq_lens, idx, gated ? log_gate : nullptr,
                                      scale, o, lse, part, st, pg, cnt);
  } else {
  const int n_units = (d.top_k + NB) / NB;
  hipLaunchKernelGGL((decode_select_split_kernel<T, D, G, NB>),
                     dim3(n_units, d.n_kv_heads, d.batch), dim3(kDecThreads),
                     2 * L.nlist * L.kc * sizeof(uint64_t), st, static_cast<const T*>(q),
                     static_cast<const T*>(K), static_cast<const T*>(V), seq_lens, L.part, L.cand,
                     L.nchunk, L.nlist, L.kc, gated, scale * kLog2e, d.n_kv_heads, d.t_max,
                     d.top_k, pg, idx, log_gate, score_lse, part, cnt, static_cast<T*>(o), lse);
  return check_launch("decode_select_split");
  }
}

template <typename T, int D, int G>
static sas_status launch_step(const sas_dims& d, const void* q, const void* K, const void* V,
                              const int32_t* seq_lens, const float* Wq, const float* summ,
                              const float* Wk, KvPages pg, int gated, float scale, int32_t* idx,
                              float* log_gate, float* score_lse, void* o, float* lse, void* ws,
                              hipStream_t st) {
  if (decode_blocks_per_unit(d) == 2)
    return launch_step_nb<T, D, G, 2>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx,
                                      log_gate, score_lse, o, lse, ws, st);
  return launch_step_nb<T, D, G, 1>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate,
                                    score_lse, o, lse, ws, st);
}

template <typename T, int D>
static sas_status step_by_group(const sas_dims& d, const void* q, const void* K, const void* V,
                                const int32_t* seq_lens, const float* Wq, const float* summ,
                                const float* Wk, KvPages pg, int gated, float scale, int32_t* idx, float* log_gate,
                                float* score_lse, void* o, float* lse, void* ws, hipStream_t st) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return launch_step<T, D, 1>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
    case 2: return launch_step<T, D, 2>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
    case 4: return launch_step<T, D, 4>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
    case 8: return launch_step<T, D, 8>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
  }
  return fail(SAS_ERR_UNSUPPORTED, "decode step: group size");
}

// workspace: the selection's | partials | one arrival count per row (int)
size_t decode_step_ws_bytes(const sas_dims& d) {
  return ((select_decode_ws_bytes(d) + 255) & ~size_t(255)) +
         ((decode_ws_bytes(d) + 255) & ~size_t(255)) +
         static_cast<size_t>(d.batch) * d.n_kv_heads * sizeof(int);
}

sas_status launch_decode_step(const sas_dims& d, const void* q, const void* K, const void* V,
                              const int32_t* seq_lens, const float* Wq, const float* summ,
                              const float* Wk, KvPages pg, int gated, float scale, int32_t* idx, float* log_gate,
                              float* score_lse, void* o, float* lse, void* ws, hipStream_t st) {
  if (d.dtype == SAS_BF16) {
    if (d.head_dim == 128)
      return step_by_group<uint16_t, 128>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
    return step_by_group<uint16_t, 64>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
  }
  if (d.head_dim == 128)
    return step_by_group<float, 128>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
  return step_by_group<float, 64>(d, q, K, V, seq_lens, Wq, summ, Wk, pg, gated, scale, idx, log_gate, score_lse, o, lse, ws, st);
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
