// Selector score, softmax gate and Top-K (SAS close reading 2.1-2.2; SAS
// summary, Method; MSA notes 4.1 for ranking the raw scores).
//
//   s_m       = qbar . summ_m,  qbar = Wq_sel . mean(q over the row) / sqrt(d_sel)
//   score_lse = LSE over the row's C history blocks
//   idx       = the min(k, C) largest s (ties -> lower m), ascending
//   log_gate  = s_idx - score_lse
//
// The score is linear in q, so the row's queries are pooled before the
// projection.  Top-K works on 64-bit keys (order-preserving score bits, then
// ~m), a strict total order, so the sort is exact and deterministic.
//
// Decode: C can reach thousands of blocks and the summary scan is the HBM
// traffic, so the row is cut into chunks of kSelChunk blocks, one workgroup
// each: score (half a wave per 128-float summary row), chunk max/sum-exp, and
// the chunk's own top-k by an LDS bitonic sort.  A second small kernel per row
// merges the chunk LSE states and the chunk candidates.
// Tiles (prefill): one workgroup per (tile, group) does everything.
#include "sas_device.h"
#include "sas_internal.h"

namespace sas {

constexpr int kSelThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max_from(v, 1);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nw; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum_from(v, 1);
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
#pragma unroll
    for (int sft = 16; sft >= 1; sft >>= 1) {
      const bool up = (l32 & sft) != 0;
#pragma unroll
      for (int j = 0; j < sft; ++j) {
        const float keep = up ? v[j + sft] : v[j];
        const float send = up ? v[j] : v[j + sft];
        v[j] = keep + __shfl_xor(send, sft, 64);
      }
    }
    const int i = base + hw + 8 * l32;
    if (i < n) sc[i] = v[0];
  }
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

// ------------------------------------------------------------- decode ---
// One launch per step: grid (chunk, group, sequence).  Every workgroup scores
// its chunk, keeps the chunk's LSE state and its top-k keys in the workspace,
// then bumps the row's arrival counter; the last workgroup of the row merges
// the states and candidates in chunk order (so the result does not depend on
// arrival order) and resets the counter to zero for the next call.
template <typename T, int D, int DS, int G>
__global__ void __launch_bounds__(kSelThreads)
select_decode_kernel(const T* __restrict__ q, const int32_t* __restrict__ seq_lens,
                     const float* __restrict__ Wq, const float* __restrict__ summ, int Hkv,
                     int t_max, int c_max, int k, int kc, int nchunk, int npow,
                     float* __restrict__ scores, unsigned* __restrict__ counters,
                     float2* __restrict__ part, uint64_t* __restrict__ cand,
                     int32_t* __restrict__ idx, float* __restrict__ log_gate,
                     float* __restrict__ score_lse) {
  __shared__ float qm[D];
  __shared__ float qs[DS];
  __shared__ float sc[kSelChunk];
  __shared__ uint64_t keys[kSelChunk];
  __shared__ float red[kSelThreads / 64];
  __shared__ int s_last;
  extern __shared__ uint64_t mkeys[];

  const int b = blockIdx.z, r = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int len = clamp_len(seq_lens[b], t_max);
  const int C = (len - 1) / kBlock;
  const int m0 = chunk * kSelChunk;
  const size_t row = static_cast<size_t>(b) * Hkv + r;
  const size_t p = row * nchunk + chunk;
  float M = -INFINITY, S = 0.f;
  if (m0 < C) {
    const int n = min(kSelChunk, C - m0);
    if (tid < D) {
      const T* qb = q + (row * G) * static_cast<size_t>(D) + tid;
      float a = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) a += load_scalar<T>(qb + h * D);
      qm[tid] = a / G;
    }
    __syncthreads();
    project_query<D, DS>(Wq, qm, qs);
    __syncthreads();
    const float* srow = summ + row * static_cast<size_t>(c_max) * DS;
    score_rows<DS>(srow + static_cast<size_t>(m0) * DS, qs, n, sc);
    __syncthreads();
    const bool valid = tid < n;
    const float s = valid ? sc[tid] : -INFINITY;
    if (scores && valid) scores[row * c_max + m0 + tid] = s;
    M = block_max(s, red);
    S = block_sum(valid ? expf(s - M) : 0.f, red);
    keys[tid] = valid ? topk_key(s, m0 + tid) : 0ull;
    bitonic_sort_desc(keys, kSelChunk);
  }
  const int kk = min(k, C);
  if (nchunk == 1) {  // the row fits one chunk: finish here
    const float lse = C > 0 ? M + logf(S) : -INFINITY;
    write_selection(keys, kk, k, lse, idx + row * k, log_gate + row * k);
    if (tid == 0) score_lse[row] = lse;
    return;
  }
  if (tid < kc) cand[p * kc + tid] = (m0 < C) ? keys[tid] : 0ull;
  if (tid == 0) part[p] = make_float2(M, S);
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(counters + row, 1u) == static_cast<unsigned>(nchunk - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const float2* pr = part + row * nchunk;
  float mloc = -INFINITY;
  for (int i = tid; i < nchunk; i += kSelThreads) mloc = fmaxf(mloc, pr[i].x);
  const float Mr = block_max(mloc, red);
  float sloc = 0.f;
  for (int i = tid; i < nchunk; i += kSelThreads) {
    const float2 v = pr[i];
    if (v.x != -INFINITY) sloc += v.y * expf(v.x - Mr);
  }
  const float L = block_sum(sloc, red);
  const float lse = C > 0 ? Mr + logf(L) : -INFINITY;
  const int ncand = nchunk * kc;
  const uint64_t* cr = cand + row * static_cast<size_t>(nchunk) * kc;
  for (int i = tid; i < npow; i += kSelThreads) mkeys[i] = i < ncand ? cr[i] : 0ull;
  bitonic_sort_desc(mkeys, npow);
  write_selection(mkeys, kk, k, lse, idx + row * k, log_gate + row * k);
  if (tid == 0) {
    score_lse[row] = lse;
    counters[row] = 0u;
  }
}

static int decode_nchunk(const sas_dims& d) {
  const int n = cdiv(d.t_max / kBlock, kSelChunk);
  return n > 0 ? n : 1;
}
static int next_pow2(int n) {
  int p = 2;
  while (p < n) p <<= 1;
  return p;
}
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: counters[rows] | part[rows*nchunk] | cand[rows*nchunk*max(k,1)]
size_t select_decode_ws_bytes(const sas_dims& d) {
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  const size_t nc = decode_nchunk(d);
  return align256(rows * sizeof(unsigned)) + align256(rows * nc * sizeof(float2)) +
         rows * nc * static_cast<size_t>(d.top_k > 0 ? d.top_k : 1) * sizeof(uint64_t);
}

template <typename T, int D, int DS, int G>
static sas_status launch_sd(const sas_dims& d, const void* q, const int32_t* seq_lens,
                            const float* Wq, const float* summ, int32_t* idx, float* log_gate,
                            float* score_lse, float* scores, void* ws, hipStream_t st) {
  const int nchunk = decode_nchunk(d);
  const int k = d.top_k;
  const int kc = k > 0 ? k : 1;
  const int npow = nchunk > 1 ? next_pow2(nchunk * kc) : 0;
  if (npow > 8192)
    return fail(SAS_ERR_UNSUPPORTED, "select: %d chunk candidates exceed the merge sort",
                nchunk * kc);
  const size_t rows = static_cast<size_t>(d.batch) * d.n_kv_heads;
  char* w = static_cast<char*>(ws);
  unsigned* counters = reinterpret_cast<unsigned*>(w);
  float2* part = reinterpret_cast<float2*>(w + align256(rows * sizeof(unsigned)));
  uint64_t* cand = reinterpret_cast<uint64_t*>(w + align256(rows * sizeof(unsigned)) +
                                               align256(rows * nchunk * sizeof(float2)));
  hipLaunchKernelGGL((select_decode_kernel<T, D, DS, G>), dim3(nchunk, d.n_kv_heads, d.batch),
                     dim3(kSelThreads), npow * sizeof(uint64_t), st, static_cast<const T*>(q),
                     seq_lens, Wq, summ, d.n_kv_heads, d.t_max, d.t_max / kBlock, k, kc, nchunk,
                     npow, scores, counters, part, cand, idx, log_gate, score_lse);
  return check_launch("select_decode");
}

// -------------------------------------------------------------- tiles ---
template <typename T, int D, int DS, int G>
__global__ void __launch_bounds__(kSelThreads)
select_tiles_kernel(const T* __restrict__ Q, int q_len, const float* __restrict__ Wq,
                    const float* __restrict__ summ, int Hkv, int c_max, int rows, int k,
                    int32_t* __restrict__ idx, float* __restrict__ log_gate,
                    float* __restrict__ score_lse, float* __restrict__ scores) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  constexpr int RG = kSelThreads / LPR;  // row groups
  __shared__ float qpart[RG][D];
  __shared__ float qm[D];
  __shared__ float qs[DS];
  __shared__ float sc[kMaxTileRows];
  __shared__ uint64_t keys[kMaxTileRows];
  __shared__ float red[kSelThreads / 64];

  const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int C = t;
  const int i0 = t * kBlock;
  const int nq = min(kBlock, q_len - i0);
  const size_t row = (static_cast<size_t>(b) * Hkv + r) * rows + t;

  // pooled query over the group's G heads and the tile's nq queries
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
    for (int e = 0; e < EPL; ++e) qpart[rg][col * EPL + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    float a = 0.f;
    for (int g = 0; g < RG; ++g) a += qpart[g][tid];
    qm[tid] = a / static_cast<float>(G * nq);
  }
  __syncthreads();
  project_query<D, DS>(Wq, qm, qs);
  __syncthreads();

  const float* srow = summ + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(c_max) * DS;
  score_rows<DS>(srow, qs, C, sc);
  __syncthreads();

  float mloc = -INFINITY;
  for (int m = tid; m < C; m += kSelThreads) mloc = fmaxf(mloc, sc[m]);
  const float M = block_max(mloc, red);
  float sloc = 0.f;
  for (int m = tid; m < C; m += kSelThreads) sloc += expf(sc[m] - M);
  const float L = block_sum(sloc, red);
  const float lse = C > 0 ? M + logf(L) : -INFINITY;
  if (scores)
    for (int m = tid; m < C; m += kSelThreads) scores[row * c_max + m] = sc[m];

  const int npow = C <= 2 ? 2 : (1 << (32 - __clz(C - 1)));
  for (int m = tid; m < npow; m += kSelThreads) keys[m] = m < C ? topk_key(sc[m], m) : 0ull;
  bitonic_sort_desc(keys, npow);
  const int kk = min(k, C);
  write_selection(keys, kk, k, lse, idx + row * k, log_gate + row * k);
  if (tid == 0) score_lse[row] = lse;
}

// ---------------------------------------------------------- dispatch ---
template <typename T, int D, int DS, int G>
struct SelDecode {
  static sas_status run(const sas_dims& d, const void* q, const int32_t* seq_lens, const float* Wq,
                        const float* summ, int32_t* idx, float* log_gate, float* score_lse,
                        float* scores, void* ws, hipStream_t st) {
    return launch_sd<T, D, DS, G>(d, q, seq_lens, Wq, summ, idx, log_gate, score_lse, scores,
                                  ws, st);
  }
};

template <typename T, int D, int DS, int G>
struct SelTiles {
  static sas_status run(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                        const float* summ, int32_t* idx, float* log_gate, float* score_lse,
                        float* scores, hipStream_t st) {
    const int rows = cdiv(q_len, kBlock);
    hipLaunchKernelGGL((select_tiles_kernel<T, D, DS, G>), dim3(rows, d.n_kv_heads, d.batch),
                       dim3(kSelThreads), 0, st, static_cast<const T*>(Q), q_len, Wq, summ,
                       d.n_kv_heads, d.t_max / kBlock, rows, d.top_k, idx, log_gate, score_lse,
                       scores);
    return check_launch("select_tiles");
  }
};

template <template <typename, int, int, int> class F, typename T, int D, int DS, typename... A>
static sas_status by_group(const sas_dims& d, A... a) {
  switch (d.n_q_heads / d.n_kv_heads) {
    case 1: return F<T, D, DS, 1>::run(d, a...);
    case 2: return F<T, D, DS, 2>::run(d, a...);
    case 4: return F<T, D, DS, 4>::run(d, a...);
    case 8: return F<T, D, DS, 8>::run(d, a...);
  }
  return fail(SAS_ERR_UNSUPPORTED, "select: group size");
}

template <template <typename, int, int, int> class F, typename T, typename... A>
static sas_status by_dims(const sas_dims& d, A... a) {
  if (d.head_dim == 64 && d.sel_dim == 64) return by_group<F, T, 64, 64>(d, a...);
  if (d.head_dim == 64 && d.sel_dim == 128) return by_group<F, T, 64, 128>(d, a...);
  if (d.head_dim == 128 && d.sel_dim == 64) return by_group<F, T, 128, 64>(d, a...);
  if (d.head_dim == 128 && d.sel_dim == 128) return by_group<F, T, 128, 128>(d, a...);
  return fail(SAS_ERR_UNSUPPORTED, "select: d=%d d_sel=%d", d.head_dim, d.sel_dim);
}

template <template <typename, int, int, int> class F, typename... A>
static sas_status by_type(const sas_dims& d, A... a) {
  if (d.dtype == SAS_BF16) return by_dims<F, uint16_t>(d, a...);
  return by_dims<F, float>(d, a...);
}

sas_status launch_select_decode(const sas_dims& d, const void* q, const int32_t* seq_lens,
                                const float* Wq, const float* summ, int32_t* idx, float* log_gate,
                                float* score_lse, float* scores, void* ws, hipStream_t st) {
  return by_type<SelDecode>(d, q, seq_lens, Wq, summ, idx, log_gate, score_lse, scores, ws, st);
}

sas_status launch_select_tiles(const sas_dims& d, const void* Q, int q_len, const float* Wq,
                               const float* summ, int32_t* idx, float* log_gate,
                               float* score_lse, float* scores, hipStream_t st) {
  return by_type<SelTiles>(d, Q, q_len, Wq, summ, idx, log_gate, score_lse, scores, st);
}

}  // namespace sas
