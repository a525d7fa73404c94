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
#include <algorithm>
#include <climits>

#include "sas_device.h"
#include "sas_internal.h"
#include "sas_mfma.h"

namespace sas {

// Staging of one 64-token block by LDS DMA (global_load_lds_dwordx4): the K
// tile at the row-read stride and the V tile at the transpose-read stride.
// One copy instruction fills 64 consecutive 16-byte positions of a tile, so
// a padded row of RB bytes spans RB / 16 positions and a tile 64 * RB / 16
// positions, i.e. RB / 16 instructions.  Lane L of instruction n takes
// position 64 n + L: row p / (RB / 16), chunk p % (RB / 16); a lane whose
// position falls in the row padding fetches the row's first chunk again
// (its bytes land in the padding, which nobody reads).  Rows at or past the
// sequence end repeat its last row: finite values whose probabilities are
// masked to zero.  Each wave issues the same number of copies per tile
// (instructions past the last repeat it), so per-wave wait counts are exact.
template <int D, int NW>
struct DmaStage {
  static constexpr int KRB = kRowStride<D> * 2, VRB = kTrStride<D> * 2;   // bytes per row
  static constexpr int KPOS = KRB / 16, VPOS = VRB / 16;                  // positions per row
  static constexpr int KINS = KPOS, VINS = VPOS;                          // copies per tile
  static constexpr int KPW = (KINS + NW - 1) / NW, VPW = (VINS + NW - 1) / NW;   // per wave
  static constexpr int KTILE = 64 * KRB, VTILE = 64 * VRB;                // bytes per tile
  int koff[KPW], voff[VPW];   // row * D + channel of the lane's chunk (row before clamping)
  int krow[KPW], vrow[VPW];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < KPW; ++n) {
      const int p = 64 * min(wave + NW * n, KINS - 1) + lane, c = p % KPOS;
      krow[n] = p / KPOS;
      koff[n] = 8 * (c < D / 8 ? c : 0);
    }
#pragma unroll
    for (int n = 0; n < VPW; ++n) {
      const int p = 64 * min(wave + NW * n, VINS - 1) + lane, c = p % VPOS;
      vrow[n] = p / VPOS;
      voff[n] = 8 * (c < D / 8 ? c : 0);
    }
  }
  // K (or V) rows tok.. of the block, `valid` of them inside the sequence,
  // into the tile at LDS byte address `dst`.
  __device__ __forceinline__ void k(const uint16_t* Kb, int valid, uint32_t dst, int wave) const {
#pragma unroll
    for (int n = 0; n < KPW; ++n)
      lds_dma<16>(Kb + static_cast<size_t>(min(krow[n], valid - 1)) * D + koff[n],
                  dst + 1024 * min(wave + NW * n, KINS - 1));
  }
  __device__ __forceinline__ void v(const uint16_t* Vb, int valid, uint32_t dst, int wave) const {
#pragma unroll
    for (int n = 0; n < VPW; ++n)
      lds_dma<16>(Vb + static_cast<size_t>(min(vrow[n], valid - 1)) * D + voff[n],
                  dst + 1024 * min(wave + NW * n, VINS - 1));
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
// every point.  K and V tiles live in two rings of four LDS buffers (block j
// in buffer j % 4).  Iteration i reads K of block i+1 and V of block i-1 and
// starts the copies of K of block i+3 and V of block i+2: each goes into the
// buffer whose last reader ran in iteration i-2 or i-1, before the barrier
// that ends iteration i-1, and has two iterations to land.  One wait + barrier
// per iteration suffices.
//
// One selection per query (idx/log_gate [B,Hkv,S,k]), one workgroup per
// (tile, group, head chunk, sequence): the workgroup walks the union of its
// queries' selected blocks in ascending order (built from a bitmap in LDS),
// and each lane, which owns one query column, takes the bias
// of its own query for the block: log g if its query selected the block, -inf
// otherwise (the per-query mask of the pages' training kernel), found by a
// cursor into its query's ascending idx row.  Blocks no query of the tile
// selected are never visited.  The running max starts at a finite floor so
// that a query whose first visited blocks are all masked keeps l = 0 and
// O = 0 until its first selected block.
template <int D, int HPW>
__global__ void __launch_bounds__(128 * HPW)
prefill_fwd_queries_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
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
  __shared__ int s_blk[kMaxTileRows + 1];
  __shared__ uint32_t s_bits[kMaxTileRows / 32];
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

  // block list: the union of the tile's per-query selections, ascending (a
  // bitmap, then a compaction by wave 0, lane w owning blocks 32w .. 32w+31),
  // then the diagonal
  for (int w = tid; w < kMaxTileRows / 32; w += NT) s_bits[w] = 0u;
  __syncthreads();
  const size_t qrow0 = (static_cast<size_t>(b) * Hkv + r) * S + static_cast<size_t>(t) * 64;
  const int n_ent = min(64, S - t * 64) * k;
  for (int e = tid; e < n_ent; e += NT) {
    const int m = idx[qrow0 * k + e];
    if (m >= 0) atomicOr(&s_bits[m >> 5], 1u << (m & 31));
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kMaxTileRows / 32 ? s_bits[lane] : 0u;
    const int cnt = __popc(w);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int pos = incl - cnt;
    while (w) {
      s_blk[pos++] = 32 * lane + (__ffs(w) - 1);
      w &= w - 1u;
    }
    const int total = __shfl(incl, 63, 64);
    if (lane == 0) {
      s_blk[total] = t;
      s_nblk = total + 1;
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
  float m_run = -1e30f, l_run = 0.f;

  // cursor into the lane's query's ascending selection (next selected block
  // and its log2-scaled gate; INT_MAX once the row is exhausted)
  const size_t qsel = ((static_cast<size_t>(b) * Hkv + r) * S + (qvalid ? qi : 0)) * k;
  int cur = 0, nxt = INT_MAX;
  float nxt_beta = 0.f;
  auto fetch = [&]() {
    nxt = INT_MAX;
    if (qvalid && cur < k) {
      const int v = idx[qsel + cur];
      if (v >= 0) {
        nxt = v;
        nxt_beta = log_gate ? log_gate[qsel + cur] * kLog2eF : 0.f;
      }
    }
  };
  fetch();

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
  using Stage = DmaStage<D, NT / 64>;
  Stage stg;
  stg.init(wave, lane);
  const uint32_t ks_lds = lds_addr_of(&Ks[0][0]), vs_lds = lds_addr_of(&Vs[0][0]);
  auto copy_k = [&](int i) {
    const int tok = s_blk[min(i, nh)] * 64;
    stg.k(Kg + static_cast<size_t>(tok) * D, S - tok, ks_lds + (i & 3) * Stage::KTILE, wave);
  };
  auto copy_v = [&](int i) {
    const int tok = s_blk[min(i, nh)] * 64;
    stg.v(Vg + static_cast<size_t>(tok) * D, S - tok, vs_lds + (i & 3) * Stage::VTILE, wave);
  };
  for (int c = tid; c < 64 * kTrStride<D> / 8; c += NT)
    *reinterpret_cast<uint4*>(&Vs[3][8 * c]) = make_uint4(0, 0, 0, 0);
  // in this order the wait below leaves exactly K of block 2 and V of block 1
  // in flight; every later wait leaves the copies of the last one and a half
  // iterations (V of block i+1, K of block i+3, V of block i+2)
  copy_k(0);
  copy_v(0);
  copy_k(1);
  copy_k(2);
  copy_v(1);
  dma_sync<Stage::KPW + Stage::VPW>();

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
    const bool hit = nxt == s_blk[it];
    const float beta2 = hit ? nxt_beta : -INFINITY;
    if (hit) {
      ++cur;
      fetch();
    }
    copy_k(it + 3);
    copy_v(it + 2);
    // A: the previous block's P V, this block's max
    block_pv<D>(Vs[(it + 3) & 3], p_prev, acc, hi);
    update_max(beta2);
    // B: the next block's scores, this block's probabilities, staging of
    // block it+2 and the loads of block it+3
    f32x16_t s_next[2];
    block_scores<D>(Ks[(it + 1) & 3], qb, s_next, l32, hi);
    probabilities(beta2);
    // K of block it+2 (read next) and V of block it (read next) have landed
    dma_sync<2 * Stage::VPW + Stage::KPW>();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) s_cur[tt] = s_next[tt];
  }
  // V of the diagonal block (and the copies past the list) have landed;
  // nothing is left in flight when the workgroup ends
  dma_sync<0>();
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

// Tile selection, persistent form: one workgroup per CU walks the work items
// w = blockIdx.x, blockIdx.x + gridDim.x, ... (item = tile, group, head chunk,
// sequence; heaviest tiles first), with the per-item arithmetic of
// prefill_fwd_queries_kernel, which therefore gives the same bits when every
// query of a tile carries the tile's selection.  The staged blocks
// of consecutive items continue one ring sequence (block i of an item sits in
// buffer (base + i) % 4), so while an item finishes its diagonal block the
// next item's block list is in LDS (its idx row loaded early into wave 0's
// registers), its Q rows are on their way into registers (no longer needed
// by the item finishing) and its first K/V copies are in flight into buffers
// the finishing item no longer reads.  The first P V of an item runs on the
// previous item's diagonal V tile with P = 0 (finite data), so only the very
// first item needs a zeroed buffer.  4% faster than one workgroup per item at
// S = 16384 (335 against 350 us).
template <int D, int HPW>
__global__ void __launch_bounds__(128 * HPW)
prefill_fwd_persistent_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                              const uint16_t* __restrict__ V, int S, int Hkv, int G, int t_max,
                              int n_tiles, int k, int batch, const int32_t* __restrict__ idx,
                              const float* __restrict__ log_gate, float scale2,
                              uint16_t* __restrict__ O, float* __restrict__ lse) {
  constexpr int NT = 128 * HPW;
  constexpr int KS = D / 16;
  constexpr int CT = D / 32;
  constexpr int NBUF = 4;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NBUF][64 * kRowStride<D>];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NBUF][64 * kTrStride<D>];
  __shared__ int s_blk[kMaxTopK + 1];
  __shared__ float s_beta[kMaxTopK + 1];
  __shared__ int s_nblk;

  const int nhc = G / HPW;
  const int per_t = Hkv * batch * nhc;   // items per tile
  const int n_items = n_tiles * per_t;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int Hq = Hkv * G;
  int w = blockIdx.x;
  if (w >= n_items) return;   // workgroup-uniform
  auto coords = [&](int ww, int& t, int& r, int& b, int& hc) {
    t = n_tiles - 1 - ww / per_t;
    int rem = ww % per_t;
    hc = rem % nhc;
    rem /= nhc;
    r = rem % Hkv;
    b = rem / Hkv;
  };
  // wave 0: an item's idx / log_gate row, loaded ahead into registers, then
  // written to the LDS block list (valid slots in order, then the diagonal)
  int pf_idx = -1;
  float pf_lg = 0.f;
  auto prefetch_list = [&](int ww) {
    int t, r, b, hc;
    coords(ww, t, r, b, hc);
    const size_t srow = (static_cast<size_t>(b) * Hkv + r) * n_tiles + t;
    pf_idx = lane < k ? idx[srow * k + lane] : -1;
    pf_lg = (lane < k && log_gate) ? log_gate[srow * k + lane] : 0.f;
  };
  auto commit_list = [&](int t) {
    const bool ok = lane < k && pf_idx >= 0;
    const unsigned long long mask = __ballot(ok);
    if (ok) {
      const int pos = __popcll(mask & ((1ull << lane) - 1ull));
      s_blk[pos] = pf_idx;
      s_beta[pos] = log_gate ? pf_lg * kLog2eF : 0.f;
    }
    if (lane == 0) {
      const int nv = __popcll(mask);
      s_blk[nv] = t;
      s_beta[nv] = 0.f;
      s_nblk = nv + 1;
    }
  };
  auto kv_rows = [&](const uint16_t* X, int b, int r) {
    return X + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;
  };
  bf16x8_t qb[KS];  // B operand of S^T = K Q^T: Q[qi][16ks + 8hi .. +8]
  auto load_q = [&](int t, int r, int b, int hc) {
    const int h = r * G + hc * HPW + (wave >> 1);
    const int qi = t * 64 + (wave & 1) * 32 + l32;
    const bool qvalid = qi < S;
    const uint16_t* qrow =
        Q + ((static_cast<size_t>(b) * Hq + h) * S + (qvalid ? qi : 0)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4*>(qrow + 16 * ks)
                                : make_uint4(0, 0, 0, 0));
  };
  using Stage = DmaStage<D, NT / 64>;
  Stage stg;
  stg.init(wave, lane);
  const uint32_t ks_lds = lds_addr_of(&Ks[0][0]), vs_lds = lds_addr_of(&Vs[0][0]);
  // block i of the current list (clamped to the diagonal nh) into ring slot `slot`
  auto copy_k = [&](const uint16_t* Kg, int nh, int i, int slot) {
    const int tok = s_blk[min(i, nh)] * 64;
    stg.k(Kg + static_cast<size_t>(tok) * D, S - tok, ks_lds + (slot & 3) * Stage::KTILE, wave);
  };
  auto copy_v = [&](const uint16_t* Vg, int nh, int i, int slot) {
    const int tok = s_blk[min(i, nh)] * 64;
    stg.v(Vg + static_cast<size_t>(tok) * D, S - tok, vs_lds + (slot & 3) * Stage::VTILE, wave);
  };
  // the first copies of an item (ring slots base ..): in this order the wait
  // that starts the item leaves at most K of block 2 and V of block 1 in flight
  auto first_copies = [&](const uint16_t* Kg, const uint16_t* Vg, int nh, int base) {
    copy_k(Kg, nh, 0, base);
    copy_v(Vg, nh, 0, base);
    copy_k(Kg, nh, 1, base + 1);
    copy_k(Kg, nh, 2, base + 2);
    copy_v(Vg, nh, 1, base + 1);
  };

  int t, r, b, hc;
  coords(w, t, r, b, hc);
  if (wave == 0) {
    prefetch_list(w);
    commit_list(t);
  }
  for (int c = tid; c < 64 * kTrStride<D> / 8; c += NT)
    *reinterpret_cast<uint4*>(&Vs[3][8 * c]) = make_uint4(0, 0, 0, 0);
  __syncthreads();
  load_q(t, r, b, hc);
  int base = 0;
  first_copies(kv_rows(K, b, r), kv_rows(V, b, r), s_nblk - 1, base);
  dma_sync<Stage::KPW + Stage::VPW>();

  for (;;) {
    const int h = r * G + hc * HPW + (wave >> 1);
    const int qloc = (wave & 1) * 32 + l32;
    const int qi = t * 64 + qloc;
    const bool qvalid = qi < S;
    const uint16_t* Kg = kv_rows(K, b, r);
    const uint16_t* Vg = kv_rows(V, b, r);
    const int nh = s_nblk - 1;
    const int wn = w + static_cast<int>(gridDim.x);
    const bool has_next = wn < n_items;

    f32x16_t acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) zero16(acc[ct]);
    float m_run = -INFINITY, l_run = 0.f;
    f32x16_t s_cur[2];
    block_scores<D>(Ks[base & 3], qb, s_cur, l32, hi);
    bf16x8_t p_prev[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p_prev[j] = as_bf16x8(make_uint4(0, 0, 0, 0));
    if (wave == 0 && has_next) prefetch_list(wn);

    // the online softmax, as in prefill_fwd_queries_kernel
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
      copy_k(Kg, nh, it + 3, base + it + 3);
      copy_v(Vg, nh, it + 2, base + it + 2);
      block_pv<D>(Vs[(base + it + 3) & 3], p_prev, acc, hi);
      update_max(beta2);
      f32x16_t s_next[2];
      block_scores<D>(Ks[(base + it + 1) & 3], qb, s_next, l32, hi);
      probabilities(beta2);
      dma_sync<2 * Stage::VPW + Stage::KPW>();
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) s_cur[tt] = s_next[tt];
    }
    dma_sync<0>();   // the copies past the list have landed; nobody reads the list again
    // the next item: its list, Q rows and first copies, while this one finishes
    int tn = 0, rn = 0, bn = 0, hcn = 0;
    const int nbase = base + nh + 1;
    if (has_next) {   // workgroup-uniform
      coords(wn, tn, rn, bn, hcn);
      if (wave == 0) commit_list(tn);
      __syncthreads();
      first_copies(kv_rows(K, bn, rn), kv_rows(V, bn, rn), s_nblk - 1, nbase);
      load_q(tn, rn, bn, hcn);
    }
    // the diagonal block: causal mask j > i
    block_pv<D>(Vs[(base + nh + 3) & 3], p_prev, acc, hi);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * tt + acc_row(v, hi) > qloc) s_cur[tt][v] = -INFINITY;
    update_max(0.f);
    probabilities(0.f);
    block_pv<D>(Vs[(base + nh) & 3], p_prev, acc, hi);
    if (qvalid) {
      store_acc_col<CT>(acc, 1.f / l_run, O + ((static_cast<size_t>(b) * Hq + h) * S + qi) * D, hi);
      if (hi == 0) lse[(static_cast<size_t>(b) * Hq + h) * S + qi] = (m_run + log2f(l_run)) * kLn2F;
    }
    if (!has_next) break;
    w = wn;
    t = tn;
    r = rn;
    b = bn;
    hc = hcn;
    base = nbase;
    dma_sync<Stage::KPW + Stage::VPW>();   // the item's K0, V0, K1 have landed
  }
}

size_t prefill_ws_bytes(const sas_dims&, int) { return 0; }

template <int D, bool PQ>
static sas_status launch_pf(const sas_dims& d, const void* Q, const void* K, const void* V,
                            int S, const int32_t* idx, const float* log_gate, float scale,
                            void* O, float* lse, hipStream_t st) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const int n_tiles = cdiv(S, kBlock);
  const float scale2 = scale * kLog2eF;
  // tile selection: persistent, one workgroup per CU (LDS holds one)
  int n_cu = 0;
  if (!PQ) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n_cu < 1)
      return fail(SAS_ERR_HIP, "prefill_fwd: cannot read the device's CU count");
  }
#define SAS_PF_CASE(HPW)                                                                   \
  if (PQ)                                                                                  \
    hipLaunchKernelGGL((prefill_fwd_queries_kernel<D, HPW>), dim3(n_tiles * (G / HPW),     \
                       d.n_kv_heads, d.batch), dim3(128 * HPW), 0, st,                      \
                       static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),    \
                       static_cast<const uint16_t*>(V), S, d.n_kv_heads, G, d.t_max,        \
                       n_tiles, d.top_k, idx, log_gate, scale2, static_cast<uint16_t*>(O),  \
                       lse);                                                                \
  else                                                                                     \
    hipLaunchKernelGGL((prefill_fwd_persistent_kernel<D, HPW>),                            \
                       dim3(std::min(n_cu, n_tiles * (G / HPW) * d.n_kv_heads * d.batch)), \
                       dim3(128 * HPW), 0, st, static_cast<const uint16_t*>(Q),            \
                       static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), S, \
                       d.n_kv_heads, G, d.t_max, n_tiles, d.top_k, d.batch, idx, log_gate,  \
                       scale2, static_cast<uint16_t*>(O), lse)
  switch (G) {
    case 1: SAS_PF_CASE(1); break;
    case 2: SAS_PF_CASE(2); break;
    default: SAS_PF_CASE(4); break;  // G = 4 or 8 (two head chunks)
  }
#undef SAS_PF_CASE
  return check_launch(PQ ? "prefill_fwd_queries" : "prefill_fwd");
}

sas_status launch_prefill_fwd(const sas_dims& d, const void* Q, const void* K, const void* V,
                              int seq_len, const int32_t* idx, const float* log_gate,
                              float scale, void* O, float* lse, void* ws, hipStream_t st) {
  (void)ws;
  if (d.head_dim == 128)
    return launch_pf<128, false>(d, Q, K, V, seq_len, idx, log_gate, scale, O, lse, st);
  return launch_pf<64, false>(d, Q, K, V, seq_len, idx, log_gate, scale, O, lse, st);
}

sas_status launch_prefill_fwd_queries(const sas_dims& d, const void* Q, const void* K,
                                      const void* V, int seq_len, const int32_t* idx,
                                      const float* log_gate, float scale, void* O, float* lse,
                                      hipStream_t st) {
  if (d.head_dim == 128)
    return launch_pf<128, true>(d, Q, K, V, seq_len, idx, log_gate, scale, O, lse, st);
  return launch_pf<64, true>(d, Q, K, V, seq_len, idx, log_gate, scale, O, lse, st);
}

}  // namespace sas
