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
//     forward): recompute S^T = K Q^T, dP^T = V dO^T, dS^T; dQ^T += K^T dS^T
//     (K^T read from the row-major K tile with the LDS transpose read).
//  3. KV-outer (one workgroup per key block x group): the workgroup finds the
//     tiles that selected its block (binary search in each later tile's
//     ascending idx row) plus the diagonal tile, then for every such tile and
//     head recomputes S = Q K^T, dP = dO V^T, dS, and accumulates
//     dV^T += dO^T P and dK^T += Q^T dS in registers: for d = 128 each wave
//     owns 16 tokens of the block for all heads, the gathered Q/dO rows
//     arriving by LDS DMA several steps ahead (bwd_dkdv_ts_kernel); for
//     d = 64 one wave per head owns all 64 tokens (bwd_dkdv_kernel).  It is
//     the only writer of dK/dV for its block and of the dlog_gate entries
//     that point at it, which it sums in a fixed order.
#include <climits>
#include <type_traits>

#include "sas_device.h"
#include "sas_internal.h"
#include "sas_mfma.h"

namespace sas {

// Per-query selection: union bitmaps of 32 words (blocks < 1024) and the
// number of gate rows per (sequence, group) (see bwd_qsel_prep_kernel).
constexpr int kUnionWords = kMaxTileRows / 32;
__host__ __device__ inline size_t qsel_rows(int n_tiles) {
  return 1 + static_cast<size_t>(n_tiles) * (n_tiles - 1) / 2;
}

// ------------------------------------------------------------ zeroing ---
// The per-query backward's block counts start at zero (a kernel, not a
// memset, so that the backward can be captured in a graph).
__global__ void __launch_bounds__(256) bwd_zero_kernel(int* __restrict__ p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

// ------------------------------------------------------------ dQ pass ---
// PQ (one selection per query): the workgroup walks the union of its tile's
// per-query selections (from the prep bitmap), each lane takes its own
// query's gate for the block (-inf where the query did not select it) from a
// cursor into the query's ascending idx row, and at a block its query selected
// it stores the sum of dS over the block's 64 tokens for its head:
// part[b,h,i,slot], which bwd_qsel_dlg_kernel sums over the group's heads.
//
// The pass also forms D_i = dO_i . O_i of its queries (each lane pair holds
// the query's dO row as its B operand; the O row comes with it) and stores
// it for the dK/dV pass, and with one selection per tile it zeroes the
// tile's dlog_gate row (the dK/dV pass then writes the valid slots).
template <int D, int HPW, bool PQ>
__global__ void __launch_bounds__(128 * HPW)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
              const uint16_t* __restrict__ dO, const float* __restrict__ lse,
              float* __restrict__ Dq, int S, int Hkv, int G, int t_max, int n_tiles, int k,
              const int32_t* __restrict__ idx, const float* __restrict__ log_gate, float scale2,
              float scale, const uint32_t* __restrict__ ubits, float* __restrict__ part,
              float* __restrict__ dlg, uint16_t* __restrict__ dQ) {
  constexpr int NT = 128 * HPW;
  constexpr int KS = D / 16, CT = D / 32;
  // two buffers: block i is staged in buffer i % 2 while block i-1 is used
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * kRowStride<D>];  // K, row reads
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][64 * kTrStride<D>];   // K, transpose reads
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][64 * kRowStride<D>];
  __shared__ int s_blk[PQ ? kMaxTileRows + 1 : kMaxTopK + 1];
  __shared__ float s_beta[PQ ? 1 : kMaxTopK + 1];
  __shared__ int s_nblk;

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
  float Dv;                 // D = dO . O: this lane's half of the channels, then both halves
  {
    uint4 dr[KS], orow[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const size_t at = qrow_i * D + 16 * ks + 8 * hi;
      qb[ks] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4*>(Q + at) : make_uint4(0, 0, 0, 0));
      dr[ks] = qvalid ? *reinterpret_cast<const uint4*>(dO + at) : make_uint4(0, 0, 0, 0);
      orow[ks] = qvalid ? *reinterpret_cast<const uint4*>(O + at) : make_uint4(0, 0, 0, 0);
    }
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float a[8], c[8];
      Vec16<uint16_t>::unpack(orow[ks], a);
      Vec16<uint16_t>::unpack(dr[ks], c);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(a[e], c[e], acc);
      db[ks] = as_bf16x8(dr[ks]);
    }
    Dv = acc + __shfl_xor(acc, 32, 64);
    if (qvalid && hi == 0) Dq[qrow_i] = Dv;
  }
  const float lse2 = qvalid ? lse[qrow_i] * kLog2eF : 0.f;
  f32x16_t dq[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) zero16(dq[ct]);

  const size_t srow = (static_cast<size_t>(b) * Hkv + r) * n_tiles + t;
  if (!PQ && dlg && hc == 0 && wave == 0 && lane < k) dlg[srow * k + lane] = 0.f;
  const uint16_t* Kg = K + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;
  const uint16_t* Vg = V + (static_cast<size_t>(b) * Hkv + r) * static_cast<size_t>(t_max) * D;

  // PQ: cursor into the lane's query's ascending selection (next selected
  // block, its slot and log2-scaled gate; INT_MAX once the row is exhausted)
  const size_t qsel = PQ ? ((static_cast<size_t>(b) * Hkv + r) * S + (qvalid ? qi : 0)) * k : 0;
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
  if constexpr (PQ) fetch();

  // block list: the valid selected blocks (in slot order), then the diagonal;
  // PQ: the union of the tile's selections in ascending order
  if (PQ && wave == 0) {
    uint32_t w = lane < kUnionWords ? ubits[srow * kUnionWords + lane] : 0u;
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
  } else if (!PQ && wave == 0) {
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
  __syncthreads();
  const int nblk = s_nblk;
  // Per-query mode: K (twice: row-read and transpose-read strides) and V of a
  // block are staged by LDS DMA (global_load_lds_dwordx4), which keeps the
  // kernel's registers (the gate cursor takes a few more) clear of staging
  // values: 238 VGPRs and no spill, 4150 -> 3680 us at S = 16384.  (With
  // one selection per tile the register staging below measured faster:
  // 509 against 536 us.)  One copy instruction fills
  // 64 consecutive 16-byte positions of a padded tile, so a row of RS
  // elements takes RS / 8 positions and a tile RS / 8 instructions; a lane
  // whose position is row padding fetches the row's first chunk again.  Rows
  // past the sequence end repeat its last row (finite; their probabilities
  // are masked to zero).  Block i + 1 is copied into the other buffer while
  // block i computes.
  constexpr int NW = NT / 64;
  auto copy_tile = [&](const uint16_t* src, int valid, uint32_t dst, auto rs_tag) {
    constexpr int RS = decltype(rs_tag)::value, POS = RS / 8;
#pragma unroll
    for (int n = 0; n < (POS + NW - 1) / NW; ++n) {
      const int ins = min(wave + NW * n, POS - 1);
      const int pos = 64 * ins + lane, row = pos / POS, c = pos % POS;
      lds_dma<16>(src + static_cast<size_t>(min(row, valid - 1)) * D + 8 * (c < D / 8 ? c : 0),
                  dst + 1024 * ins);
    }
  };
  using RowTag = std::integral_constant<int, kRowStride<D>>;
  using TrTag = std::integral_constant<int, kTrStride<D>>;
  const uint32_t ks_lds = lds_addr_of(&Ks[0][0]), kt_lds = lds_addr_of(&Kt[0][0]),
                 vs_lds = lds_addr_of(&Vs[0][0]);
  auto copy_block = [&](int i, int buf) {
    const int tok = s_blk[i] * 64;
    const uint16_t* kb = Kg + static_cast<size_t>(tok) * D;
    const uint16_t* vb = Vg + static_cast<size_t>(tok) * D;
    copy_tile(kb, S - tok, ks_lds + buf * (64 * kRowStride<D> * 2), RowTag{});
    copy_tile(kb, S - tok, kt_lds + buf * (64 * kTrStride<D> * 2), TrTag{});
    copy_tile(vb, S - tok, vs_lds + buf * (64 * kRowStride<D> * 2), RowTag{});
  };
  // Tile mode: each thread's share of the block's K and V rows (16-byte
  // chunks) is loaded into registers one block ahead of its LDS store.
  constexpr int TOT = 64 * (D / 8), CH = PQ ? 1 : (TOT + NT - 1) / NT;
  uint4 kreg[CH], vreg[CH];
  auto load_block = [&](int i) {
    const int tok = s_blk[i] * 64;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int x = tid + c * NT, row = x / (D / 8), cc = x % (D / 8);
      const bool ok = x < TOT && tok + row < S;
      kreg[c] = ok ? *reinterpret_cast<const uint4*>(Kg + static_cast<size_t>(tok + row) * D + cc * 8)
                   : make_uint4(0, 0, 0, 0);
      vreg[c] = ok ? *reinterpret_cast<const uint4*>(Vg + static_cast<size_t>(tok + row) * D + cc * 8)
                   : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int x = tid + c * NT, row = x / (D / 8), cc = x % (D / 8);
      if (x < TOT) {
        lds_store_row8<kRowStride<D>>(Ks[buf], row, cc * 8, kreg[c]);
        lds_store_row8<kTrStride<D>>(Kt[buf], row, cc * 8, kreg[c]);
        lds_store_row8<kRowStride<D>>(Vs[buf], row, cc * 8, vreg[c]);
      }
    }
  };
  if constexpr (PQ) {
    copy_block(0, 0);
    dma_sync<0>();
  } else {
    load_block(0);
    store_block(0);
    __syncthreads();
  }

  for (int it = 0; it < nblk; ++it) {
    const bool diag = it == nblk - 1;
    float beta2;
    int hit_slot = -1;
    if constexpr (PQ) {
      const bool hit = nxt == s_blk[it];
      beta2 = hit ? nxt_beta : (diag ? 0.f : -INFINITY);
      if (hit) {
        hit_slot = cur++;
        fetch();
      }
    } else {
      beta2 = s_beta[it];
    }
    float dsq = 0.f;   // PQ: sum of dS over the block's tokens (this lane's rows)
    const int buf = it & 1;
    if (it + 1 < nblk) {   // lands (PQ) or is in flight (tile) while this block computes
      if constexpr (PQ) copy_block(it + 1, buf ^ 1);
      else load_block(it + 1);
    }
    const float off = beta2 - lse2;
    // one 32-token half at a time, so only one S^T / dP^T pair is live
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x16_t st, dp;
      zero16(st);
      zero16(dp);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = 32 * tt + l32, col = 16 * ks + 8 * hi;
        st = mfma32x32x16(lds_row8<kRowStride<D>>(Ks[buf], row, col), qb[ks], st);
        dp = mfma32x32x16(lds_row8<kRowStride<D>>(Vs[buf], row, col), db[ks], dp);
      }
      if (diag || !qvalid) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int tok = 32 * tt + acc_row(v, hi);
          const bool ok = qvalid && !(diag && tok > qloc);
          const float p = ok ? fast_exp2(fmaf(st[v], scale2, off)) : 0.f;
          st[v] = p * (dp[v] - Dv);  // dS^T
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) st[v] = fast_exp2(fmaf(st[v], scale2, off)) * (dp[v] - Dv);
      }
      if constexpr (PQ) {
#pragma unroll
        for (int v = 0; v < 16; ++v) dsq += st[v];
      }
      // dQ^T (D x 32 queries) += K^T dS^T over this half's k-steps j = 2tt, 2tt+1
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const bf16x8_t bop = acc_to_bop(&st, jj);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          dq[ct] = mfma32x32x16(lds_aop_tr_perm<kTrStride<D>>(Kt[buf], 32 * ct, 2 * tt + jj, hi),
                                bop, dq[ct]);
      }
    }
    if constexpr (PQ) {
      dsq += __shfl_xor(dsq, 32, 64);   // the other 32 token rows of the query
      if (hit_slot >= 0 && hi == 0)
        part[((static_cast<size_t>(b) * Hq + h) * S + qi) * k + hit_slot] = dsq;
    }
    if constexpr (PQ) {
      dma_sync<0>();   // the next block has landed; every wave is done with this one
    } else {
      if (it + 1 < nblk) store_block(buf ^ 1);
      __syncthreads();
    }
  }
  if (qvalid) store_acc_col<CT>(dq, scale, dQ + qrow_i * D, hi);
}

// The tiles that read key block m of one (sequence, group): the diagonal
// tile first, then every later tile whose ascending idx row contains m, in
// ascending tile order, with the slot and the log-gate (base 2) of the entry.
// All NWV waves of the workgroup call it; returns the entry count.
template <int NWV>
__device__ int reading_tiles(int m, int n_tiles, int k, const int32_t* __restrict__ idx_rows,
                             const float* __restrict__ lg_rows, int* list_t, int* list_slot,
                             float* list_beta, int* s_count, int* s_wcount) {
  constexpr int NT = 64 * NWV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    list_t[0] = m;
    list_slot[0] = -1;
    list_beta[0] = 0.f;
    *s_count = 1;
  }
  __syncthreads();
  for (int base = m + 1; base < n_tiles; base += NT) {
    const int t = base + tid;
    int slot = -1;
    if (t < n_tiles && k > 0) {
      const int32_t* row = idx_rows + static_cast<size_t>(t) * k;
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
    int off = *s_count;
    for (int w = 0; w < wave; ++w) off += s_wcount[w];
    if (slot >= 0) {
      list_t[off + before] = t;
      list_slot[off + before] = slot;
      list_beta[off + before] = lg_rows ? lg_rows[static_cast<size_t>(t) * k + slot] * kLog2eF : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
      int add = 0;
      for (int w = 0; w < NWV; ++w) add += s_wcount[w];
      *s_count += add;
    }
    __syncthreads();
  }
  return *s_count;
}

// ------------------------------------------- per-query selection prep ---
// With one selection per query (idx/log_gate [B,Hkv,S,k]) the backward needs,
// per (sequence, group, tile t): the union of the tile's per-query selections
// as a bitmap (32 words: blocks < 1024), the exclusive prefix counts of its
// words (the rank of a block in the union), and one row of 64 base-2 gates
// per union block: row[q] = log g of query 64t+q for that block, or -inf if
// the query did not select it.  Rows of tile t start at 1 + t(t-1)/2 (a tile
// has at most t union blocks); row 0 is all zeros (the diagonal block).

__global__ void __launch_bounds__(256)
bwd_qsel_prep_kernel(int S, int Hkv, int n_tiles, int k, const int32_t* __restrict__ idx,
                     const float* __restrict__ log_gate, uint32_t* __restrict__ ubits,
                     int* __restrict__ ucnt, float* __restrict__ table, int* __restrict__ qcnt) {
  __shared__ uint32_t bits[kUnionWords];
  __shared__ int cnt[kUnionWords];
  __shared__ int bcnt[kMaxTileRows];   // queries of this tile selecting each block
  const int t = blockIdx.x, r = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const size_t grow = static_cast<size_t>(b) * Hkv + r;
  const size_t qrow0 = grow * S + static_cast<size_t>(t) * 64;
  const int n_ent = min(64, S - 64 * t) * k;
  float* tab = table + grow * qsel_rows(n_tiles) * 64;
  if (tid < kUnionWords) bits[tid] = 0u;
  for (int m = tid; m < t; m += 256) bcnt[m] = 0;
  if (t == 0 && tid < 64) tab[tid] = 0.f;   // row 0: the diagonal block's zero gates
  __syncthreads();
  for (int e = tid; e < n_ent; e += 256) {
    const int m = idx[qrow0 * k + e];
    if (m >= 0) {
      atomicOr(&bits[m >> 5], 1u << (m & 31));
      atomicAdd(&bcnt[m], 1);
    }
  }
  __syncthreads();
  // selecting queries of block m over all tiles: one integer add per (tile,
  // selected block) (order-free, so the totals are exact and reproducible)
  if (qcnt)
    for (int m = tid; m < t; m += 256)
      if (bcnt[m]) atomicAdd(&qcnt[grow * n_tiles + m], bcnt[m]);
  if (tid < 64) {
    const uint32_t w = tid < kUnionWords ? bits[tid] : 0u;
    int incl = __popc(w);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (tid >= o) incl += v;
    }
    if (tid < kUnionWords) {
      cnt[tid] = incl - __popc(w);
      ubits[(grow * n_tiles + t) * kUnionWords + tid] = w;
      ucnt[(grow * n_tiles + t) * kUnionWords + tid] = incl - __popc(w);
    }
  }
  __syncthreads();
  const int n_union = cnt[kUnionWords - 1] + __popc(bits[kUnionWords - 1]);
  float* rows = tab + (1 + static_cast<size_t>(t) * (t - 1) / 2) * 64;
  for (int i = tid; i < n_union * 64; i += 256) rows[i] = -INFINITY;
  __syncthreads();
  for (int e = tid; e < n_ent; e += 256) {
    const int m = idx[qrow0 * k + e];
    if (m >= 0) {
      const int rank = cnt[m >> 5] + __popc(bits[m >> 5] & ((1u << (m & 31)) - 1u));
      rows[rank * 64 + e / k] = log_gate ? log_gate[qrow0 * k + e] * kLog2eF : 0.f;
    }
  }
}

// dlog_gate[b,r,i,slot] = sum over the G heads of the group, in head order,
// of the dQ pass's per-(query, head, slot) partials; 0 on empty slots.
__global__ void __launch_bounds__(256)
bwd_qsel_dlg_kernel(int S, int Hkv, int G, int k, const int32_t* __restrict__ idx,
                    const float* __restrict__ part, float* __restrict__ dlg, size_t n) {
  const size_t x = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (x >= n) return;
  const int slot = static_cast<int>(x % k);
  const size_t qi = (x / k) % S, grow = x / (static_cast<size_t>(k) * S);
  const size_t b = grow / Hkv, r = grow % Hkv;
  float tot = 0.f;
  if (idx[x] >= 0)
    for (int g = 0; g < G; ++g)
      tot += part[(((b * Hkv + r) * G + g) * S + qi) * k + slot];
  dlg[x] = tot;
}

// Per-block lists of the queries that selected each key block (d = 128
// dK/dV pass under per-query selection): block m's list holds, in ascending
// query order, every query i >= 64(m+1) whose selection contains m, with its
// base-2 gate, padded with masked entries (gate -inf, a valid query index) to
// a multiple of 64; qoff[m] is where it starts.  Built in a fixed order (the
// counts by integer atomics, the lists by one workgroup per block walking
// the readers in tile order), so the dK/dV sums stay bitwise reproducible.
constexpr int kQlistScanThreads = 1024;

__global__ void __launch_bounds__(kQlistScanThreads)
bwd_qlist_scan_kernel(int n_tiles, const int* __restrict__ qcnt, int* __restrict__ qoff) {
  __shared__ int part[kQlistScanThreads / 64];
  const size_t grow = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid < n_tiles ? (qcnt[grow * n_tiles + tid] + 63) & ~63 : 0;
  int incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += part[w];
  if (tid < n_tiles) qoff[grow * (n_tiles + 1) + tid] = base + incl - c;
  if (tid == kQlistScanThreads - 1) qoff[grow * (n_tiles + 1) + n_tiles] = base + incl;
}

template <int NWV>
__device__ int reading_tiles_pq(int m, int n_tiles, const uint32_t* __restrict__ ubits,
                                const int* __restrict__ ucnt, int* list_t, int* list_row,
                                int* s_count, int* s_wcount);

__global__ void __launch_bounds__(256)
bwd_qlist_fill_kernel(int S, int Hkv, int n_tiles, size_t cap,
                      const uint32_t* __restrict__ ubits, const int* __restrict__ ucnt,
                      const float* __restrict__ gtab, const int* __restrict__ qoff,
                      int* __restrict__ qlist, float* __restrict__ qbeta) {
  constexpr int NWV = 4;
  __shared__ int list_t[kMaxTileRows];
  __shared__ int list_row[kMaxTileRows];
  __shared__ int cnt_e[kMaxTileRows];
  __shared__ int s_count;
  __shared__ int s_wcount[NWV];
  const int m = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t grow = static_cast<size_t>(b) * Hkv + r;
  const int n_list = reading_tiles_pq<NWV>(m, n_tiles, ubits + grow * n_tiles * kUnionWords,
                                           ucnt + grow * n_tiles * kUnionWords, list_t, list_row,
                                           &s_count, s_wcount);
  const float* gt = gtab + grow * qsel_rows(n_tiles) * 64;
  // pass 1: how many queries of each reading tile selected m (entry 0 is the
  // diagonal tile, not part of the list)
  for (int e = 1 + wave; e < n_list; e += NWV) {
    const bool sel = gt[static_cast<size_t>(list_row[e]) * 64 + lane] > -INFINITY;
    const int c = __popcll(__ballot(sel));
    if (lane == 0) cnt_e[e] = c;
  }
  __syncthreads();
  if (tid == 0) {   // exclusive prefix in entry (= tile) order
    int acc = 0;
    for (int e = 1; e < n_list; ++e) {
      const int c = cnt_e[e];
      cnt_e[e] = acc;
      acc += c;
    }
    cnt_e[0] = acc;   // the list length
  }
  __syncthreads();
  const int o0 = qoff[grow * (n_tiles + 1) + m], o1 = qoff[grow * (n_tiles + 1) + m + 1];
  // the lists of one (sequence, group) are contiguous in its slice of cap entries
  int* ql = qlist + grow * cap + o0;
  float* qb = qbeta + grow * cap + o0;
  // pass 2: the queries of each reading tile, in ascending order
  for (int e = 1 + wave; e < n_list; e += NWV) {
    const float g = gt[static_cast<size_t>(list_row[e]) * 64 + lane];
    const bool sel = g > -INFINITY;
    const unsigned long long mask = __ballot(sel);
    if (sel) {
      const int at = cnt_e[e] + __popcll(mask & ((1ull << lane) - 1ull));
      ql[at] = 64 * list_t[e] + lane;
      qb[at] = g;
    }
  }
  // padding: masked entries that repeat a valid query index
  const int len = cnt_e[0];
  const int pad_q = min(64 * (m + 1), S - 1);
  for (int at = len + tid; at < o1 - o0; at += 256) {
    ql[at] = pad_q;
    qb[at] = -INFINITY;
  }
}

// The readers of key block m under per-query selection: the diagonal tile
// (gate row 0) first, then every later tile whose union contains m, in
// ascending order, with the index of the gate row of (tile, m).
template <int NWV>
__device__ int reading_tiles_pq(int m, int n_tiles, const uint32_t* __restrict__ ubits,
                                const int* __restrict__ ucnt, int* list_t, int* list_row,
                                int* s_count, int* s_wcount) {
  constexpr int NT = 64 * NWV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wd = m >> 5;
  const uint32_t below = (1u << (m & 31)) - 1u;
  if (tid == 0) {
    list_t[0] = m;
    list_row[0] = 0;
    *s_count = 1;
  }
  __syncthreads();
  for (int base = m + 1; base < n_tiles; base += NT) {
    const int t = base + tid;
    int row = -1;
    if (t < n_tiles) {
      const uint32_t w = ubits[static_cast<size_t>(t) * kUnionWords + wd];
      if ((w >> (m & 31)) & 1u)
        row = 1 + t * (t - 1) / 2 + ucnt[static_cast<size_t>(t) * kUnionWords + wd] +
              __popc(w & below);
    }
    const unsigned long long mask = __ballot(row >= 0);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) s_wcount[wave] = __popcll(mask);
    __syncthreads();
    int off = *s_count;
    for (int w = 0; w < wave; ++w) off += s_wcount[w];
    if (row >= 0) {
      list_t[off + before] = t;
      list_row[off + before] = row;
    }
    __syncthreads();
    if (tid == 0) {
      int add = 0;
      for (int w = 0; w < NWV; ++w) add += s_wcount[w];
      *s_count += add;
    }
    __syncthreads();
  }
  return *s_count;
}

// --------------------------------------------------------- dK/dV pass ---
// One workgroup per (key block m, group r, sequence) with up to 4 waves; wave
// w handles heads w, w + 4, ... of the group and all 64 tokens of the block,
// keeping dK^T and dV^T (channels x tokens) in accumulator registers.  K and
// V rows of the block are staged once in shared LDS (B operands of S = Q K^T
// and dP = dO V^T).  For every tile that reads the block and every head, the
// wave loads the tile's Q and dO rows straight into registers as A operands,
// then copies them into its own LDS region, from which the LDS transpose read
// yields the A operands of dK^T += Q^T dS and dV^T += dO^T P; the waves never
// wait for each other between tiles.  dlog_gate partials are summed over
// waves at the end.
// PQ (one selection per query): readers from the prep bitmaps, per-query gates
// from the prep's gate rows (loaded with lse and D), no dlog_gate here.
template <int D, int NWV, bool PQ>
__global__ void __launch_bounds__(64 * NWV)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ lse, const float* __restrict__ Dq, int S, int Hkv,
                int G, int t_max, int n_tiles, int k, const int32_t* __restrict__ idx,
                const float* __restrict__ log_gate, float scale2, float scale,
                const uint32_t* __restrict__ ubits, const int* __restrict__ ucnt,
                const float* __restrict__ gtab, uint16_t* __restrict__ dK,
                uint16_t* __restrict__ dV, float* __restrict__ dlg) {
  constexpr int NT = 64 * NWV;
  constexpr int KS = D / 16, CT = D / 32;
  // One LDS arena: K rows and V rows (row reads), then per wave the 32 query
  // rows of Q and dO of the current half tile (transpose reads).  At the end
  // it is reused for the cross-wave dK/dV sum: NWV x 32 x (D + 1) floats.
  constexpr int RS = kRowStride<D>, TS = kTrStride<D>;
  constexpr int kArena = 2 * 64 * RS + 2 * NWV * 32 * TS;   // bf16 elements
  static_assert(NWV * 32 * (D + 1) * 4 <= kArena * 2, "reduction buffer");
  __shared__ __attribute__((aligned(16))) uint16_t arena[kArena];
  uint16_t* const Ks = arena;
  uint16_t* const Vs = arena + 64 * RS;
  __shared__ int list_t[kMaxTileRows];
  __shared__ int list_slot[kMaxTileRows];
  __shared__ float dsum_s[NWV][kMaxTileRows];
  __shared__ float lse_w[NWV][64];   // per wave: lse (base 2) and D of the tile's queries
  __shared__ float dq_w[NWV][64];
  __shared__ float bq_w[PQ ? NWV : 1][64];     // PQ: the queries' base-2 gates
  __shared__ float list_beta[kMaxTileRows];   // log-gate (base 2) of each entry
  __shared__ int s_count;
  __shared__ int s_wcount[NWV];

  // Early blocks are read by many more tiles than late ones (block 0 by
  // every tile that selects it), so the grid runs block-major across the
  // groups: the heaviest workgroups of every group start first.
  const int m = static_cast<int>(blockIdx.x) / Hkv, r = static_cast<int>(blockIdx.x) % Hkv;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int Hq = Hkv * G;
  const size_t grow = static_cast<size_t>(b) * Hkv + r;

  int n_list;
  if constexpr (PQ)
    n_list = reading_tiles_pq<NWV>(m, n_tiles, ubits + grow * n_tiles * kUnionWords,
                                   ucnt + grow * n_tiles * kUnionWords, list_t, list_slot,
                                   &s_count, s_wcount);
  else
    n_list = reading_tiles<NWV>(m, n_tiles, k, idx + grow * n_tiles * k,
                                log_gate ? log_gate + grow * n_tiles * k : nullptr, list_t,
                                list_slot, list_beta, &s_count, s_wcount);
  const float* gt = PQ ? gtab + grow * qsel_rows(n_tiles) * 64 : nullptr;

  // ---- stage the block's K and V rows (B operands, shared by the waves)
  const int tok0 = 64 * m;
  stage_rows<D, NT>(K + (grow * t_max + tok0) * D, S - tok0, Ks, nullptr, tid);
  stage_rows<D, NT>(V + (grow * t_max + tok0) * D, S - tok0, Vs, nullptr, tid);
  __syncthreads();

  f32x16_t dk[2][CT], dv[2][CT];  // [token tile][channel tile]
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      zero16(dk[tt][ct]);
      zero16(dv[tt][ct]);
    }
  uint16_t* qt_s = arena + 2 * 64 * RS + wave * 32 * TS;
  uint16_t* dot_s = arena + 2 * 64 * RS + (NWV + wave) * 32 * TS;

  // lse and D of the wave's next (entry, head) pair are loaded one pair
  // ahead, so their memory latency overlaps the current pair's work
  float pre_l = 0.f, pre_d = 0.f, pre_b = 0.f;
  auto fetch_rows = [&](int e2, int g2) {
    const int q2 = 64 * list_t[e2];
    const size_t hrow2 = (static_cast<size_t>(b) * Hq + r * G + g2) * S + q2;
    const bool ok = lane < min(64, S - q2);
    pre_l = ok ? lse[hrow2 + lane] * kLog2eF : 0.f;
    pre_d = ok ? Dq[hrow2 + lane] : 0.f;
    if constexpr (PQ) pre_b = gt[static_cast<size_t>(list_slot[e2]) * 64 + lane];
  };
  if (wave < G) fetch_rows(0, wave);

  for (int e = 0; e < n_list; ++e) {
    const int t = list_t[e];
    const bool diag = e == 0;
    const float beta2 = PQ ? 0.f : list_beta[e];
    const int q0 = 64 * t;
    const int nq = min(64, S - q0);
    float dsum = 0.f;
    for (int g = wave; g < G; g += NWV) {
      const size_t hrow = (static_cast<size_t>(b) * Hq + r * G + g) * S + q0;
      lse_w[wave][lane] = pre_l;
      dq_w[wave][lane] = pre_d;
      if constexpr (PQ) bq_w[wave][lane] = pre_b;
      if (g + NWV < G) fetch_rows(e, g + NWV);
      else if (e + 1 < n_list) fetch_rows(e + 1, wave);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
#pragma unroll 1
      for (int qt = 0; qt < 2; ++qt) {
        // A operands: Q and dO rows of queries 32qt + l32
        const int qa_row = 32 * qt + l32;
        const bool qok = qa_row < nq;
        bf16x8_t qa[KS], da[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qa[ks] = as_bf16x8(qok ? *reinterpret_cast<const uint4*>(Q + (hrow + qa_row) * D + 16 * ks + 8 * hi)
                                 : make_uint4(0, 0, 0, 0));
          da[ks] = as_bf16x8(qok ? *reinterpret_cast<const uint4*>(dO + (hrow + qa_row) * D + 16 * ks + 8 * hi)
                                 : make_uint4(0, 0, 0, 0));
        }
        // S = Q K^T and dP = dO V^T (32 queries x 64 tokens)
        f32x16_t s[2], dp[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          zero16(s[tt]);
          zero16(dp[tt]);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int row = 32 * tt + l32, col = 16 * ks + 8 * hi;
            s[tt] = mfma32x32x16(qa[ks], lds_row8<RS>(Ks, row, col), s[tt]);
            dp[tt] = mfma32x32x16(da[ks], lds_row8<RS>(Vs, row, col), dp[tt]);
          }
        }
        // this half tile's Q and dO rows into the wave's LDS (row-major; the
        // dK/dV A operands read them back transposed)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          lds_store_row8<TS>(qt_s, l32, 16 * ks + 8 * hi, __builtin_bit_cast(uint4, qa[ks]));
          lds_store_row8<TS>(dot_s, l32, 16 * ks + 8 * hi, __builtin_bit_cast(uint4, da[ks]));
        }
        // P and dS (rows: queries, columns: this lane's token)
        if (diag || nq < 64 || tok0 + 64 > S) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int tok = 32 * tt + l32;
            const bool tok_ok = tok0 + tok < S;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int q = 32 * qt + acc_row(v, hi);
              const bool ok = tok_ok && q < nq && !(diag && tok > q);
              const float bb = PQ ? bq_w[PQ ? wave : 0][q] : beta2;
              const float p = ok ? fast_exp2(fmaf(s[tt][v], scale2, bb - lse_w[wave][q])) : 0.f;
              const float ds = p * (dp[tt][v] - dq_w[wave][q]);
              s[tt][v] = p;
              dp[tt][v] = ds;
              dsum += ds;
            }
          }
        } else {
          float lo[16], dd[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int q = 32 * qt + acc_row(v, hi);
            lo[v] = (PQ ? bq_w[PQ ? wave : 0][q] : beta2) - lse_w[wave][q];
            dd[v] = dq_w[wave][q];
          }
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float p = fast_exp2(fmaf(s[tt][v], scale2, lo[v]));
              const float ds = p * (dp[tt][v] - dd[v]);
              s[tt][v] = p;
              dp[tt][v] = ds;
              dsum += ds;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // dV^T += dO^T P and dK^T += Q^T dS; k-step j = queries 32qt + 16j..
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const bf16x8_t pb = acc_to_bop(&s[tt], j);
            const bf16x8_t sb = acc_to_bop(&dp[tt], j);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              dv[tt][ct] = mfma32x32x16(lds_aop_tr_perm<TS>(dot_s, 32 * ct, j, hi), pb, dv[tt][ct]);
              dk[tt][ct] = mfma32x32x16(lds_aop_tr_perm<TS>(qt_s, 32 * ct, j, hi), sb, dk[tt][ct]);
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();  // transposed buffers are free again
      }
    }
    dsum = wave_sum_from(dsum, 1);
    if (lane == 0) dsum_s[wave][e] = dsum;
  }
  __syncthreads();
  // dlog_gate: one writer per (tile, slot) entry, heads summed in wave order
  for (int e = 1 + tid; !PQ && e < n_list; e += NT) {
    float tot = 0.f;
    for (int w = 0; w < NWV; ++w) tot += dsum_s[w][e];
    dlg[(grow * n_tiles + list_t[e]) * k + list_slot[e]] = tot;
  }
  // ---- sum dK^T / dV^T over the waves and store: per (tensor, 32-token
  // half) every wave writes its tiles to its own slice of the arena at once,
  // then all threads add the slices in wave order and store bf16 rows.
  float* red = reinterpret_cast<float*>(arena);   // [NWV][32][D + 1]
  constexpr int RSTR = D + 1;                     // the pad spreads a column over the banks
#pragma unroll
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      __syncthreads();
      float* mine = red + wave * 32 * RSTR;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          mine[l32 * RSTR + 32 * ct + acc_row(v, hi)] = which ? dv[tt][ct][v] : dk[tt][ct][v];
      __syncthreads();
      uint16_t* dst = which ? dV : dK;
      const float mul = which ? 1.f : scale;
      for (int i = tid; i < 32 * (D / 4); i += NT) {
        const int tl = i / (D / 4), c4 = (i % (D / 4)) * 4;
        const int tok = 32 * tt + tl;
        if (tok0 + tok < S) {
          uint32_t wv[4];
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            float x = 0.f;
            for (int w = 0; w < NWV; ++w) x += red[(w * 32 + tl) * RSTR + c4 + e4];
            uint32_t u = __float_as_uint(x * mul);
            u += 0x7FFFu + ((u >> 16) & 1u);
            wv[e4] = u >> 16;
          }
          uint2 pk;
          pk.x = wv[0] | (wv[1] << 16);
          pk.y = wv[2] | (wv[3] << 16);
          *reinterpret_cast<uint2*>(dst + (grow * t_max + tok0 + tok) * D + c4) = pk;
        }
      }
    }
  }
}

// ------------------------------------------ dK/dV pass, token split ---
// D = 128.  One workgroup per (key block m, group r, sequence) with four
// waves; wave w owns tokens 16w..16w+15 of the block for every head of the
// group and keeps their dK^T and dV^T (D x 16 each) in registers, so no
// cross-wave sum is needed.  The work is a sequence of steps (entry e, head
// g, query half qt).  A step's 32 Q rows, 32 dO rows and the 32 queries' lse
// and D go from global memory straight into one slot of an LDS ring (LDS
// DMA, kTsSlots slots), kTsSlots - 1 steps ahead of the step being computed,
// so the latency of these gathered rows overlaps the products of earlier
// steps; the four waves share every slot.  Two workgroups fit on a CU.
//
// Products per step and wave (v_mfma_f32_16x16x32_bf16): S = Q K^T and
// dP = dO V^T (32 queries x 16 tokens; K and V rows of the wave's tokens are
// B operands held in registers), then dV^T += dO^T P and dK^T += Q^T dS with
// the query index as the contraction: the accumulators of the two 16-query
// tiles are the B operand as they lie in the lanes, and the LDS transpose
// read yields the A operand in the same query order.
//
// Slot layout: row q (0..31) of Q or dO takes 256 bytes; its 16-byte chunk c
// sits at position c ^ f(q % 16) with f(q) = 2 (q % 8) + (q / 4) % 2.  The
// high bits 2 (q % 8) give the transpose reads (8 rows x 2 chunks per 32
// lanes) distinct chunk pairs; the low bit keeps the 16-byte row reads (16
// rows, one chunk) free of conflicts.  A low bit of q / 8 instead made the row
// reads 2-way conflicting (measured: 9.5 against 5.5 clk per wave read; the
// transpose reads take 3.2 clk with either).  The DMA writes 64 lanes x 16
// bytes contiguously, so each lane fetches the chunk that belongs at its
// position.
constexpr int kTsSlots = 4;
constexpr int kTsRow = 256;                          // bytes per Q / dO row (D = 128)
constexpr int kTsTensor = 32 * kTsRow;               // one tensor of a slot
constexpr int kTsSlot = 2 * kTsTensor + 64 * 4;      // Q, dO, lse[32], D[32]

__device__ __forceinline__ int ts_swz(int q) { return 2 * (q & 7) + ((q >> 2) & 1); }


// PQ (one selection per query): after the diagonal tile, the entries are
// groups of 64 from the block's list of selecting queries (bwd_qlist_*), so
// only (query, block) pairs that were selected are multiplied.  Each wave
// gathers its Q/dO rows by the list's query indices (scalar loads of the
// indices), wave 0 the lse and D of the 32 listed queries, and wave 1 copies
// their 32 base-2 gates into the slot (padding entries carry -inf; the
// diagonal tile takes the zero gate row 0 of the prep table).  No dlog_gate
// is formed here (the dQ pass does it).
template <int G, bool PQ>
__global__ void __launch_bounds__(256, 2)
bwd_dkdv_ts_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const float* __restrict__ lse, const float* __restrict__ Dq, int S, int Hkv,
                   int t_max, int n_tiles, int k, const int32_t* __restrict__ idx,
                   const float* __restrict__ log_gate, float scale2, float scale, int n_hot,
                   int max_chunks, float* __restrict__ hot_part, int* __restrict__ hot_cnt,
                   const float* __restrict__ gtab, const int* __restrict__ qoff,
                   const int* __restrict__ qlist, const float* __restrict__ qbeta, size_t qcap,
                   uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                   float* __restrict__ dlg) {
  constexpr int D = 128, NWV = 4, KS = D / 32, CT = D / 16;
  constexpr int SLOT = kTsSlot + (PQ ? 64 * 4 : 0);   // + the step's gates (PQ)
  __shared__ __attribute__((aligned(16))) unsigned char ring[kTsSlots * SLOT];
  __shared__ int list_t[kMaxTileRows];
  __shared__ int list_slot[kMaxTileRows];
  __shared__ float list_beta[kMaxTileRows];
  __shared__ float red[2][NWV];
  __shared__ int s_count;
  __shared__ int s_wcount[NWV];

  // Grid: first the hot blocks m < n_hot, max_chunks workgroups each (block,
  // then chunk, then group), then every other block with one workgroup.
  int m, r, chunk;
  {
    const int x = static_cast<int>(blockIdx.x), hot = n_hot * max_chunks * Hkv;
    if (x < hot) {
      m = x / (max_chunks * Hkv);
      chunk = (x / Hkv) % max_chunks;
      r = x % Hkv;
    } else {
      m = n_hot + (x - hot) / Hkv;
      chunk = 0;
      r = (x - hot) % Hkv;
    }
  }
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, i4 = lane >> 4;
  const int Hq = Hkv * G;
  const size_t grow = static_cast<size_t>(b) * Hkv + r;

  int n_list;
  int q_o0 = 0;   // PQ: start of the block's query list
  if constexpr (PQ) {
    q_o0 = qoff[grow * (n_tiles + 1) + m];
    n_list = 1 + (qoff[grow * (n_tiles + 1) + m + 1] - q_o0) / 64;
    if (tid == 0) list_t[0] = m;
    __syncthreads();
  } else {
    n_list = reading_tiles<NWV>(m, n_tiles, k, idx + grow * n_tiles * k,
                                log_gate ? log_gate + grow * n_tiles * k : nullptr, list_t,
                                list_slot, list_beta, &s_count, s_wcount);
  }
  const float* gt = PQ ? gtab + grow * qsel_rows(n_tiles) * 64 : nullptr;
  const int* qlg = PQ ? qlist + grow * qcap : nullptr;
  const float* qbg = PQ ? qbeta + grow * qcap : nullptr;
  // Hot-block chunking: a hot block read by more than kHotCap tiles is split
  // over ceil(n_list / kHotCap) workgroups, chunk c taking entries c, c + nc,
  // c + 2nc, ... (interleaved, so the chunks sweep the tiles together and
  // share them in the L2, as one workgroup's sweep would); each chunk leaves
  // an fp32 partial of dK^T/dV^T that the reduction kernel sums in chunk
  // order.  Other blocks (and hot blocks with few readers) are done by chunk
  // 0 alone.
  const bool split = m < n_hot && n_list > kHotCap;
  const int n_chunks = split ? (n_list + kHotCap - 1) / kHotCap : 1;
  const size_t hot_slot = (grow * n_hot + m) * static_cast<size_t>(max_chunks) + chunk;
  if (m < n_hot && chunk == 0 && tid == 0) hot_cnt[grow * n_hot + m] = split ? n_chunks : 0;
  if (chunk >= n_chunks) return;   // workgroup-uniform: no barrier follows for anyone
  const int n_mine = (n_list - chunk + n_chunks - 1) / n_chunks;   // entries chunk + j nc
  const int n_steps = n_mine * G * 2;
  const uint32_t ring_lds = lds_addr_of(ring);

  // ---- LDS DMA of step s2 into slot s2 % kTsSlots.  Every wave copies rows
  // 8w..8w+7 of Q and of dO (two 1 KB copies each), wave 0 also the lse and
  // D of the 32 queries.  Steps past the end repeat the last step's copies
  // (into a slot nobody reads), so every step issues the same number of
  // copies per wave and the wait counts below stay exact.  Query rows past
  // the sequence end repeat its last row (finite values; masked below).
  const int wv_s = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int s2) {
    const int sc = min(s2, n_steps - 1);
    const int qt2 = sc & 1, g2 = (sc >> 1) % G, e2 = chunk + ((sc >> 1) / G) * n_chunks;
    const int qbase = 64 * list_t[e2] + 32 * qt2;
    const size_t hrow = (static_cast<size_t>(b) * Hq + r * G + g2) * S;
    const uint32_t slot = ring_lds + (s2 % kTsSlots) * SLOT;
    // the query of each copied row: contiguous in the diagonal tile, else from
    // the block's list (wave-uniform position: scalar loads)
    const bool listed = PQ && e2 > 0;
    const int p0 = __builtin_amdgcn_readfirstlane(q_o0 + 64 * (e2 - 1) + 32 * qt2);
    int rq[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int ql = 8 * wave + 4 * n + i4;
      rq[n] = min(qbase + ql, S - 1);
    }
    if (listed) {
      const int* wl = qlg + p0 + 8 * wv_s;
      int r8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r8[j] = __builtin_amdgcn_readfirstlane(wl[j]);   // scalar loads
#pragma unroll
      for (int n = 0; n < 2; ++n)
        rq[n] = i4 == 0 ? r8[4 * n] : i4 == 1 ? r8[4 * n + 1] : i4 == 2 ? r8[4 * n + 2] : r8[4 * n + 3];
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int row0 = 8 * wave + 4 * n;
      const int ql = row0 + i4;
      const size_t src = (hrow + rq[n]) * D + 8 * (l16 ^ ts_swz(ql));
      lds_dma<16>(Q + src, slot + row0 * kTsRow);
      lds_dma<16>(dO + src, slot + kTsTensor + row0 * kTsRow);
    }
    if (wave == 0) {
      int rl = min(qbase + (lane & 31), S - 1);
      if (listed) {
        const int* wl = qlg + p0;
        int r32[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) r32[j] = __builtin_amdgcn_readfirstlane(wl[j]);
#pragma unroll
        for (int j = 0; j < 32; ++j) rl = (lane & 31) == j ? r32[j] : rl;
      }
      const float* src = (lane < 32 ? lse : Dq) + hrow + rl;
      lds_dma<4>(src, slot + 2 * kTsTensor);
    }
    if (PQ && wave == 1)   // gates of the 32 queries (lanes 32..63 repeat them)
      lds_dma<4>(listed ? qbg + p0 + (lane & 31) : gt + 32 * qt2 + (lane & 31),
                 slot + 2 * kTsTensor + 256);
  };
  // ---- K and V rows of the wave's tokens: B operands, k-step ks holds
  // channels 32ks + 8 i4 .. +7 of token 16w + l16 (zero past the sequence)
  const int tok0 = 64 * m;
  const int tok = 16 * wave + l16;
  const bool tok_ok = tok0 + tok < S;
  bf16x8_t kb[KS], vb[KS];
  {
    const size_t row = (grow * t_max + tok0 + (tok_ok ? tok : 0)) * D + 8 * i4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 kx = *reinterpret_cast<const uint4*>(K + row + 32 * ks);
      const uint4 vx = *reinterpret_cast<const uint4*>(V + row + 32 * ks);
      kb[ks] = as_bf16x8(tok_ok ? kx : make_uint4(0, 0, 0, 0));
      vb[ks] = as_bf16x8(tok_ok ? vx : make_uint4(0, 0, 0, 0));
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < kTsSlots - 1; ++s2) issue(s2);

  f32x4_t dk[CT], dv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      dk[ct][v] = 0.f;
      dv[ct][v] = 0.f;
    }

  // per-lane LDS offsets.  Row reads (A of S and dP): row 16 qtile + l16,
  // chunk 4 ks + i4.  Transpose reads (A of dV^T and dK^T): rows
  // 4 i4 + l16/4 (+16), bytes 32 ct + 8 (l16 % 4) of the row.
  const int fr = ts_swz(l16);
  const int rd_base = l16 * kTsRow + 16 * ((i4 ^ fr) & 3);
  const int rd_x = fr >> 2;
  const int q1 = 4 * i4 + (l16 >> 2);
  const int ft = ts_swz(q1);
  const int tr_base = q1 * kTsRow + 16 * (((l16 >> 1) & 1) ^ (ft & 1)) + 8 * (l16 & 1);
  const int tr_x = ft >> 1;

  float dsum = 0.f;
  int pending = -1;   // entry whose per-wave dlog_gate partials sit in red[pslot]
  int pslot = 0;
  for (int s = 0; s < n_steps; ++s) {
    // this wave's copies for step s are done once at most the copies of
    // kTsSlots - 2 later steps remain; the barrier makes every wave's copies
    // visible and frees the slot read in step s - 1 for the next copy
    if (wave == 0 || (PQ && wave == 1)) dma_sync<5 * (kTsSlots - 2)>();
    else dma_sync<4 * (kTsSlots - 2)>();
    issue(s + kTsSlots - 1);
    if (!PQ && pending >= 1 && tid == 0) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) tot += red[pslot][w];
      dlg[(grow * n_tiles + list_t[pending]) * k + list_slot[pending]] = tot;
    }
    if (pending >= 0) pending = -1;

    const int jl = (s >> 1) / G;   // the chunk's local entry number
    const int qt = s & 1, g = (s >> 1) % G, e = chunk + jl * n_chunks;
    const bool diag = e == 0;
    const float beta2 = PQ ? 0.f : list_beta[e];
    const int nq = (PQ && e > 0) ? 64 : min(64, S - 64 * list_t[e]);
    const unsigned char* slot = ring + (s % kTsSlots) * SLOT;
    const float* bq = reinterpret_cast<const float*>(slot + 2 * kTsTensor + 256);   // PQ gates
    const unsigned char* Qs = slot;
    const unsigned char* Os = slot + kTsTensor;
    const float* ls = reinterpret_cast<const float*>(slot + 2 * kTsTensor);

    // S and dP: 32 queries (two 16-row tiles) x the wave's 16 tokens
    f32x4_t sa[2], pa[2];
#pragma unroll
    for (int qtile = 0; qtile < 2; ++qtile) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sa[qtile][v] = 0.f;
        pa[qtile][v] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = qtile * 16 * kTsRow + rd_base + 64 * (ks ^ rd_x);
        const bf16x8_t qa = as_bf16x8(*reinterpret_cast<const uint4*>(Qs + off));
        const bf16x8_t oa = as_bf16x8(*reinterpret_cast<const uint4*>(Os + off));
        sa[qtile] = mfma16x16x32(qa, kb[ks], sa[qtile]);
        pa[qtile] = mfma16x16x32(oa, vb[ks], pa[qtile]);
      }
    }
    // P and dS; lane holds queries 16 qtile + 4 i4 + v of token tok
#pragma unroll
    for (int qtile = 0; qtile < 2; ++qtile)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = 16 * qtile + 4 * i4 + v;
        const int qq = 32 * qt + q;
        const bool ok = tok_ok && qq < nq && !(diag && tok > qq);
        const float p =
            ok ? fast_exp2(fmaf(sa[qtile][v], scale2, (PQ ? bq[q] : beta2) - ls[q] * kLog2eF))
               : 0.f;
        const float ds = p * (pa[qtile][v] - ls[32 + q]);
        sa[qtile][v] = p;
        pa[qtile][v] = ds;
        dsum += ds;
      }
    bf16x8_t pb, sb;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pb[v] = static_cast<__bf16>(sa[0][v]);
      pb[4 + v] = static_cast<__bf16>(sa[1][v]);
      sb[v] = static_cast<__bf16>(pa[0][v]);
      sb[4 + v] = static_cast<__bf16>(pa[1][v]);
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the 32 queries of the step
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int off = tr_base + 32 * (ct ^ tr_x);
      const uint2 o0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(Os + off));
      const uint2 o1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(Os + off + 16 * kTsRow));
      const uint2 x0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(Qs + off));
      const uint2 x1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(Qs + off + 16 * kTsRow));
      dv[ct] = mfma16x16x32(as_bf16x8(make_uint4(o0.x, o0.y, o1.x, o1.y)), pb, dv[ct]);
      dk[ct] = mfma16x16x32(as_bf16x8(make_uint4(x0.x, x0.y, x1.x, x1.y)), sb, dk[ct]);
    }
    // last step of the entry: the wave's dlog_gate partial
    if (!PQ && qt == 1 && g == G - 1) {
      const float w = wave_sum_from(dsum, 1);
      if (lane == 0) red[jl & 1][wave] = w;
      dsum = 0.f;
      pending = e;
      pslot = jl & 1;
    }
  }
  dma_sync<0>();
  if (!PQ && pending >= 1 && tid == 0) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) tot += red[pslot][w];
    dlg[(grow * n_tiles + list_t[pending]) * k + list_slot[pending]] = tot;
  }
  // ---- store: lane holds channels 16 ct + 4 i4 + v of token tok
  if (split) {   // fp32 partial, dK^T unscaled: [dK | dV][64 tokens][D]
    float* dst = hot_part + hot_slot * (2 * 64 * D) + tok * D + 4 * i4;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      *reinterpret_cast<float4*>(dst + 16 * ct) = make_float4(dk[ct][0], dk[ct][1], dk[ct][2], dk[ct][3]);
      *reinterpret_cast<float4*>(dst + 64 * D + 16 * ct) =
          make_float4(dv[ct][0], dv[ct][1], dv[ct][2], dv[ct][3]);
    }
  } else if (tok_ok) {
    const size_t orow = (grow * t_max + tok0 + tok) * D + 4 * i4;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      uint2 pk, pv;
      pk.x = bf16_rne(dk[ct][0] * scale) | (bf16_rne(dk[ct][1] * scale) << 16);
      pk.y = bf16_rne(dk[ct][2] * scale) | (bf16_rne(dk[ct][3] * scale) << 16);
      pv.x = bf16_rne(dv[ct][0]) | (bf16_rne(dv[ct][1]) << 16);
      pv.y = bf16_rne(dv[ct][2]) | (bf16_rne(dv[ct][3]) << 16);
      *reinterpret_cast<uint2*>(dK + orow + 16 * ct) = pk;
      *reinterpret_cast<uint2*>(dV + orow + 16 * ct) = pv;
    }
  }
}

// Sum of the chunk partials of the split hot blocks, in chunk order (one
// workgroup per (hot block, group, sequence); blocks that were not split
// have a count of 0 and were stored by their single workgroup).
__global__ void __launch_bounds__(256)
bwd_hot_reduce_kernel(const float* __restrict__ hot_part, const int* __restrict__ hot_cnt,
                      int S, int Hkv, int t_max, int n_hot, int max_chunks, float scale,
                      uint16_t* __restrict__ dK, uint16_t* __restrict__ dV) {
  constexpr int D = 128;
  const int m = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const size_t grow = static_cast<size_t>(b) * Hkv + r;
  const int nc = hot_cnt[grow * n_hot + m];
  if (nc == 0) return;
  const float* base = hot_part + (grow * n_hot + m) * static_cast<size_t>(max_chunks) * (2 * 64 * D);
  for (int i = threadIdx.x; i < 2 * 64 * D / 4; i += 256) {
    const int which = i / (64 * D / 4), rem = i % (64 * D / 4);
    const int tok = rem / (D / 4), c4 = (rem % (D / 4)) * 4;
    if (64 * m + tok >= S) continue;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < nc; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(base + static_cast<size_t>(c) * (2 * 64 * D) + 4 * static_cast<size_t>(i));
      a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
    }
    const float mul = which ? 1.f : scale;
    uint2 pk;
    pk.x = bf16_rne(a.x * mul) | (bf16_rne(a.y * mul) << 16);
    pk.y = bf16_rne(a.z * mul) | (bf16_rne(a.w * mul) << 16);
    uint16_t* dst = which ? dV : dK;
    *reinterpret_cast<uint2*>(dst + (grow * t_max + 64 * m + tok) * D + c4) = pk;
  }
}

// ------------------------------------------------------------ launcher ---
// dK/dV hot-block chunking (d = 128): blocks m < n_hot may be split into up
// to max_chunks workgroups; their fp32 partials and chunk counts follow D.
static int hot_blocks(int n_tiles) { return n_tiles < kHotBlocks ? n_tiles : kHotBlocks; }
static int hot_max_chunks(int n_tiles) { return cdiv(n_tiles, kHotCap); }
static size_t hot_part_floats(const sas_dims& d, int n_tiles) {
  return static_cast<size_t>(d.batch) * d.n_kv_heads * hot_blocks(n_tiles) *
         hot_max_chunks(n_tiles) * (2 * 64 * 128);
}
static size_t align_up256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: D [B,Hq,S] fp32 | (d = 128) hot partials | hot chunk counts;
// per-query selection adds: dlog_gate partials [B,Hq,S,k] fp32 | union bitmaps
// [B,Hkv,n_tiles,32] | their word prefix counts | gate rows
// [B,Hkv,1 + n_tiles(n_tiles-1)/2,64] fp32.
struct BwdWs {
  size_t dq, hot_part, hot_cnt, part, ubits, ucnt, gtab, qcnt, qoff, qlist, qbeta, qcap, total;
};
static BwdWs bwd_ws_layout(const sas_dims& d, int seq_len, bool pq) {
  BwdWs w{};
  const int n_tiles = cdiv(seq_len, kBlock);
  const size_t rows = static_cast<size_t>(d.batch) * d.n_q_heads * seq_len;
  const size_t groups = static_cast<size_t>(d.batch) * d.n_kv_heads;
  size_t off = 0;
  w.dq = off;
  off += rows * sizeof(float);
  if (d.head_dim == 128) {
    off = align_up256(off);
    w.hot_part = off;
    off += hot_part_floats(d, n_tiles) * sizeof(float);
    off = align_up256(off);
    w.hot_cnt = off;
    off += groups * hot_blocks(n_tiles) * sizeof(int);
  }
  if (pq) {
    off = align_up256(off);
    w.part = off;
    off += rows * static_cast<size_t>(d.top_k) * sizeof(float);
    off = align_up256(off);
    w.ubits = off;
    off += groups * n_tiles * kUnionWords * sizeof(uint32_t);
    off = align_up256(off);
    w.ucnt = off;
    off += groups * n_tiles * kUnionWords * sizeof(int);
    off = align_up256(off);
    w.gtab = off;
    off += groups * qsel_rows(n_tiles) * 64 * sizeof(float);
    // per-block lists of selecting queries (d = 128 dK/dV pass), each padded to 64
    w.qcap = static_cast<size_t>(seq_len) * d.top_k + 64 * static_cast<size_t>(n_tiles);
    off = align_up256(off);
    w.qcnt = off;
    off += groups * n_tiles * sizeof(int);
    off = align_up256(off);
    w.qoff = off;
    off += groups * (n_tiles + 1) * sizeof(int);
    off = align_up256(off);
    w.qlist = off;
    off += groups * w.qcap * sizeof(int);
    off = align_up256(off);
    w.qbeta = off;
    off += groups * w.qcap * sizeof(float);
  }
  w.total = off;
  return w;
}
size_t bwd_ws_bytes(const sas_dims& d, int seq_len) { return bwd_ws_layout(d, seq_len, false).total; }
size_t bwd_queries_ws_bytes(const sas_dims& d, int seq_len) {
  return bwd_ws_layout(d, seq_len, true).total;
}

template <int D, bool PQ>
static sas_status launch_bwd_d(const sas_dims& d, const void* Q, const void* K, const void* V,
                               const void* O, const void* dO, const float* lse, int S,
                               const int32_t* idx, const float* log_gate, float scale, void* dQ,
                               void* dK, void* dV, float* dlg, void* ws, hipStream_t st) {
  const int G = d.n_q_heads / d.n_kv_heads;
  const int n_tiles = cdiv(S, kBlock);
  const float scale2 = scale * kLog2eF;
  const BwdWs lay = bwd_ws_layout(d, S, PQ);
  char* wsb = static_cast<char*>(ws);
  float* Dq = reinterpret_cast<float*>(wsb + lay.dq);
  float* part = PQ ? reinterpret_cast<float*>(wsb + lay.part) : nullptr;
  uint32_t* ubits = PQ ? reinterpret_cast<uint32_t*>(wsb + lay.ubits) : nullptr;
  int* ucnt = PQ ? reinterpret_cast<int*>(wsb + lay.ucnt) : nullptr;
  float* gtab = PQ ? reinterpret_cast<float*>(wsb + lay.gtab) : nullptr;
  const bool qlists = PQ && D == 128;   // the d = 128 dK/dV pass walks per-block query lists
  int* qcnt = qlists ? reinterpret_cast<int*>(wsb + lay.qcnt) : nullptr;
  int* qoff = qlists ? reinterpret_cast<int*>(wsb + lay.qoff) : nullptr;
  int* qlist = qlists ? reinterpret_cast<int*>(wsb + lay.qlist) : nullptr;
  float* qbeta = qlists ? reinterpret_cast<float*>(wsb + lay.qbeta) : nullptr;
  const size_t groups = static_cast<size_t>(d.batch) * d.n_kv_heads;
  // D = rowsum(dO * O) is formed by the dQ pass, which also zeroes the tile
  // backward's dlog_gate; the per-query block counts are zeroed here (the
  // per-query dlog_gate is written whole by its reduction kernel).
  sas_status s = SAS_OK;
  if constexpr (PQ) {
    if (qlists) {
      const size_t n_zero = groups * n_tiles;
      hipLaunchKernelGGL(bwd_zero_kernel, dim3(static_cast<unsigned>((n_zero + 255) / 256)),
                         dim3(256), 0, st, qcnt, n_zero);
      s = check_launch("bwd_zero");
      if (s != SAS_OK) return s;
    }
    hipLaunchKernelGGL(bwd_qsel_prep_kernel, dim3(n_tiles, d.n_kv_heads, d.batch), dim3(256), 0,
                       st, S, d.n_kv_heads, n_tiles, d.top_k, idx, log_gate, ubits, ucnt, gtab,
                       qcnt);
    s = check_launch("bwd_qsel_prep");
    if (s != SAS_OK) return s;
    if (qlists) {
      hipLaunchKernelGGL(bwd_qlist_scan_kernel, dim3(static_cast<unsigned>(groups)),
                         dim3(kQlistScanThreads), 0, st, n_tiles, qcnt, qoff);
      s = check_launch("bwd_qlist_scan");
      if (s != SAS_OK) return s;
      hipLaunchKernelGGL(bwd_qlist_fill_kernel, dim3(n_tiles, d.n_kv_heads, d.batch), dim3(256),
                         0, st, S, d.n_kv_heads, n_tiles, lay.qcap, ubits, ucnt, gtab, qoff,
                         qlist, qbeta);
      s = check_launch("bwd_qlist_fill");
      if (s != SAS_OK) return s;
    }
  }
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* kk = static_cast<const uint16_t*>(K);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  const uint16_t* dop = static_cast<const uint16_t*>(dO);
#define SAS_DQ_CASE(HPW)                                                                       \
  hipLaunchKernelGGL((bwd_dq_kernel<D, HPW, PQ>), dim3(n_tiles * (G / HPW), d.n_kv_heads,       \
                     d.batch), dim3(128 * HPW), 0, st, q, kk, v,                                \
                     static_cast<const uint16_t*>(O), dop, lse, Dq, S, d.n_kv_heads, G, d.t_max, \
                     n_tiles, d.top_k, idx, log_gate, scale2, scale, ubits, part,               \
                     (d.top_k > 0) ? dlg : nullptr, static_cast<uint16_t*>(dQ))
  switch (G) {
    case 1: SAS_DQ_CASE(1); break;
    case 2: SAS_DQ_CASE(2); break;
    default: SAS_DQ_CASE(4); break;
  }
#undef SAS_DQ_CASE
  s = check_launch("bwd_dq");
  if (s != SAS_OK) return s;
  if (PQ && d.top_k > 0 && dlg) {
    const size_t n = static_cast<size_t>(d.batch) * d.n_kv_heads * S * d.top_k;
    hipLaunchKernelGGL(bwd_qsel_dlg_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, st, S, d.n_kv_heads, G, d.top_k, idx, part, dlg, n);
    s = check_launch("bwd_qsel_dlg");
    if (s != SAS_OK) return s;
  }
  if constexpr (D == 128) {
    const int n_hot = hot_blocks(n_tiles), max_chunks = hot_max_chunks(n_tiles);
    float* hot_part = reinterpret_cast<float*>(wsb + lay.hot_part);
    int* hot_cnt = reinterpret_cast<int*>(wsb + lay.hot_cnt);
    const int grid_x = (n_hot * max_chunks + (n_tiles - n_hot)) * d.n_kv_heads;
#define SAS_DKDV_TS(GG)                                                                          \
  hipLaunchKernelGGL((bwd_dkdv_ts_kernel<GG, PQ>), dim3(grid_x, 1, d.batch), dim3(256), 0, st, q, \
                     kk, v, dop, lse, Dq, S, d.n_kv_heads, d.t_max, n_tiles, d.top_k, idx,        \
                     log_gate, scale2, scale, n_hot, max_chunks, hot_part, hot_cnt, gtab, qoff,   \
                     qlist, qbeta, lay.qcap, static_cast<uint16_t*>(dK),                           \
                     static_cast<uint16_t*>(dV), dlg)
    switch (G) {
      case 1: SAS_DKDV_TS(1); break;
      case 2: SAS_DKDV_TS(2); break;
      case 4: SAS_DKDV_TS(4); break;
      default: SAS_DKDV_TS(8); break;
    }
#undef SAS_DKDV_TS
    s = check_launch("bwd_dkdv_ts");
    if (s != SAS_OK || max_chunks == 1) return s;
    hipLaunchKernelGGL(bwd_hot_reduce_kernel, dim3(n_hot, d.n_kv_heads, d.batch), dim3(256), 0,
                       st, hot_part, hot_cnt, S, d.n_kv_heads, d.t_max, n_hot, max_chunks, scale,
                       static_cast<uint16_t*>(dK), static_cast<uint16_t*>(dV));
    return check_launch("bwd_hot_reduce");
  }
#define SAS_DKDV_CASE(NWV)                                                                     \
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NWV, PQ>), dim3(n_tiles * d.n_kv_heads, 1, d.batch),     \
                     dim3(64 * NWV), 0, st, q, kk, v, dop, lse, Dq, S, d.n_kv_heads, G, d.t_max, \
                     n_tiles, d.top_k, idx, log_gate, scale2, scale, ubits, ucnt, gtab,           \
                     static_cast<uint16_t*>(dK), static_cast<uint16_t*>(dV), dlg)
  switch (G) {
    case 1: SAS_DKDV_CASE(1); break;
    case 2: SAS_DKDV_CASE(2); break;
    default: SAS_DKDV_CASE(4); break;
  }
#undef SAS_DKDV_CASE
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
    return launch_bwd_d<128, false>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ,
                                    dK, dV, dlog_gate, ws, st);
  return launch_bwd_d<64, false>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK,
                                 dV, dlog_gate, ws, st);
}

sas_status launch_bwd_queries(const sas_dims& d, const void* Q, const void* K, const void* V,
                              const void* O, const void* dO, const float* lse, int seq_len,
                              const int32_t* idx, const float* log_gate, float scale, void* dQ,
                              void* dK, void* dV, float* dlog_gate, void* ws, hipStream_t st) {
  if (cdiv(seq_len, kBlock) > kMaxTileRows)
    return fail(SAS_ERR_UNSUPPORTED, "backward: seq_len=%d gives more than %d tiles", seq_len,
                kMaxTileRows);
  if (d.head_dim == 128)
    return launch_bwd_d<128, true>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ,
                                   dK, dV, dlog_gate, ws, st);
  return launch_bwd_d<64, true>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK,
                                dV, dlog_gate, ws, st);
}

}  // namespace sas
