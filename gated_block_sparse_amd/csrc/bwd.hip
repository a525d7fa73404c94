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
//     head recomputes S = Q K^T (a lane owns one token column), dP = dO V^T,
//     dS, and accumulates dV^T += dO^T P and dK^T += Q^T dS in registers, one
//     wave per head.  It is the only writer of dK/dV for its block and of the
//     dlog_gate entries that point at it, which it sums over heads in a fixed
//     order.
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
  // two buffers: block i is staged in buffer i % 2 while block i-1 is used
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * kRowStride<D>];  // K, row reads
  __shared__ __attribute__((aligned(16))) uint16_t Kt[2][64 * kTrStride<D>];   // K, transpose reads
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][64 * kRowStride<D>];
  __shared__ int s_blk[kMaxTopK + 1];
  __shared__ float s_beta[kMaxTopK + 1];
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

  // block list: the valid selected blocks (in slot order), then the diagonal
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
  __syncthreads();
  const int nblk = s_nblk;
  // per-thread share of one block's K and V rows (16-byte chunks), loaded into
  // registers one block ahead of its LDS store
  constexpr int TOT = 64 * (D / 8), CH = (TOT + NT - 1) / NT;
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
  load_block(0);
  store_block(0);
  __syncthreads();

  for (int it = 0; it < nblk; ++it) {
    const bool diag = it == nblk - 1;
    const float beta2 = s_beta[it];
    const int buf = it & 1;
    if (it + 1 < nblk) load_block(it + 1);   // in flight while this block computes
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
    if (it + 1 < nblk) store_block(buf ^ 1);
    __syncthreads();
  }
  if (qvalid) store_acc_col<CT>(dq, scale, dQ + qrow_i * D, hi);
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
template <int D, int NWV>
__global__ void __launch_bounds__(64 * NWV)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ lse, const float* __restrict__ Dq, int S, int Hkv,
                int G, int t_max, int n_tiles, int k, const int32_t* __restrict__ idx,
                const float* __restrict__ log_gate, float scale2, float scale,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, float* __restrict__ dlg) {
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

  // ---- the tiles that read this block: the diagonal one, then every later
  // tile whose ascending idx row contains m (in ascending tile order)
  if (tid == 0) {
    list_t[0] = m;
    list_slot[0] = -1;
    list_beta[0] = 0.f;
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
    int off = s_count;
    for (int w = 0; w < wave; ++w) off += s_wcount[w];
    if (slot >= 0) {
      list_t[off + before] = t;
      list_slot[off + before] = slot;
      list_beta[off + before] = log_gate ? log_gate[(grow * n_tiles + t) * k + slot] * kLog2eF : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
      int add = 0;
      for (int w = 0; w < NWV; ++w) add += s_wcount[w];
      s_count += add;
    }
    __syncthreads();
  }
  const int n_list = s_count;

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
  float pre_l = 0.f, pre_d = 0.f;
  auto fetch_rows = [&](int e2, int g2) {
    const int q2 = 64 * list_t[e2];
    const size_t hrow2 = (static_cast<size_t>(b) * Hq + r * G + g2) * S + q2;
    const bool ok = lane < min(64, S - q2);
    pre_l = ok ? lse[hrow2 + lane] * kLog2eF : 0.f;
    pre_d = ok ? Dq[hrow2 + lane] : 0.f;
  };
  if (wave < G) fetch_rows(0, wave);

  for (int e = 0; e < n_list; ++e) {
    const int t = list_t[e];
    const bool diag = e == 0;
    const float beta2 = list_beta[e];
    const int q0 = 64 * t;
    const int nq = min(64, S - q0);
    float dsum = 0.f;
    for (int g = wave; g < G; g += NWV) {
      const size_t hrow = (static_cast<size_t>(b) * Hq + r * G + g) * S + q0;
      lse_w[wave][lane] = pre_l;
      dq_w[wave][lane] = pre_d;
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
              const float p = ok ? fast_exp2(fmaf(s[tt][v], scale2, beta2 - lse_w[wave][q])) : 0.f;
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
            lo[v] = beta2 - lse_w[wave][q];
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
  for (int e = 1 + tid; e < n_list; e += NT) {
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
#define SAS_DKDV_CASE(NWV)                                                                     \
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NWV>), dim3(n_tiles * d.n_kv_heads, 1, d.batch),         \
                     dim3(64 * NWV), 0, st, q, kk, v, dop, lse, Dq, S, d.n_kv_heads, G, d.t_max, \
                     n_tiles, d.top_k, idx, log_gate, scale2, scale,                              \
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
    return launch_bwd_d<128>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK, dV,
                             dlog_gate, ws, st);
  return launch_bwd_d<64>(d, Q, K, V, O, dO, lse, seq_len, idx, log_gate, scale, dQ, dK, dV,
                          dlog_gate, ws, st);
}

}  // namespace sas
