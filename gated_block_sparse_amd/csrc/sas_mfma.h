// gfx950 matrix-core helpers shared by the prefill forward and backward.
//
// v_mfma_f32_32x32x16_bf16 lane layouts (lane l, l32 = l % 32, hi = l / 32):
//   A (32 x 16): lane holds A[l32][8*hi .. 8*hi+7]
//   B (16 x 32): lane holds B[8*hi .. 8*hi+7][l32]
//   D (32 x 32): lane holds D[8*(v/4) + 4*hi + v%4][l32], v = 0..15
// so a row-major matrix with the contraction index contiguous feeds either
// operand with one 16-byte read per lane, and the 16 results of a lane all
// sit in one column.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void zero16(f32x16_t& x) {
#pragma unroll
  for (int v = 0; v < 16; ++v) x[v] = 0.f;
}
// Row index (within a 32-row tile) of accumulator element v of a lane.
__device__ __forceinline__ int acc_row(int v, int hi) { return 8 * (v >> 2) + 4 * hi + (v & 3); }

// B operand for a contraction over the 32 rows of two accumulator tiles:
// k-step j (0..3) takes the 16 rows 16j..16j+15 in the order the lane holds
// them (elements 8*(j%2) .. +8 of tile j/2).  The matching A operand reads
// rows 16j + 4*hi + {0..3} and 16j + 8 + 4*hi + {0..3} (lds_aop_tr_perm).
__device__ __forceinline__ bf16x8_t acc_to_bop(const f32x16_t* tiles, int j) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(tiles[j >> 1][8 * (j & 1) + e]);
  return r;
}
// ds_read_b64_tr_b16 (gfx950 LDS transpose read).  Within each group of 16
// lanes, lane j supplies an 8-byte chunk C_j; lane 4a+b receives element b of
// C_a, C_{a+4}, C_{a+8}, C_{a+12} (layout checked on the GPU).  So if lane j
// points at row k0 + j/4, columns c0 + 4*(j%4) of a row-major matrix, lane t
// of the group receives rows k0..k0+3 of column c0 + t.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_t*)((__attribute__((address_space(3))) uint16_t*)p));
  return __builtin_bit_cast(uint2, v);
}
// LDS tiles of 64 (or 32) rows x D bf16 are row-major with a padded row
// stride chosen for how the tile is read (64 banks of 4 bytes):
//   * kRowStride = D + 8 for 16-byte row reads, one chunk of 16 consecutive
//     rows per pass (row r starts 4r banks further: all 64 banks once);
//   * kTrStride = D + 32 for the transpose reads below, which take 4
//     consecutive rows x 64 bytes per pass (rows 16 banks apart).
// Each stride conflicts for the other pattern (4-way), so a tile that is
// read both ways is staged twice.  (An XOR swizzle serves both patterns, but
// its addresses cannot be folded into instruction offsets and the kernels
// then run out of registers.)  Staging writes of consecutive chunks are
// conflict-free at either stride for D = 128.
template <int D> constexpr int kRowStride = D + 8;
template <int D> constexpr int kTrStride = D + 32;

// A operand of v_mfma_f32_32x32x16_bf16 whose M index is a COLUMN of a
// row-major LDS tile X of row stride RS (K along the rows): lane (l32, hi)
// gets column i0 + l32, K elements 0-3 from rows k0..k0+3 and 4-7 from rows
// k1..k1+3 (callers pass per-lane k0/k1 that depend on hi).
template <int RS>
__device__ __forceinline__ bf16x8_t lds_aop_tr(const uint16_t* X, int i0, int k0, int k1) {
  const int lane = threadIdx.x & 63, g = lane >> 4, jj = lane & 15;
  const int col = i0 + 16 * (g & 1) + 4 * (jj & 3);
  const int ro = jj >> 2;
  const uint2 a = lds_read_tr16(X + (k0 + ro) * RS + col);
  const uint2 b = lds_read_tr16(X + (k1 + ro) * RS + col);
  return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}
// The A operand matching acc_to_bop(tiles, j): rows 16j + 4hi + {0..3} and
// 16j + 8 + 4hi + {0..3} of the tile, column i0 + l32.
template <int RS>
__device__ __forceinline__ bf16x8_t lds_aop_tr_perm(const uint16_t* X, int i0, int j, int hi) {
  return lds_aop_tr<RS>(X, i0, 16 * j + 4 * hi, 16 * j + 8 + 4 * hi);
}
// 16-byte row read: elements col..col+7 of row r (col % 8 == 0).
template <int RS>
__device__ __forceinline__ bf16x8_t lds_row8(const uint16_t* X, int r, int col) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(X + r * RS + col));
}
template <int RS>
__device__ __forceinline__ void lds_store_row8(uint16_t* X, int r, int col, uint4 v) {
  *reinterpret_cast<uint4*>(X + r * RS + col) = v;
}

// Stage a 64-row block of a row-major [rows][D] bf16 matrix into LDS tiles:
// `rm` at the row-read stride and, when not null, `tr` at the transpose-read
// stride.  Rows at or beyond `valid` read as zero.  Every thread of the block
// participates.
template <int D, int NT>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src, int valid,
                                           uint16_t* rm, uint16_t* tr, int tid) {
  for (int c = tid; c < 64 * (D / 8); c += NT) {
    const int row = c / (D / 8), cc = c % (D / 8);
    uint4 u = make_uint4(0, 0, 0, 0);
    if (row < valid) u = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row) * D + cc * 8);
    if (rm) lds_store_row8<kRowStride<D>>(rm, row, cc * 8, u);
    if (tr) lds_store_row8<kTrStride<D>>(tr, row, cc * 8, u);
  }
}

// Store a lane's accumulator tiles (channels as rows, one column per lane)
// scaled by `mul` as bf16 into row `dst` (4 consecutive channels per write).
template <int CT>
__device__ __forceinline__ void store_acc_col(const f32x16_t* acc, float mul, uint16_t* dst, int hi) {
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int c0 = 32 * ct + 8 * grp + 4 * hi;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t u = __float_as_uint(acc[ct][4 * grp + e] * mul);
        u += 0x7FFFu + ((u >> 16) & 1u);
        w[e] = u >> 16;
      }
      uint2 pk;
      pk.x = w[0] | (w[1] << 16);
      pk.y = w[2] | (w[3] << 16);
      *reinterpret_cast<uint2*>(dst + c0) = pk;
    }
}


typedef __attribute__((ext_vector_type(4))) float f32x4_t;
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- LDS DMA (global_load_lds).
// LDS byte address of a __shared__ object (what M0 takes).
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const unsigned char*)p));
}
// One LDS DMA copy: every lane fetches BYTES (16 or 4) from its own global
// address; lane L's bytes land at LDS address lds_addr + L * BYTES (M0 holds
// the wave-uniform base).  Issued from asm so that the compiler does not
// track it: it would otherwise make every later read of the ring wait for
// all copies in flight; completion is waited for explicitly (dma_sync).  M0
// is saved and restored around the copy.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* g, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t keep;
  if constexpr (BYTES == 16)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
        : "=&s"(keep) : "s"(m0v), "v"(g) : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "global_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
        : "=&s"(keep) : "s"(m0v), "v"(g) : "memory");
}

// Waits until at most N of this wave's vector-memory operations (here: LDS
// DMA copies) are outstanding and its LDS operations are done, then joins the
// workgroup barrier.  Written as one asm statement with a memory clobber so
// that no LDS access moves across it; a fence would wait for every copy in
// flight, including those of later steps.
template <int N>
__device__ __forceinline__ void dma_sync() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace sas
