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
// rows 16j + 4*hi + {0..3} and 16j + 8 + 4*hi + {0..3}.
__device__ __forceinline__ bf16x8_t acc_to_bop(const f32x16_t* tiles, int j) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(tiles[j >> 1][8 * (j & 1) + e]);
  return r;
}
// The matching A operand from a [M][stride] bf16 LDS matrix whose columns are
// the contraction rows: row = M index of this lane, k-step j.
__device__ __forceinline__ bf16x8_t lds_aop_perm(const uint16_t* row, int j, int hi) {
  const uint2 lo = *reinterpret_cast<const uint2*>(row + 16 * j + 4 * hi);
  const uint2 up = *reinterpret_cast<const uint2*>(row + 16 * j + 8 + 4 * hi);
  return as_bf16x8(make_uint4(lo.x, lo.y, up.x, up.y));
}

// Stage a 64-row block of a row-major [rows][D] bf16 matrix into LDS twice:
// row-major (stride D+8) and transposed (stride 64+8).  Rows at or beyond
// `valid` read as zero.  Every thread of the block participates.
template <int D, int NT>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src, int valid,
                                           uint16_t* rm, uint16_t* tr, int tid) {
  constexpr int RSTR = D + 8, TSTR = 64 + 8;
  if (rm) {
    for (int c = tid; c < 64 * (D / 8); c += NT) {
      const int row = c / (D / 8), cc = c % (D / 8);
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row < valid) u = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row) * D + cc * 8);
      *reinterpret_cast<uint4*>(&rm[row * RSTR + cc * 8]) = u;
    }
  }
  if (tr) {
    for (int p = tid; p < 32 * (D / 8); p += NT) {
      const int tp = p % 32, cc = p / 32;
      const int r0 = 2 * tp;
      uint4 u0 = make_uint4(0, 0, 0, 0), u1 = make_uint4(0, 0, 0, 0);
      if (r0 < valid) u0 = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(r0) * D + cc * 8);
      if (r0 + 1 < valid) u1 = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(r0 + 1) * D + cc * 8);
      const uint32_t w0[4] = {u0.x, u0.y, u0.z, u0.w};
      const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = (w0[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const uint32_t b = (w1[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        *reinterpret_cast<uint32_t*>(&tr[(cc * 8 + e) * TSTR + r0]) = a | (b << 16);
      }
    }
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

}  // namespace sas
