// Device helpers shared by the libsas kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

// Storage types: float (fp32) or uint16_t holding bf16 bits.
template <typename T> struct Vec16;  // 16 bytes of T unpacked to floats
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xFFFF0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xFFFF0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xFFFF0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xFFFF0000u);
  }
};

template <typename T> __device__ __forceinline__ float load_scalar(const T* p);
template <> __device__ __forceinline__ float load_scalar<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_scalar<uint16_t>(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

template <typename T> __device__ __forceinline__ void store_scalar(T* p, float v);
template <> __device__ __forceinline__ void store_scalar<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_scalar<uint16_t>(uint16_t* p, float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  *p = static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ int clamp_len(int T, int t_max) {
  return T < 1 ? 1 : (T > t_max ? t_max : T);
}

// Butterfly reductions across lanes whose ids differ only in the bits of
// [lo, 64): xor-shuffle with masks lo, 2lo, ..., 32.
__device__ __forceinline__ float wave_sum_from(float v, int lo) {
  for (int m = lo; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max_from(float v, int lo) {
  for (int m = lo; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
// Reductions across the lanes [0, n) of each aligned group of n lanes.
__device__ __forceinline__ float group_sum(float v, int n) {
  for (int m = 1; m < n; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Order-preserving map of an fp32 score to uint32 (larger float -> larger
// integer); -0 and +0 map to the same value.
__device__ __forceinline__ uint32_t score_bits(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float score_from_bits(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// Composite Top-K key: higher score first, then lower block index.  0 is
// below every real key and marks "no candidate".
__device__ __forceinline__ uint64_t topk_key(float s, int m) {
  return (static_cast<uint64_t>(score_bits(s)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(m));
}
__device__ __forceinline__ int key_block(uint64_t k) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFu));
}
__device__ __forceinline__ float key_score(uint64_t k) {
  return score_from_bits(static_cast<uint32_t>(k >> 32));
}

// In-LDS bitonic sort of n (power of two) keys into DESCENDING order by the
// whole workgroup (blockDim.x threads).  Ends with a barrier.
__device__ inline void bitonic_sort_desc(uint64_t* keys, int n) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = tid; i < n / 2; i += nt) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        uint64_t a = keys[lo], b = keys[hi];
        if ((a < b) == desc) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
    }
  }
  __syncthreads();
}

}  // namespace sas
