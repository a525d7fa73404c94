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

// 2^x with the hardware transcendental (v_exp_f32, about 1 ulp; results below
// the normal range flush to 0, which is what a softmax wants).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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
// DPP lane moves inside a row of 16 lanes (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each row

// Sum over each aligned group of n lanes (n a power of two, <= 64); every
// lane of the group receives the sum.  Within a row the partner lanes come
// from DPP moves: after the xor-1 and xor-2 steps each quad holds its sum,
// so the half-row and row mirrors pair whole quads and half rows.
__device__ __forceinline__ float group_sum(float v, int n) {
  if (n >= 2) v += dpp_mov<kDppXor1>(v);
  if (n >= 4) v += dpp_mov<kDppXor2>(v);
  if (n >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if (n >= 16) v += dpp_mov<kDppMirror>(v);
  if (n >= 32) v += __shfl_xor(v, 16, 64);
  if (n >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float group_max(float v, int n) {
  if (n >= 2) v = fmaxf(v, dpp_mov<kDppXor1>(v));
  if (n >= 4) v = fmaxf(v, dpp_mov<kDppXor2>(v));
  if (n >= 8) v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  if (n >= 16) v = fmaxf(v, dpp_mov<kDppMirror>(v));
  if (n >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if (n >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Transposed butterfly over the 32 lanes of each half wave: lane l32 starts
// with 32 partial values v[0..31] and ends with v[0] = the sum over the half
// wave of v[l32].  31 shuffles in all.  The keep/send choice is an integer
// blend so the compiler cannot turn it into dynamic register indexing.
__device__ __forceinline__ float transpose_sum32(float* v, int l32) {
#pragma unroll
  for (int sft = 16; sft >= 1; sft >>= 1) {
    const uint32_t up = (l32 & sft) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int j = 0; j < sft; ++j) {
      const uint32_t a = __float_as_uint(v[j]), b = __float_as_uint(v[j + sft]);
      const float keep = __uint_as_float((b & up) | (a & ~up));
      const float send = __uint_as_float((a & up) | (b & ~up));
      v[j] = keep + __shfl_xor(send, sft, 64);
    }
  }
  return v[0];
}

// The same with R < 32 partial values: the transposing steps run over the
// low log2(R) lane bits, then plain butterfly sums over the rest; lane l32
// ends with the sum of v[l32 % R] over the half wave.
template <int R>
__device__ __forceinline__ float transpose_sum(float* v, int l32) {
  static_assert(R >= 1 && R <= 32 && (R & (R - 1)) == 0, "R: power of two up to 32");
#pragma unroll
  for (int sft = R / 2; sft >= 1; sft >>= 1) {
    const uint32_t up = (l32 & sft) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int j = 0; j < sft; ++j) {
      const uint32_t a = __float_as_uint(v[j]), b = __float_as_uint(v[j + sft]);
      const float keep = __uint_as_float((b & up) | (a & ~up));
      const float send = __uint_as_float((a & up) | (b & ~up));
      v[j] = keep + __shfl_xor(send, sft, 64);
    }
  }
  float s = v[0];
#pragma unroll
  for (int sft = R; sft < 32; sft <<= 1) s += __shfl_xor(s, sft, 64);
  return s;
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

// 64-bit xor shuffle inside a wave.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Bitonic sort of one key per lane across a wave into DESCENDING lane order
// (lane 0 holds the largest).  Wave-synchronous: no LDS, no barrier.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t other = shfl_xor_u64(key, stride);
      const bool desc = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      const bool keep_max = (lower == desc);
      key = keep_max ? (key > other ? key : other) : (key < other ? key : other);
    }
  }
  return key;
}

// Number of entries greater than x in a DESCENDING sorted list of n keys.
__device__ __forceinline__ int count_greater_desc(const uint64_t* list, int n, uint64_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list[mid] > x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

}  // namespace sas
