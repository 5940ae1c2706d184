// Device helpers shared by the libdllm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

typedef uint16_t bf16;  // raw bfloat16 storage

__device__ __forceinline__ float bf2f(bf16 v) { return __uint_as_float(((uint32_t)v) << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct io<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16* p, float v) { *p = f2bf(v); }
};

// Rows of a per-sequence list in compact order: entry m of the concatenation
// of idx[b][0..n[b]) over b (counts clamped to [0, L]).  Returns false when m
// is past the total or the listed row is outside [0, L).
__device__ __forceinline__ bool row_of(const int32_t* __restrict__ idx, const int32_t* __restrict__ n,
                                       int B, int L, int m, int& b, int& i) {
  int off = 0;
  for (int bb = 0; bb < B; ++bb) {
    const int c = min(max(n[bb], 0), L);
    if (m < off + c) {
      b = bb;
      i = idx[(size_t)bb * L + (m - off)];
      return i >= 0 && i < L;
    }
    off += c;
  }
  return false;
}

// Total listed rows (same clamping), bounded by the caller's `cap` (the grid
// and the partial buffers are sized for cap rows; rows past it are skipped).
__device__ __forceinline__ int total_rows(const int32_t* __restrict__ n, int B, int cap) {
  int s = 0;
  for (int b = 0; b < B; ++b) s += min(max(n[b], 0), 1 << 24);
  return s < cap ? s : cap;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a block of NW waves (fixed order, deterministic).  `red` holds NW
// entries of LDS.  Every thread gets the total.
template <int NW, typename F>
__device__ __forceinline__ F block_sum(F v, F* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  F t = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) t += red[i];
  return t;
}

}  // namespace dllm
