// Device helpers shared by the libdllm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace dllm {

// Kernel attributes (the dynamic LDS limit) are set per device: `done` keeps
// one bit per device id.  Runs `set` on the current device the first time
// (again after a failure) and returns its status.
template <typename F>
inline hipError_t once_per_device(std::atomic<unsigned long long>& done, F set) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = (dev >= 0 && dev < 64) ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = set();
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

typedef uint16_t bf16;  // raw bfloat16 storage

__device__ __forceinline__ float bf2f(bf16 v) { return __uint_as_float(((uint32_t)v) << 16); }

typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));

// Two floats -> packed bfloat16 pair (a in the low half), round to nearest
// even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  const f32x2_hw v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}

// SiLU for the bf16 paths: x / (1 + e^-x) from the hardware base-2
// exponential and reciprocal (a few fp32 ulps, far inside the bf16 rounding
// the result then takes).
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// float -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)(pack2bf(f, 0.0f) & 0xffffu); }

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

// row_of for a kernel that loaded n[0] and sequence 0's entry idx[min(m, L-1)]
// itself, together with its other row-independent loads (one memory round
// trip for a one-sequence batch); later sequences take row_of.  i0 is the
// starting value on every path, so the compiler keeps its load where the
// caller issued it.
__device__ __forceinline__ bool row_resolve(const int32_t* __restrict__ idx, const int32_t* __restrict__ n, int B,
                                            int L, int m, int n0, int i0, int& b, int& i) {
  b = 0;
  i = i0;
  if (m < min(max(n0, 0), L)) return i >= 0 && i < L;
  return B > 1 && row_of(idx, n, B, L, m, b, i);
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
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// A wave-uniform pointer, made visibly uniform so that it can live in scalar
// registers (LDS DMA requests take their base address from an SGPR pair).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
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

// Packed activation layout (bf16 GEMM inputs).  A row-major [M][K] operand is
// stored as 32x16 MFMA A-fragments: fragment (kt = k/16, mt = m/32) occupies
// 1 KB at ((kt * MTt + mt) * 64 + lane) * 8 elements, where MTt is the number
// of 32-row tiles the buffer holds and lane = m%32 + 32*((k%16)/8) holds the 8
// consecutive k of its row.  A wave loads one fragment with one 16-byte load
// per lane, and a wave's row tiles for one k-step are contiguous.
__device__ __forceinline__ size_t apack_off(int m, int k, int MTt) {
  const int kt = k >> 4, mt = m >> 5, lane = (m & 31) + ((k >> 3) & 1) * 32;
  return (((size_t)kt * MTt + mt) * 64 + lane) * 8 + (k & 7);
}

// Key cache offset inside one (sequence, kv head) block of L32 * dh elements
// (L32 = L rounded up to 32), in matrix-core fragment order: a wave reads the
// fragment of 32 keys x 16 dims as one contiguous 1 KB.  The value cache is
// row-major in the same block ([L32][dh]): element (j, t) at j * dh + t.
__device__ __forceinline__ size_t kc_off(int j, int t, int dh) {
  return (((size_t)(j >> 5) * (dh >> 4) + (t >> 4)) * 64 + (j & 31) + 32 * ((t >> 3) & 1)) * 8 + (t & 7);
}
__device__ __forceinline__ int l32_of(int L) { return (L + 31) & ~31; }

// Store 8 consecutive values of row m starting at column k8 (a multiple of 8)
// of a GEMM input: packed fragments for bf16 (one 16-byte store), row-major
// [..][ld] for fp32.
__device__ __forceinline__ void store_a8(bf16* A, int m, int k8, int MTt, int /*ld*/, const float* v) {
  uint4 w;
  w.x = pack2bf(v[0], v[1]);
  w.y = pack2bf(v[2], v[3]);
  w.z = pack2bf(v[4], v[5]);
  w.w = pack2bf(v[6], v[7]);
  *reinterpret_cast<uint4*>(A + apack_off(m, k8, MTt)) = w;
}
__device__ __forceinline__ void store_a8(float* A, int m, int k8, int /*MTt*/, int ld, const float* v) {
  float* p = A + (size_t)m * ld + k8;
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = v[j];
}
// One element of a GEMM input (packed for bf16).
__device__ __forceinline__ void store_a1(bf16* A, int m, int k, int MTt, int, float v) { A[apack_off(m, k, MTt)] = f2bf(v); }
__device__ __forceinline__ void store_a1(float* A, int m, int k, int, int ld, float v) { A[(size_t)m * ld + k] = v; }

// Row-wide (normalising) kernels: one workgroup of RT threads per row, each
// thread holding up to RV groups of 8 consecutive values in registers.
constexpr int RT = 512;  // threads of the row-wide (normalising) kernels
constexpr int RV = 2;    // groups of 8 per thread: d <= RT * 8 * RV

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// RMSNorm (fp32 statistics) of the d values at x times the gain g, stored as
// row m of a GEMM input (packed for bf16).  One workgroup of RT threads; red
// holds RT / 64 floats of LDS.
template <typename T>
__device__ __forceinline__ void norm_row_store(const T* __restrict__ x, int d, float eps,
                                               const float* __restrict__ g, T* __restrict__ A, int m, int MTt,
                                               float* red) {
  float v[RV][8];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    const int c8 = (threadIdx.x + r * RT) * 8;
    if (c8 < d) {
      load8<T>(x + c8, v[r]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[r][e] * v[r][e];
    }
  }
  ss = block_sum<RT / 64>(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    const int c8 = (threadIdx.x + r * RT) * 8;
    if (c8 < d) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[r][e] * inv * g[c8 + e];
      store_a8(A, m, c8, MTt, d, o);
    }
  }
}

// The S split partials p[s * stride] of four consecutive columns, loaded
// unconditionally (issued back to back), and their sum in split order.
template <int S>
__device__ __forceinline__ void load_splits4(const float* __restrict__ p, size_t stride, float4 (&t)[S]) {
#pragma unroll
  for (int s = 0; s < S; ++s) t[s] = *reinterpret_cast<const float4*>(p + (size_t)s * stride);
}
template <int S>
__device__ __forceinline__ float4 add_splits4(const float4 (&t)[S]) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    acc.x += t[s].x;
    acc.y += t[s].y;
    acc.z += t[s].z;
    acc.w += t[s].w;
  }
  return acc;
}

// Sum of S split partials p[s * stride] in split order, loads issued in
// batches of 8 so they overlap.
template <typename F>
__device__ __forceinline__ F sum_splits(const F* __restrict__ p, size_t stride, int S) {
  F acc = F(0);
  for (int s0 = 0; s0 < S; s0 += 8) {
    F v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (s0 + j < S) ? p[(size_t)(s0 + j) * stride] : F(0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) acc += v[j];
  }
  return acc;
}

}  // namespace dllm
