// SPA-Cache method step 1 ("Singular proxy for adaptive caching in diffusion
// language models"): project each changed row's layer input onto the rank-r
// value subspace, x W_r, and score it by the cosine against the proxy cached
// at the row's last refresh (lowest similarity = most drift).
//
// Every decision-feeding quantity is fp64.  The attention-norm gain is folded
// into the basis once, Wg = diag(g1) W_r: for bf16/fp32 x and fp32 g1, W_r the
// triple product x*g1*w is rounded exactly once either way, so x . Wg equals
// (x * g1) . W_r up to the order of the fp64 sum.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int PX_ROWS = 32;   // rows per workgroup (8 per wave)
constexpr int PX_KC = 32;     // k per LDS chunk
constexpr int PX_TARGET = 512;

static int proxy_splits(int max_rows, int d) {
  const int rt = (max_rows + PX_ROWS - 1) / PX_ROWS;
  const int kt = d / PX_KC;
  int s = 1;
  while (s * 2 <= kt && kt % (s * 2) == 0 && rt * s * 2 <= PX_TARGET) s *= 2;
  return s;
}

size_t proxy_partial_doubles(int max_rows, int d, int r) {
  size_t best = 0;
  for (int m = 1; m <= max_rows; ++m) {
    const size_t v = (size_t)proxy_splits(m, d) * (size_t)m * r;
    if (v > best) best = v;
  }
  return best;
}

// partial[s][m][j] = sum_{k in split s} x[m][k] * Wg[k][j]
template <typename T, int CPL>
__global__ __launch_bounds__(256) void proxy_partial_kernel(int B, int L, int d, int r, int kps, int cap,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ n,
                                                            const T* __restrict__ H,
                                                            const double* __restrict__ wg,
                                                            double* __restrict__ partial) {
  __shared__ double xs[PX_ROWS][PX_KC + 1];
  __shared__ double ws[PX_KC][64 * CPL];
  __shared__ long long rowoff[PX_ROWS];
  const int M = total_rows(n, B, cap);
  const int r0 = blockIdx.x * PX_ROWS;
  if (r0 >= M) return;
  const int split = blockIdx.y;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  if (tid < PX_ROWS) {
    int b, i;
    rowoff[tid] = (r0 + tid < M && row_of(idx, n, B, L, r0 + tid, b, i)) ? (long long)((size_t)b * L + i) * d : -1;
  }
  double acc[8][CPL];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[a][c] = 0.0;
  const int kbeg = split * kps;
  __syncthreads();
  for (int k0 = kbeg; k0 < kbeg + kps; k0 += PX_KC) {
    for (int e = tid; e < PX_ROWS * PX_KC; e += 256) {
      const int rr = e / PX_KC, kk = e - rr * PX_KC;
      const long long off = rowoff[rr];
      xs[rr][kk] = off >= 0 ? (double)io<T>::ld(H + off + k0 + kk) : 0.0;
    }
    for (int e = tid; e < PX_KC * 64 * CPL; e += 256) {
      const int kk = e / (64 * CPL), j = e - kk * (64 * CPL);
      ws[kk][j] = j < r ? wg[(size_t)(k0 + kk) * r + j] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < PX_KC; ++kk) {
      double wv_[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) wv_[c] = ws[kk][lane + 64 * c];
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const double xv = xs[wv * 8 + a][kk];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[a][c] = fma(xv, wv_[c], acc[a][c]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int m = r0 + wv * 8 + a;
    if (m < M) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int j = lane + 64 * c;
        if (j < r) partial[((size_t)split * M + m) * r + j] = acc[a][c];
      }
    }
  }
}

// C = sum of split partials (fixed order); score = 0.5 |C/|C| - P/|P||^2.
__global__ __launch_bounds__(64) void proxy_finish_kernel(int B, int L, int r, int S, int cap,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ n,
                                                          const double* __restrict__ partial,
                                                          double* __restrict__ pcur,
                                                          const double* __restrict__ pref,
                                                          double* __restrict__ score) {
  int b, i;
  const int m = blockIdx.x;
  if (!row_of(idx, n, B, L, m, b, i)) return;
  const int M = total_rows(n, B, cap);
  const int lane = threadIdx.x;
  const size_t row = (size_t)b * L + i;
  double c[2], p[2];
  double cc = 0.0, pp = 0.0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j = lane + 64 * t;
    c[t] = 0.0;
    p[t] = 0.0;
    if (j < r) {
      const double v = sum_splits(partial + (size_t)m * r + j, (size_t)M * r, S);
      c[t] = v;
      p[t] = pref[row * r + j];
      pcur[row * r + j] = v;
    }
    cc += c[t] * c[t];
    pp += p[t] * p[t];
  }
  cc = wave_sum(cc);
  pp = wave_sum(pp);
  const double nc = sqrt(cc), np = sqrt(pp);
  double s_out;
  if (nc == 0.0 && np == 0.0) {
    s_out = 0.0;
  } else if (nc == 0.0 || np == 0.0) {
    s_out = 1.0;
  } else {
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (lane + 64 * t < r) {
        const double dl = c[t] / nc - p[t] / np;
        acc += dl * dl;
      }
    }
    s_out = 0.5 * wave_sum(acc);
  }
  if (lane == 0) score[row] = s_out;
}

hipError_t launch_proxy_drift(hipStream_t st, bool bf16m, int max_rows, int B, int L, int d, int r,
                              const int32_t* idx, const int32_t* n, const void* H, const double* wg,
                              double* partial, double* pcur, const double* pref, double* score) {
  if (max_rows <= 0) return hipSuccess;
  const int S = proxy_splits(max_rows, d);
  const int kps = d / S;
  dim3 grid((max_rows + PX_ROWS - 1) / PX_ROWS, S);
#define PX_LAUNCH(T, CPL)                                                                         \
  hipLaunchKernelGGL((proxy_partial_kernel<T, CPL>), grid, dim3(256), 0, st, B, L, d, r, kps, max_rows, idx, n, \
                     (const T*)H, wg, partial)
  if (r > 128) return hipErrorInvalidValue;
  if (bf16m) {
    if (r <= 64) PX_LAUNCH(bf16, 1);
    else PX_LAUNCH(bf16, 2);
  } else {
    if (r <= 64) PX_LAUNCH(float, 1);
    else PX_LAUNCH(float, 2);
  }
#undef PX_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proxy_finish_kernel, dim3(max_rows), dim3(64), 0, st, B, L, r, S, max_rows, idx, n, partial, pcur,
                     pref, score);
  return hipGetLastError();
}

// Wg[k][j] = g1[k] * W_r[k][j] (exact in fp64).
__global__ void fold_proxy_kernel(int d, int r, const float* __restrict__ g1, const float* __restrict__ wr,
                                  double* __restrict__ out) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (size_t)d * r) return;
  const int k = (int)(e / r);
  out[e] = (double)g1[k] * (double)wr[e];
}

hipError_t launch_fold_proxy(hipStream_t st, int d, int r, const float* g1, const float* wr, double* out) {
  const size_t total = (size_t)d * r;
  hipLaunchKernelGGL(fold_proxy_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, d, r, g1, wr,
                     out);
  return hipGetLastError();
}

}  // namespace dllm
