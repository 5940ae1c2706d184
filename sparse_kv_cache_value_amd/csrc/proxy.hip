// SPA-Cache method step 1 ("Singular proxy for adaptive caching in diffusion
// language models"): project each changed row's layer input onto the rank-r
// value subspace, x W_r, and score it by the cosine against the proxy cached
// at the row's last refresh (lowest similarity = most drift).
//
// Every decision-feeding quantity is fp64.  The normalised input's gain g1 is
// applied to x in fp64 (exactly), and the basis is kept in fp32 as given, so
// every product x*g1*w is rounded exactly once, as in the fp64 definition; only
// the order of the fp64 sum differs.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int PX_KC = 32;      // k per LDS chunk
constexpr int PX_TARGET = 512;  // workgroups to aim for
constexpr int PX_SMAX = 32;     // most K splits (bounds the partial traffic)
constexpr int PX_RPT = 8;       // rows per thread

// Basis width as stored: r rounded up to 32, 64 or 128 (zero columns).
int proxy_rpad(int r) { return r <= 32 ? 32 : (r <= 64 ? 64 : 128); }

static int proxy_rows_per_wg(int rpad) { return (256 / rpad) * PX_RPT; }

static int proxy_splits(int max_rows, int d, int rpad) {
  const int rm = proxy_rows_per_wg(rpad);
  const int rt = (max_rows + rm - 1) / rm;
  const int kt = d / PX_KC;
  int s = 1;
  while (s * 2 <= kt && kt % (s * 2) == 0 && rt * s * 2 <= PX_TARGET && s * 2 <= PX_SMAX) s *= 2;
  return s;
}

size_t proxy_partial_doubles(int max_rows, int d, int r) {
  const int rpad = proxy_rpad(r);
  size_t best = 0;
  for (int m = 1; m <= max_rows; ++m) {
    const size_t v = (size_t)proxy_splits(m, d, rpad) * (size_t)m * rpad;
    if (v > best) best = v;
  }
  return best;
}

template <typename T>
struct XVec;  // one global load of consecutive layer-input values
template <>
struct XVec<bf16> {
  static constexpr int N = 8;
  using V = uint4;
  static __device__ __forceinline__ void unpack(const V& u, double* o) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = (double)__uint_as_float(w[e] << 16);
      o[2 * e + 1] = (double)__uint_as_float(w[e] & 0xffff0000u);
    }
  }
};
template <>
struct XVec<float> {
  static constexpr int N = 4;
  using V = float4;
  static __device__ __forceinline__ void unpack(const V& u, double* o) {
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
};

// partial[s][m][j] = sum over k in split s of (x[m][k] g1[k]) W_r[k][j].
// Thread (rg, j) owns column j of rows rg*8 .. rg*8+7 of the workgroup's
// tile; chunks of 32 k are staged in LDS as fp64, the next chunk's global
// loads issued before the current chunk's arithmetic.  x*g1 is exact in fp64
// (at most 24+24 significant bits), so each FMA rounds the exact triple
// product once, as the fp64 definition does.
template <typename T, int RPAD>
__global__ __launch_bounds__(256) void proxy_partial_kernel(int B, int L, int d, int kps, int cap,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ n,
                                                            const T* __restrict__ H,
                                                            const float* __restrict__ g1,
                                                            const float* __restrict__ wr,
                                                            double* __restrict__ partial) {
  constexpr int RG = 256 / RPAD, RM = RG * PX_RPT;
  constexpr int XV = XVec<T>::N;
  constexpr int XLOADS = (RM * PX_KC / XV + 255) / 256;
  constexpr int WLOADS = PX_KC * RPAD / 4 / 256;
  constexpr int XS = PX_KC + 2;  // row stride (doubles): 16-byte aligned pairs
  __shared__ __align__(16) double xs[RM * XS];
  __shared__ double ws[PX_KC * RPAD];
  __shared__ long long rowoff[RM];
  const int M = total_rows(n, B, cap);
  const int r0 = blockIdx.x * RM;
  if (r0 >= M) return;
  const int tid = threadIdx.x, j = tid % RPAD, rg = tid / RPAD;
  if (tid < RM) {
    int b, i;
    rowoff[tid] = (r0 + tid < M && row_of(idx, n, B, L, r0 + tid, b, i)) ? (long long)((size_t)b * L + i) * d : -1;
  }
  __syncthreads();
  const int kbeg = blockIdx.y * kps, nch = kps / PX_KC;
  typename XVec<T>::V xr[XLOADS];
  float4 gr[XLOADS][XV / 4];
  float4 wrg[WLOADS];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int q = 0; q < XLOADS; ++q) {
      const int e = tid + 256 * q, row = e / (PX_KC / XV), kk = (e % (PX_KC / XV)) * XV;
      const long long off = (e < RM * PX_KC / XV) ? rowoff[row] : -1;
      if (off >= 0) {
        xr[q] = *reinterpret_cast<const typename XVec<T>::V*>(H + off + k0 + kk);
#pragma unroll
        for (int h = 0; h < XV / 4; ++h) gr[q][h] = *reinterpret_cast<const float4*>(g1 + k0 + kk + 4 * h);
      } else {
        xr[q] = {};
#pragma unroll
        for (int h = 0; h < XV / 4; ++h) gr[q][h] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int q = 0; q < WLOADS; ++q) {
      const int e = tid + 256 * q;
      wrg[q] = *reinterpret_cast<const float4*>(wr + (size_t)(k0 + e / (RPAD / 4)) * RPAD + (e % (RPAD / 4)) * 4);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int q = 0; q < XLOADS; ++q) {
      const int e = tid + 256 * q;
      if (e < RM * PX_KC / XV) {
        const int row = e / (PX_KC / XV), kk = (e % (PX_KC / XV)) * XV;
        double xv[XV];
        XVec<T>::unpack(xr[q], xv);
#pragma unroll
        for (int h = 0; h < XV / 4; ++h) {
          xs[row * XS + kk + 4 * h + 0] = xv[4 * h + 0] * (double)gr[q][h].x;
          xs[row * XS + kk + 4 * h + 1] = xv[4 * h + 1] * (double)gr[q][h].y;
          xs[row * XS + kk + 4 * h + 2] = xv[4 * h + 2] * (double)gr[q][h].z;
          xs[row * XS + kk + 4 * h + 3] = xv[4 * h + 3] * (double)gr[q][h].w;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < WLOADS; ++q) {
      const int e = tid + 256 * q;
      double* w = ws + (e / (RPAD / 4)) * RPAD + (e % (RPAD / 4)) * 4;
      w[0] = wrg[q].x; w[1] = wrg[q].y; w[2] = wrg[q].z; w[3] = wrg[q].w;
    }
  };
  double acc[PX_RPT];
#pragma unroll
  for (int a = 0; a < PX_RPT; ++a) acc[a] = 0.0;
  fetch(kbeg);
  for (int c = 0; c < nch; ++c) {
    stage();
    __syncthreads();
    if (c + 1 < nch) fetch(kbeg + (c + 1) * PX_KC);
#pragma unroll 4
    for (int kk = 0; kk < PX_KC; kk += 2) {
      const double w0 = ws[kk * RPAD + j], w1 = ws[(kk + 1) * RPAD + j];
#pragma unroll
      for (int a = 0; a < PX_RPT; ++a) {
        const double2 xv = *reinterpret_cast<const double2*>(xs + (rg * PX_RPT + a) * XS + kk);
        acc[a] = fma(xv.x, w0, acc[a]);
        acc[a] = fma(xv.y, w1, acc[a]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < PX_RPT; ++a) {
    const int m = r0 + rg * PX_RPT + a;
    if (m < M) partial[((size_t)blockIdx.y * M + m) * RPAD + j] = acc[a];
  }
}

// C = sum of the split partials (fixed order: split groups in sequence, each
// group's splits in sequence); score = 0.5 |C/|C| - P/|P||^2, 0 when both
// proxies vanish, 1 when exactly one does.
template <int RPAD>
__global__ __launch_bounds__(256) void proxy_finish_kernel(int B, int L, int r, int S, int cap,
                                                           const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ n,
                                                           const double* __restrict__ partial,
                                                           double* __restrict__ pcur,
                                                           const double* __restrict__ pref,
                                                           double* __restrict__ score) {
  constexpr int SG = 256 / RPAD;
  constexpr int PER = PX_SMAX / SG > 0 ? PX_SMAX / SG : 1;
  __shared__ double gs[SG][RPAD];
  __shared__ double red[2][4];
  int b, i;
  const int m = blockIdx.x;
  if (!row_of(idx, n, B, L, m, b, i)) return;
  const int M = total_rows(n, B, cap);
  const int tid = threadIdx.x, j = tid % RPAD, sg = tid / RPAD;
  const size_t row = (size_t)b * L + i;
  const int per = (S + SG - 1) / SG, s0 = sg * per;
  double t[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int s = s0 + q;
    t[q] = (q < per && s < S) ? partial[((size_t)s * M + m) * RPAD + j] : 0.0;
  }
  double v = 0.0;
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (q < per && s0 + q < S) v += t[q];
  gs[sg][j] = v;
  __syncthreads();
  double c = 0.0, p = 0.0;
  if (sg == 0) {
#pragma unroll
    for (int g = 0; g < SG; ++g) c += gs[g][j];
    if (j < r) {
      p = pref[row * r + j];
      pcur[row * r + j] = c;
    } else {
      c = 0.0;
    }
  }
  // |C|^2 and |P|^2 over the first RPAD threads (waves 0 .. RPAD/64 - 1)
  double cc = wave_sum(c * c), pp = wave_sum(p * p);
  const int wv = tid >> 6, lane = tid & 63;
  if (lane == 0 && wv < 4) {
    red[0][wv] = cc;
    red[1][wv] = pp;
  }
  __syncthreads();
  cc = 0.0;
  pp = 0.0;
  for (int w = 0; w < (RPAD + 63) / 64; ++w) {
    cc += red[0][w];
    pp += red[1][w];
  }
  const double nc = sqrt(cc), np = sqrt(pp);
  double dl = 0.0;
  if (sg == 0 && j < r && nc > 0.0 && np > 0.0) {
    const double e = c / nc - p / np;
    dl = e * e;
  }
  const double ss = wave_sum(dl);
  __syncthreads();
  if (lane == 0 && wv < 4) red[0][wv] = ss;
  __syncthreads();
  if (tid == 0) {
    double s_out;
    if (nc == 0.0 && np == 0.0) {
      s_out = 0.0;
    } else if (nc == 0.0 || np == 0.0) {
      s_out = 1.0;
    } else {
      double acc = 0.0;
      for (int w = 0; w < (RPAD + 63) / 64; ++w) acc += red[0][w];
      s_out = 0.5 * acc;
    }
    score[row] = s_out;
  }
}

hipError_t launch_proxy_drift(hipStream_t st, bool bf16m, int max_rows, int B, int L, int d, int r,
                              const int32_t* idx, const int32_t* n, const void* H, const float* g1,
                              const float* wr, double* partial, double* pcur, const double* pref, double* score) {
  if (max_rows <= 0) return hipSuccess;
  if (r > 128 || d % PX_KC) return hipErrorInvalidValue;
  const int rpad = proxy_rpad(r);
  const int S = proxy_splits(max_rows, d, rpad);
  const int kps = d / S;
  const int rm = proxy_rows_per_wg(rpad);
  dim3 grid((max_rows + rm - 1) / rm, S);
#define PX_LAUNCH(T, RP)                                                                                  \
  hipLaunchKernelGGL((proxy_partial_kernel<T, RP>), grid, dim3(256), 0, st, B, L, d, kps, max_rows, idx, n, \
                     (const T*)H, g1, wr, partial)
#define PX_BY_RPAD(T)          \
  if (rpad == 32) PX_LAUNCH(T, 32);  \
  else if (rpad == 64) PX_LAUNCH(T, 64); \
  else PX_LAUNCH(T, 128);
  if (bf16m) {
    PX_BY_RPAD(bf16)
  } else {
    PX_BY_RPAD(float)
  }
#undef PX_BY_RPAD
#undef PX_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define PF_LAUNCH(RP)                                                                                              \
  hipLaunchKernelGGL((proxy_finish_kernel<RP>), dim3(max_rows), dim3(256), 0, st, B, L, r, S, max_rows, idx, n, \
                     partial, pcur, pref, score)
  if (rpad == 32) PF_LAUNCH(32);
  else if (rpad == 64) PF_LAUNCH(64);
  else PF_LAUNCH(128);
#undef PF_LAUNCH
  return hipGetLastError();
}

// Stored basis: W_r as fp32 [d][rpad], columns r .. rpad-1 zero.
__global__ void pad_proxy_kernel(int d, int r, int rpad, const float* __restrict__ wr, float* __restrict__ out) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (size_t)d * rpad) return;
  const int k = (int)(e / rpad), j = (int)(e % rpad);
  out[e] = j < r ? wr[(size_t)k * r + j] : 0.0f;
}

hipError_t launch_pad_proxy(hipStream_t st, int d, int r, const float* wr, float* out) {
  const int rpad = proxy_rpad(r);
  const size_t total = (size_t)d * rpad;
  hipLaunchKernelGGL(pad_proxy_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, d, r, rpad, wr,
                     out);
  return hipGetLastError();
}

}  // namespace dllm
