// Polestar-Cache drift path (Polestar page, section 2A): a local window of
// prefix, current and suffix blocks; spherical k-means of the window's layer
// inputs; NVFP4 codes of the residuals (the compressed proxy); attention of
// the cluster centroids' queries over the window keys ("proxy attention");
// cluster drift = KL between this step's and the previous step's proxy
// attention; the top drifting clusters' rows are refreshed.
//
// Decision math is fp64.  The k-means runs on the window's Gram matrix:
// with unit rows x_i and a centroid c_j = sum_{i in S_j} x_i / |sum x_i|,
// every dot product c_j . x_k = (sum_{i in S_j} G_ik) / sqrt(sum_{i,i' in S_j}
// G_ii'), so the iterations need only G (W x W, fp64, built once per layer on
// the fp64 matrix cores) and the explicit centroids are formed once at the end.
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int PS_SD = 128;    // dims per Gram slice
constexpr int PS_WMAX = 120;  // window rows: the k-means keeps W x W fp64 in LDS

__device__ __forceinline__ int ps_window_start(int bs, int L, int blk, int W) {
  return min(max(bs - blk, 0), L - W);
}

// ---------------------------------------------------------------------------
// Gram partials: part[b][s][i][j] = sum over dims of slice s of x_i x_j, for
// the W window rows of sequence b (raw layer inputs, fp64 products are exact).
// Upper-triangle 16x16 tiles on v_mfma_f64_16x16x4_f64, mirrored on store.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void ps_gram_kernel(int L, int d, int blk, int W, const int32_t* __restrict__ bstart,
                                                      const T* __restrict__ H, double* __restrict__ part) {
  extern __shared__ double xs[];  // [TW*16][PS_SD + 1]
  const int b = blockIdx.y, s = blockIdx.x, nsl = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ws = ps_window_start(bstart[b], L, blk, W);
  const int TW = (W + 15) / 16;
  const int XS = PS_SD + 1;
  const int d0 = s * PS_SD;
  for (int e = tid; e < TW * 16 * PS_SD; e += 256) {
    const int r = e / PS_SD, t = e - r * PS_SD;
    xs[r * XS + t] = r < W ? (double)io<T>::ld(H + ((size_t)b * L + ws + r) * d + d0 + t) : 0.0;
  }
  __syncthreads();
  const int npairs = TW * (TW + 1) / 2;
  const size_t pbase = ((size_t)b * nsl + s) * W * W;
  for (int p = wv; p < npairs; p += 4) {
    int ti = 0, rem = p;
    while (rem >= TW - ti) {
      rem -= TW - ti;
      ++ti;
    }
    const int tj = ti + rem;
    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
    const int ra = ti * 16 + (lane & 15), rb = tj * 16 + (lane & 15), kq = lane >> 4;
#pragma unroll 4
    for (int k = 0; k < PS_SD; k += 4)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xs[ra * XS + k + kq], xs[rb * XS + k + kq], acc, 0, 0, 0);
    // D register e of lane l: row l/16 + 4e of tile ti, column l%16 of tile tj
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = ti * 16 + (lane >> 4) + 4 * e, j = tj * 16 + (lane & 15);
      if (i < W && j < W) {
        part[pbase + (size_t)i * W + j] = acc[e];
        part[pbase + (size_t)j * W + i] = acc[e];
      }
    }
  }
}

// R[b][i][j] = sum over slices in slice order.
__global__ void ps_gram_reduce_kernel(int W, int nsl, const double* __restrict__ part, double* __restrict__ R) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= W * W) return;
  const double* p = part + (size_t)b * nsl * W * W + e;
  double acc = 0.0;
  for (int s = 0; s < nsl; ++s) acc += p[(size_t)s * W * W];
  R[(size_t)b * W * W + e] = acc;
}

// ---------------------------------------------------------------------------
// Spherical k-means on the Gram matrix (one workgroup per sequence, wave j
// owns cluster j).  Seeds: window rows stride*j.  Each iteration: assign each
// row to the cluster of largest dot product (lowest index on ties); every
// cluster with members and a non-zero member sum becomes the normalised
// member sum; others keep their centroid.  Then a final assignment.  Outputs
// the assignment, the row norms and each centroid's coefficients over the
// unit rows.  A cluster's members come from two 64-row ballots and are
// visited in ascending row order; member sums and the squared norm are added
// in that order.
// ---------------------------------------------------------------------------
constexpr int PS_KM_THREADS = 1024;  // 16 waves: one per cluster (K <= 16)

__global__ __launch_bounds__(PS_KM_THREADS) void ps_kmeans_kernel(int W, int K, int iters, const double* __restrict__ R,
                                                                 int32_t* __restrict__ assign,
                                                                 double* __restrict__ norms,
                                                                 double* __restrict__ coef, int32_t* __restrict__ nsel) {
  extern __shared__ double sm[];
  double* G = sm;                 // [W][W]  Gram of the unit rows
  double* D = G + W * W;          // [K][W]  centroid . unit row
  double* nrm = D + K * W;        // [W]
  int* a = reinterpret_cast<int*>(nrm + W);  // [W] (W <= 128)
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const double* Rb = R + (size_t)b * W * W;
  for (int i = tid; i < W; i += PS_KM_THREADS) nrm[i] = sqrt(Rb[(size_t)i * W + i]);
  __syncthreads();
  for (int e = tid; e < W * W; e += PS_KM_THREADS) {
    const int i = e / W, j = e - i * W;
    const double ni = nrm[i], nj = nrm[j];
    G[e] = (ni > 0.0 && nj > 0.0) ? Rb[e] / (ni * nj) : 0.0;
  }
  const int stride = W / K;
  double* cf = coef + (size_t)b * K * W;
  __syncthreads();
  for (int e = tid; e < K * W; e += PS_KM_THREADS) {
    const int j = e / W, k = e - j * W;
    D[e] = G[(size_t)(stride * j) * W + k];
    cf[e] = (k == stride * j) ? 1.0 : 0.0;
  }
  __syncthreads();
  auto do_assign = [&]() {
    for (int i = tid; i < W; i += PS_KM_THREADS) {
      int best = 0;
      double bv = D[i];
      for (int j = 1; j < K; ++j) {
        const double v = D[j * W + i];
        if (v > bv) {
          bv = v;
          best = j;
        }
      }
      a[i] = best;
    }
    __syncthreads();
  };
  for (int it = 0; it < iters; ++it) {
    do_assign();
    if (wv < K) {
      const int j = wv;
      // members of cluster j, rows 0..63 and 64..127
      const unsigned long long m0 = __ballot(lane < W && a[lane] == j);
      const unsigned long long m1 = __ballot(lane + 64 < W && a[lane + 64] == j);
      // member sums of this lane's columns k = lane, lane + 64
      double v0 = 0.0, v1 = 0.0;
      for (int h = 0; h < 2; ++h) {
        unsigned long long m = h ? m1 : m0;
        while (m) {
          const int i = __ffsll((long long)m) - 1 + 64 * h;
          m &= m - 1;
          if (lane < W) v0 += G[(size_t)i * W + lane];
          if (lane + 64 < W) v1 += G[(size_t)i * W + lane + 64];
        }
      }
      // |member sum|^2 = sum over member columns k (ascending) of v[k]
      double n2 = 0.0;
      for (int h = 0; h < 2; ++h) {
        unsigned long long m = h ? m1 : m0;
        while (m) {
          const int k = __ffsll((long long)m) - 1;
          m &= m - 1;
          n2 += __shfl(h ? v1 : v0, k, 64);
        }
      }
      if ((m0 | m1) != 0ull && n2 > 0.0) {
        const double inv = 1.0 / sqrt(n2);
        if (lane < W) {
          D[j * W + lane] = v0 * inv;
          cf[j * W + lane] = ((m0 >> lane) & 1ull) ? inv : 0.0;
        }
        if (lane + 64 < W) {
          D[j * W + lane + 64] = v1 * inv;
          cf[j * W + lane + 64] = ((m1 >> lane) & 1ull) ? inv : 0.0;
        }
      }
    }
    __syncthreads();
  }
  do_assign();
  for (int i = tid; i < W; i += PS_KM_THREADS) {
    assign[(size_t)b * W + i] = a[i];
    norms[(size_t)b * W + i] = nrm[i];
  }
  if (tid == 0) nsel[b] = K;  // centroid rows of this sequence for the query GEMM
}

// ---------------------------------------------------------------------------
// Explicit centroids c_j = sum_i coef[j][i] * x_i / |x_i| (fp64, ascending i),
// and the packed query-path input bf16(RMSNorm(c_j) * g1) (fp64 norm, rounded
// to fp32 then to the storage dtype, as the layer's own input path).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void ps_centroid_kernel(int L, int d, int blk, int W, int K, float eps, int MTt,
                                                          const int32_t* __restrict__ bstart,
                                                          const T* __restrict__ H, const double* __restrict__ coef,
                                                          const double* __restrict__ norms,
                                                          const float* __restrict__ g1, double* __restrict__ cent,
                                                          T* __restrict__ A) {
  __shared__ double red[4];
  __shared__ int mem[128];
  __shared__ double w[128];
  __shared__ int nm;
  const int b = blockIdx.y, j = blockIdx.x, tid = threadIdx.x;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  if (tid == 0) {
    int c = 0;
    for (int i = 0; i < W; ++i) {
      const double cw = coef[((size_t)b * K + j) * W + i];
      if (cw != 0.0) {
        mem[c] = i;
        w[c] = cw;
        ++c;
      }
    }
    nm = c;
  }
  __syncthreads();
  double* cj = cent + ((size_t)b * K + j) * d;
  double ss = 0.0;
  for (int t = tid; t < d; t += 256) {
    double acc = 0.0;
    for (int q = 0; q < nm; ++q) {
      const int i = mem[q];
      const double x = (double)io<T>::ld(H + ((size_t)b * L + ws + i) * d + t);
      acc += w[q] * (x / norms[(size_t)b * W + i]);
    }
    cj[t] = acc;
    ss += acc * acc;
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const double tot = red[0] + red[1] + red[2] + red[3];
  const double rms = sqrt(tot / (double)d + (double)eps);
  const int m = b * K + j;
  for (int t8 = tid * 8; t8 < d; t8 += 256 * 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)(cj[t8 + e] / rms * (double)g1[t8 + e]);
    store_a8(A, m, t8, MTt, d, v);
  }
}

// ---------------------------------------------------------------------------
// NVFP4 residual codes: r = x/|x| - c_a; per 16 elements s = E4M3(amax/6)
// (round to nearest even, saturating at 448), codes = E2M1(r/s) (nearest
// even, saturating at 6, sign bit for negative values); s = 0 gives zeros.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int e4m3_code(double v) {
  if (!(v > 0.0)) return 0;
  if (v >= 448.0) return 0x7E;
  if (v < 0.015625) {  // subnormal range, units of 2^-9
    const int mq = (int)rint(v * 512.0);
    return mq;  // 8 is the smallest normal, 0x08
  }
  int e;
  const double fr = frexp(v, &e);  // v = fr * 2^e, fr in [0.5, 1)
  const double mant = fr * 2.0;     // [1, 2), exponent e-1
  int ex = e - 1;
  int mq = (int)rint((mant - 1.0) * 8.0);
  if (mq == 8) {
    mq = 0;
    ++ex;
  }
  const int code = ((ex + 7) << 3) | mq;
  return code > 0x7E ? 0x7E : code;
}

__device__ __forceinline__ double e4m3_val(int c) {
  const int ex = (c >> 3) & 0xF, mq = c & 7;
  if (ex == 0) return (double)mq * 0.001953125;
  return (1.0 + mq * 0.125) * ldexp(1.0, ex - 7);
}

__device__ __forceinline__ int e2m1_code(double v) {
  const double u = fabs(v);
  int c;
  if (u < 0.25) c = 0;
  else if (u == 0.25) c = 0;
  else if (u < 0.75) c = 1;
  else if (u <= 1.25) c = 2;
  else if (u < 1.75) c = 3;
  else if (u <= 2.5) c = 4;
  else if (u < 3.5) c = 5;
  else if (u <= 5.0) c = 6;
  else c = 7;
  return c | (v < 0.0 ? 8 : 0);
}

template <typename T>
__global__ __launch_bounds__(256) void ps_codes_kernel(int L, int d, int blk, int W, const int32_t* __restrict__ bstart,
                                                       const T* __restrict__ H, const double* __restrict__ norms,
                                                       const int32_t* __restrict__ assign,
                                                       const double* __restrict__ cent, int K,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int b = blockIdx.y, i = blockIdx.x;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  const double n = norms[(size_t)b * W + i];
  const double* c = cent + ((size_t)b * K + assign[(size_t)b * W + i]) * d;
  const T* x = H + ((size_t)b * L + ws + i) * d;
  uint8_t* cd = codes + ((size_t)b * W + i) * (d / 2);
  uint8_t* sc = scales + ((size_t)b * W + i) * (d / 16);
  for (int g = threadIdx.x; g < d / 16; g += blockDim.x) {
    double r[16];
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const double xh = n > 0.0 ? (double)io<T>::ld(x + 16 * g + e) / n : 0.0;
      r[e] = xh - c[16 * g + e];
      amax = fmax(amax, fabs(r[e]));
    }
    const int scode = e4m3_code(amax / 6.0);
    sc[g] = (uint8_t)scode;
    const double s = e4m3_val(scode);
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const int lo = s != 0.0 ? e2m1_code(r[e] / s) : 0;
      const int hi = s != 0.0 ? e2m1_code(r[e + 1] / s) : 0;
      cd[8 * g + e / 2] = (uint8_t)(lo | (hi << 4));
    }
  }
}

// ---------------------------------------------------------------------------
// Centroid queries: sum of the q GEMM's split partials, RoPE at the seed
// row's position (same tables and arithmetic as the layer's query path).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void ps_query_kernel(int L, int blk, int W, int K, int Hq, int dh, int S, int M,
                                                       int ldp, const int32_t* __restrict__ bstart,
                                                       const float* __restrict__ part, const float* __restrict__ rc,
                                                       const float* __restrict__ rs, T* __restrict__ q) {
  const int m = blockIdx.x, b = m / K, j = m - b * K;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  const int pos = ws + (W / K) * j;
  const int nq = Hq * dh, half = dh / 2;
  const float* p0 = part + (size_t)m * ldp;
  for (int e = threadIdx.x; e < Hq * half; e += 256) {
    const int h = e / half, t = e - h * half;
    const int c0 = h * dh + t, c1 = c0 + half;
    float a = 0.f, c = 0.f;
    for (int s = 0; s < S; ++s) {
      a += p0[(size_t)s * M * ldp + c0];
      c += p0[(size_t)s * M * ldp + c1];
    }
    const float cs = rc[(size_t)pos * half + t], sn = rs[(size_t)pos * half + t];
    io<T>::st(q + (size_t)m * nq + c0, a * cs - c * sn);
    io<T>::st(q + (size_t)m * nq + c1, c * cs + a * sn);
  }
}

// ---------------------------------------------------------------------------
// Proxy attention and per-head KL: for query head h, log A[j][w] =
// log-softmax_w(q_j . k_w / sqrt(dh)) over the window keys of h's KV group
// (fp64), KL_h[j] = sum_w A (log A - log A_prev); log A replaces log A_prev.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void ps_attn_kl_kernel(int L, int blk, int W, int K, int Hq, int Hkv, int dh,
                                                         const int32_t* __restrict__ bstart,
                                                         const T* __restrict__ q, const T* __restrict__ Kc,
                                                         double* __restrict__ logA, double* __restrict__ klp) {
  extern __shared__ double sm[];
  double* qs = sm;            // [K][dh]
  double* ks = qs + K * dh;   // [W][dh + 1]
  double* sc = ks + W * (dh + 1);  // [K][W]
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  const int B = gridDim.y;
  const int g = (h * Hkv) / Hq;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  const int nq = Hq * dh, DS = dh + 1;
  for (int e = tid; e < K * dh; e += 256) {
    const int j = e / dh, t = e - j * dh;
    qs[e] = (double)io<T>::ld(q + ((size_t)b * K + j) * nq + h * dh + t);
  }
  const T* kb = Kc + ((size_t)b * Hkv + g) * (size_t)l32_of(L) * dh;
  for (int e = tid; e < W * dh; e += 256) {
    const int w = e / dh, t = e - w * dh;
    ks[w * DS + t] = (double)io<T>::ld(kb + kc_off(ws + w, t, dh));
  }
  __syncthreads();
  const double sq = sqrt((double)dh);
  for (int e = tid; e < K * W; e += 256) {
    const int j = e / W, w = e - j * W;
    double acc = 0.0;
    for (int t = 0; t < dh; ++t) acc += qs[j * dh + t] * ks[w * DS + t];
    sc[e] = acc / sq;
  }
  __syncthreads();
  // one wave per cluster row: log-softmax, KL against the previous step
  const int lane = tid & 63, wv = tid >> 6;
  for (int j = wv; j < K; j += 4) {
    double mx = -INFINITY;
    for (int w = lane; w < W; w += 64) mx = fmax(mx, sc[j * W + w]);
    mx = wave_max(mx);
    double se = 0.0;
    for (int w = lane; w < W; w += 64) se += exp(sc[j * W + w] - mx);
    se = wave_sum(se);
    const double lse = log(se);
    double* la = logA + (((size_t)b * K + j) * Hq + h) * W;
    double kl = 0.0;
    for (int w = lane; w < W; w += 64) {
      const double lv = (sc[j * W + w] - mx) - lse;
      kl += exp(lv) * (lv - la[w]);
      la[w] = lv;
    }
    kl = wave_sum(kl);
    if (lane == 0) klp[((size_t)b * Hq + h) * K + j] = kl;
  }
  (void)B;
}

// ---------------------------------------------------------------------------
// Cluster drift (mean over heads; 0 on a window's first step), top clusters
// (largest drift, lowest index on ties), index set I = current block rows +
// members of the top clusters, ascending.  Records the window start.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void ps_select_kernel(int L, int blk, int W, int K, int Hq, int top,
                                                        const int32_t* __restrict__ bstart,
                                                        const int32_t* __restrict__ assign,
                                                        const double* __restrict__ klp, int32_t* __restrict__ wstart,
                                                        double* __restrict__ kl_out, int32_t* __restrict__ top_out,
                                                        int32_t* __restrict__ idx, int32_t* __restrict__ n_out) {
  __shared__ double kl[16];
  __shared__ int sel[16];
  __shared__ int flag[128];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int bs = bstart[b];
  const int ws = ps_window_start(bs, L, blk, W);
  const bool valid = wstart[b] == ws;
  if (tid < K) {
    double acc = 0.0;
    for (int h = 0; h < Hq; ++h) acc += klp[((size_t)b * Hq + h) * K + tid];
    kl[tid] = valid ? acc / (double)Hq : 0.0;
    kl_out[(size_t)b * K + tid] = kl[tid];
  }
  __syncthreads();
  if (tid < K) {
    // rank of cluster tid by (drift desc, index asc)
    int r = 0;
    for (int j = 0; j < K; ++j) r += (kl[j] > kl[tid]) || (kl[j] == kl[tid] && j < tid);
    sel[tid] = r < top;
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0;
    for (int j = 0; j < K; ++j)
      if (sel[j]) top_out[(size_t)b * top + c++] = j;
    wstart[b] = ws;
  }
  if (tid < W) {
    const int row = ws + tid;
    flag[tid] = (row >= bs && row < bs + blk) || sel[assign[(size_t)b * W + tid]];
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0;
    for (int i = 0; i < W; ++i)
      if (flag[i]) idx[(size_t)b * L + c++] = ws + i;
    n_out[b] = c;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int ps_gram_slices(int d) { return d / PS_SD; }

hipError_t launch_ps_gram(hipStream_t st, bool bf16m, int B, int L, int d, int blk, int W, const int32_t* bstart,
                          const void* H, double* part, double* R) {
  if (d % PS_SD || W > PS_WMAX || W < 1) return hipErrorInvalidValue;
  const int nsl = d / PS_SD;
  const size_t lds = (size_t)((W + 15) / 16) * 16 * (PS_SD + 1) * sizeof(double);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)ps_gram_kernel<bf16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(128 * (PS_SD + 1) * sizeof(double)));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)ps_gram_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(128 * (PS_SD + 1) * sizeof(double)));  // up to 8 tiles of 16 rows
    if (e != hipSuccess) return e;
    attr = true;
  }
  if (bf16m)
    hipLaunchKernelGGL(ps_gram_kernel<bf16>, dim3(nsl, B), dim3(256), lds, st, L, d, blk, W, bstart,
                       (const bf16*)H, part);
  else
    hipLaunchKernelGGL(ps_gram_kernel<float>, dim3(nsl, B), dim3(256), lds, st, L, d, blk, W, bstart,
                       (const float*)H, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ps_gram_reduce_kernel, dim3((W * W + 255) / 256, B), dim3(256), 0, st, W, nsl, part, R);
  return hipGetLastError();
}

hipError_t launch_ps_kmeans(hipStream_t st, int B, int W, int K, int iters, const double* R, int32_t* assign,
                            double* norms, double* coef, int32_t* nsel) {
  if (W > PS_WMAX || W > 128 || K > 16 || K < 1 || W < K) return hipErrorInvalidValue;
  const size_t lds = ((size_t)W * W + K * W + W) * sizeof(double) + (size_t)W * sizeof(int);
  static bool attr = false;
  if (!attr) {
    const size_t mx = ((size_t)PS_WMAX * PS_WMAX + 16 * PS_WMAX + PS_WMAX) * sizeof(double) + PS_WMAX * sizeof(int);
    hipError_t e = hipFuncSetAttribute((const void*)ps_kmeans_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)mx);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(ps_kmeans_kernel, dim3(B), dim3(PS_KM_THREADS), lds, st, W, K, iters, R, assign, norms, coef,
                     nsel);
  return hipGetLastError();
}

hipError_t launch_ps_centroids(hipStream_t st, bool bf16m, int B, int L, int d, int blk, int W, int K, float eps,
                               int MTt, const int32_t* bstart, const void* H, const double* coef,
                               const double* norms, const float* g1, double* cent, void* A) {
  if (bf16m)
    hipLaunchKernelGGL(ps_centroid_kernel<bf16>, dim3(K, B), dim3(256), 0, st, L, d, blk, W, K, eps, MTt, bstart,
                       (const bf16*)H, coef, norms, g1, cent, (bf16*)A);
  else
    hipLaunchKernelGGL(ps_centroid_kernel<float>, dim3(K, B), dim3(256), 0, st, L, d, blk, W, K, eps, MTt, bstart,
                       (const float*)H, coef, norms, g1, cent, (float*)A);
  return hipGetLastError();
}

hipError_t launch_ps_codes(hipStream_t st, bool bf16m, int B, int L, int d, int blk, int W, int K,
                           const int32_t* bstart, const void* H, const double* norms, const int32_t* assign,
                           const double* cent, uint8_t* codes, uint8_t* scales) {
  if (bf16m)
    hipLaunchKernelGGL(ps_codes_kernel<bf16>, dim3(W, B), dim3(256), 0, st, L, d, blk, W, bstart, (const bf16*)H,
                       norms, assign, cent, K, codes, scales);
  else
    hipLaunchKernelGGL(ps_codes_kernel<float>, dim3(W, B), dim3(256), 0, st, L, d, blk, W, bstart, (const float*)H,
                       norms, assign, cent, K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_ps_queries(hipStream_t st, bool bf16m, int B, int L, int blk, int W, int K, int Hq, int dh, int S,
                             int ldp, const int32_t* bstart, const float* part, const float* rc, const float* rs,
                             void* q) {
  const int M = B * K;
  if (bf16m)
    hipLaunchKernelGGL(ps_query_kernel<bf16>, dim3(M), dim3(256), 0, st, L, blk, W, K, Hq, dh, S, M, ldp, bstart, part,
                       rc, rs, (bf16*)q);
  else
    hipLaunchKernelGGL(ps_query_kernel<float>, dim3(M), dim3(256), 0, st, L, blk, W, K, Hq, dh, S, M, ldp, bstart,
                       part, rc, rs, (float*)q);
  return hipGetLastError();
}

hipError_t launch_ps_attn_kl(hipStream_t st, bool bf16m, int B, int L, int blk, int W, int K, int Hq, int Hkv,
                             int dh, const int32_t* bstart, const void* q, const void* Kc, double* logA, double* klp) {
  const size_t lds = ((size_t)K * dh + (size_t)W * (dh + 1) + (size_t)K * W) * sizeof(double);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)ps_attn_kl_kernel<bf16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)ps_attn_kl_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  if (bf16m)
    hipLaunchKernelGGL(ps_attn_kl_kernel<bf16>, dim3(Hq, B), dim3(256), lds, st, L, blk, W, K, Hq, Hkv, dh, bstart,
                       (const bf16*)q, (const bf16*)Kc, logA, klp);
  else
    hipLaunchKernelGGL(ps_attn_kl_kernel<float>, dim3(Hq, B), dim3(256), lds, st, L, blk, W, K, Hq, Hkv, dh, bstart,
                       (const float*)q, (const float*)Kc, logA, klp);
  return hipGetLastError();
}

hipError_t launch_ps_select(hipStream_t st, int B, int L, int blk, int W, int K, int Hq, int top,
                            const int32_t* bstart, const int32_t* assign, const double* klp, int32_t* wstart,
                            double* kl, int32_t* top_out, int32_t* idx, int32_t* n) {
  if (W > PS_WMAX || K > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ps_select_kernel, dim3(B), dim3(128), 0, st, L, blk, W, K, Hq, top, bstart, assign, klp, wstart,
                     kl, top_out, idx, n);
  return hipGetLastError();
}

}  // namespace dllm
