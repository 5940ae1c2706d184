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

constexpr int PS_WMAX = 120;  // window rows: the k-means keeps W x W fp64 in LDS

__device__ __forceinline__ int ps_window_start(int bs, int L, int blk, int W) {
  return min(max(bs - blk, 0), L - W);
}

// Eight consecutive elements (16-byte aligned for bf16, 32 for fp32) as
// doubles.
__device__ __forceinline__ void ld8d(const bf16* p, double* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = (double)__uint_as_float(w[e] << 16);
    v[2 * e + 1] = (double)__uint_as_float(w[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8d(const float* p, double* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 c = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
}

// ---------------------------------------------------------------------------
// Gram partials R[b][s][i][j] = sum over the dims of split s of x_i x_j, for
// the W window rows of sequence b (raw layer inputs; fp64 products of the
// stored values are exact); the k-means adds the PS_GRAM_SPLITS partials in
// split order.  One workgroup per (upper-triangle pair of 16-row tiles,
// sequence, split); the 8 waves of all splits take interleaved 32-dim chunks
// on v_mfma_f64_16x16x4_f64 and a workgroup adds its waves' tiles in wave
// order.  Within a chunk, lane l feeds row l%16 and the 8 dims
// 8*(l/16) .. 8*(l/16)+7 one per MFMA (the same order for both operands, so
// every dim's product enters once).  The tile is stored at (i, j) and (j, i);
// diagonal tiles store only i <= j, so R is exactly symmetric.
// ---------------------------------------------------------------------------
constexpr int PS_GRAM_WAVES = 8;
constexpr int PS_GRAM_SPLITS = 4;

template <typename T>
__global__ __launch_bounds__(64 * PS_GRAM_WAVES) void ps_gram_kernel(int L, int d, int blk, int W,
                                                                     const int32_t* __restrict__ bstart,
                                                                     const T* __restrict__ H,
                                                                     double* __restrict__ R) {
  __shared__ f64x4_t red[PS_GRAM_WAVES][64];
  const int b = blockIdx.y, sp = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int TW = (W + 15) / 16;
  int ti = 0, rem = blockIdx.x;
  while (rem >= TW - ti) {
    rem -= TW - ti;
    ++ti;
  }
  const int tj = ti + rem;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  const int ra = ti * 16 + (lane & 15), rb = tj * 16 + (lane & 15);
  const int k8 = (lane >> 4) * 8;
  const T* pa = H + ((size_t)b * L + ws + min(ra, W - 1)) * d + k8;
  const T* pb = H + ((size_t)b * L + ws + min(rb, W - 1)) * d + k8;
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
  // chunk stride over all waves of all splits; four chunks per pass, all
  // loads issued before the MFMAs
  constexpr int CS = PS_GRAM_SPLITS * PS_GRAM_WAVES * 32;
  for (int c0 = (sp * PS_GRAM_WAVES + wv) * 32; c0 < d; c0 += 4 * CS) {
    double xa[4][8], xb[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = min(c0 + u * CS, d - 32);
      ld8d(pa + c, xa[u]);
      ld8d(pb + c, xb[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool live = c0 + u * CS < d;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (ra >= W || !live) xa[u][e] = 0.0;
        if (rb >= W || !live) xb[u][e] = 0.0;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[u][e], xb[u][e], acc, 0, 0, 0);
    }
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
  f64x4_t t = red[0][lane];
#pragma unroll
  for (int w = 1; w < PS_GRAM_WAVES; ++w) t += red[w][lane];
  // D register e of lane l: row l/16 + 4e of tile ti, column l%16 of tile tj
  double* Rb = R + ((size_t)b * PS_GRAM_SPLITS + sp) * W * W;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = ti * 16 + (lane >> 4) + 4 * e, j = tj * 16 + (lane & 15);
    if (i < W && j < W && (ti != tj || i <= j)) {
      Rb[(size_t)i * W + j] = t[e];
      Rb[(size_t)j * W + i] = t[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Spherical k-means on the Gram matrix (one workgroup per sequence, wave j
// owns cluster j).  Seeds: window rows stride*j.  Each iteration: assign each
// row to the cluster of largest dot product (lowest index on ties); every
// cluster with members and a non-zero member sum becomes the normalised
// member sum; others keep their centroid.  Then a final assignment.  Outputs
// the assignment, the row norms and each centroid's coefficients over the
// unit rows.  A cluster's members come from two 64-row ballots and are
// visited in ascending row order (eight at a time, their rows read together);
// member sums and the squared norm are added in that order.
// ---------------------------------------------------------------------------
constexpr int PS_KM_THREADS = 1024;  // 16 waves: one per cluster (K <= 16)
constexpr int PS_KM_EPT = 9;         // Gram elements a thread loads at once (one pass for W <= 96)

__global__ __launch_bounds__(PS_KM_THREADS) void ps_kmeans_kernel(int W, int K, int iters, const double* __restrict__ R,
                                                                 int32_t* __restrict__ assign,
                                                                 double* __restrict__ norms,
                                                                 double* __restrict__ coef, int32_t* __restrict__ nsel) {
  extern __shared__ double sm[];
  double* G = sm;                 // [W][W]  Gram of the unit rows
  double* D = G + W * W;          // [K][W]  centroid . unit row
  double* nrm = D + K * W;        // [W]
  double* dump = nrm + W;         // [1]  target of the stores past the Gram
  int* a = reinterpret_cast<int*>(dump + 1);  // [W] (W <= 128)
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  // Gram = sum of the split partials in split order (a thread's loads for up
  // to PS_KM_EPT elements issued together), then normalised
  const double* Rb = R + (size_t)b * PS_GRAM_SPLITS * W * W;
  const int WW = W * W;
  for (int e0 = tid; e0 < WW; e0 += PS_KM_EPT * PS_KM_THREADS) {
    double v[PS_KM_EPT][PS_GRAM_SPLITS];
#pragma unroll
    for (int u = 0; u < PS_KM_EPT; ++u)
#pragma unroll
      for (int q = 0; q < PS_GRAM_SPLITS; ++q)
        v[u][q] = Rb[(size_t)q * WW + min(e0 + u * PS_KM_THREADS, WW - 1)];
#pragma unroll
    for (int u = 0; u < PS_KM_EPT; ++u) {
      const int e = e0 + u * PS_KM_THREADS;
      double t = v[u][0];
#pragma unroll
      for (int q = 1; q < PS_GRAM_SPLITS; ++q) t += v[u][q];
      // unconditional store (so the loads stay in the batch above)
      *(e < WW ? G + e : dump) = t;
    }
  }
  __syncthreads();
  for (int i = tid; i < W; i += PS_KM_THREADS) nrm[i] = sqrt(G[(size_t)i * W + i]);
  __syncthreads();
  {
    // unit-row Gram G[i][j] / (|x_i| |x_j|): thread column j = tid % 128,
    // rows tid / 128 + 8 t (a wave touches one row, conflict-free)
    const int j = tid & 127;
    if (j < W) {
      const double nj = nrm[j];
      for (int i = tid >> 7; i < W; i += PS_KM_THREADS / 128) {
        const double ni = nrm[i];
        double* g = G + (size_t)i * W + j;
        *g = (ni > 0.0 && nj > 0.0) ? *g / (ni * nj) : 0.0;
      }
    }
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
  for (int i = tid; i < W; i += PS_KM_THREADS) a[i] = -1;
  // returns whether any row changed cluster
  auto do_assign = [&]() -> bool {
    int changed = 0;
    for (int i = tid; i < W; i += PS_KM_THREADS) {
      // all K dot products read first (one LDS latency), then compared in
      // cluster order
      double dv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) dv[j] = D[(j < K ? j : K - 1) * W + i];
      int best = 0;
      double bv = dv[0];
#pragma unroll
      for (int j = 1; j < 16; ++j)
        if (j < K && dv[j] > bv) {
          bv = dv[j];
          best = j;
        }
      changed |= a[i] != best;
      a[i] = best;
    }
    return __syncthreads_or(changed) != 0;
  };
  for (int it = 0; it < iters; ++it) {
    // an unchanged assignment rebuilds the same centroids, so every later
    // iteration repeats this one: stop early (the result is identical)
    if (!do_assign()) break;
    if (wv < K) {
      const int j = wv;
      // members of cluster j, rows 0..63 and 64..127
      const unsigned long long m0 = __ballot(lane < W && a[lane] == j);
      const unsigned long long m1 = __ballot(lane + 64 < W && a[lane + 64] == j);
      // member sums of this lane's columns k = lane, lane + 64; members are
      // taken eight at a time (their rows read together), added in
      // ascending row order
      double v0 = 0.0, v1 = 0.0;
      for (int h = 0; h < 2; ++h) {
        unsigned long long m = h ? m1 : m0;
        while (m) {
          int ii[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            ii[u] = m ? __ffsll((long long)m) - 1 + 64 * h : -1;
            m &= m - 1;
          }
          double g0[8], g1[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (ii[u] >= 0) {
              g0[u] = lane < W ? G[(size_t)ii[u] * W + lane] : 0.0;
              g1[u] = lane + 64 < W ? G[(size_t)ii[u] * W + lane + 64] : 0.0;
            }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (ii[u] >= 0) {
              if (lane < W) v0 += g0[u];
              if (lane + 64 < W) v1 += g1[u];
            }
        }
      }
      // |member sum|^2 = sum over member columns k (ascending) of v[k], eight
      // shuffles at a time
      double n2 = 0.0;
      for (int h = 0; h < 2; ++h) {
        unsigned long long m = h ? m1 : m0;
        const double vh = h ? v1 : v0;
        while (m) {
          int kk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            kk[u] = m ? __ffsll((long long)m) - 1 : -1;
            m &= m - 1;
          }
          double sv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (kk[u] >= 0) sv[u] = __shfl(vh, kk[u], 64);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (kk[u] >= 0) n2 += sv[u];
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
  (void)do_assign();
  for (int i = tid; i < W; i += PS_KM_THREADS) {
    assign[(size_t)b * W + i] = a[i];
    norms[(size_t)b * W + i] = nrm[i];
  }
  if (tid == 0) nsel[b] = K;  // centroid rows of this sequence for the query GEMM
}

// ---------------------------------------------------------------------------
// Explicit centroids c_j = sum_i coef[j][i] * x_i / |x_i| (fp64, ascending i),
// and the packed query-path input bf16(RMSNorm(c_j) * g1) (fp64 norm, rounded
// to fp32 then to the storage dtype, as the layer's own input path).  One
// workgroup per (cluster, sequence); each thread owns 8 consecutive dims (of
// up to 8192) and reads the members' rows raw, CB at a time, so their loads
// overlap; the members' weights and norms are staged in LDS.
// ---------------------------------------------------------------------------
constexpr int PS_CENT_THREADS = 512;

template <typename T>
struct RawRow8;  // 8 consecutive stored values of a row, as loaded
template <>
struct RawRow8<bf16> {
  static constexpr int CB = 16;  // member rows in flight per thread
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void widen(double* v) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = (double)__uint_as_float(w[e] << 16);
      v[2 * e + 1] = (double)__uint_as_float(w[e] & 0xffff0000u);
    }
  }
};
template <>
struct RawRow8<float> {
  static constexpr int CB = 8;
  float4 a, c;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    c = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void widen(double* v) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }
};

template <typename T>
__global__ __launch_bounds__(PS_CENT_THREADS) void ps_centroid_kernel(
    int L, int d, int blk, int W, int K, float eps, int MTt, const int32_t* __restrict__ bstart,
    const T* __restrict__ H, const double* __restrict__ coef, const double* __restrict__ norms,
    const float* __restrict__ g1, double* __restrict__ cent, T* __restrict__ A) {
  constexpr int CB = RawRow8<T>::CB;
  constexpr int NIT = 2;  // dims per thread: NIT groups of 8 (d <= 8192)
  __shared__ double red[PS_CENT_THREADS / 64];
  __shared__ int mem[128];
  __shared__ double wmem[128], nmem[128];
  __shared__ int nm_s;
  const int b = blockIdx.y, j = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  const double* cw = coef + ((size_t)b * K + j) * W;
  const double* nb = norms + (size_t)b * W;
  if (wv == 0) {  // members in ascending row order (W <= 128), with weight and norm
    const double w0 = lane < W ? cw[lane] : 0.0, w1 = lane + 64 < W ? cw[lane + 64] : 0.0;
    const double n0 = lane < W ? nb[lane] : 0.0, n1 = lane + 64 < W ? nb[lane + 64] : 0.0;
    const bool f0 = lane < W && w0 != 0.0;
    const bool f1 = lane + 64 < W && w1 != 0.0;
    const unsigned long long m0 = __ballot(f0), m1 = __ballot(f1);
    const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int c0 = __popcll(m0);
    if (f0) {
      const int k = __popcll(m0 & below);
      mem[k] = lane;
      wmem[k] = w0;
      nmem[k] = n0;
    }
    if (f1) {
      const int k = c0 + __popcll(m1 & below);
      mem[k] = lane + 64;
      wmem[k] = w1;
      nmem[k] = n1;
    }
    if (lane == 0) nm_s = c0 + __popcll(m1);
  }
  __syncthreads();
  const int nm = nm_s;
  const T* xw = H + ((size_t)b * L + ws) * d;
  double* cj = cent + ((size_t)b * K + j) * d;
  double acc[NIT][8];
  double ss = 0.0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int t8 = (tid + it * PS_CENT_THREADS) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[it][e] = 0.0;
    if (t8 >= d) continue;
    for (int q0 = 0; q0 < nm; q0 += CB) {
      // every row address first, then the CB loads back to back
      const T* src[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) src[u] = xw + (size_t)mem[min(q0 + u, nm - 1)] * d + t8;
      RawRow8<T> raw[CB];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < CB; ++u) raw[u].load(src[u]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < CB; ++u)
        if (q0 + u < nm) {
          double x[8];
          raw[u].widen(x);
          const double wq = wmem[q0 + u], nq = nmem[q0 + u];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[it][e] += wq * (x[e] / nq);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cj[t8 + e] = acc[it][e];
      ss += acc[it][e] * acc[it][e];
    }
  }
  const double tot = block_sum<PS_CENT_THREADS / 64>(ss, red);
  const double rms = sqrt(tot / (double)d + (double)eps);
  const int m = b * K + j;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int t8 = (tid + it * PS_CENT_THREADS) * 8;
    if (t8 >= d) continue;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)(acc[it][e] / rms * (double)g1[t8 + e]);
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
    // the row's and the centroid's values loaded unconditionally (issued
    // together), then the unit row (zero for a zero row)
    double xv[16], cv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      xv[e] = (double)io<T>::ld(x + 16 * g + e);
      cv[e] = c[16 * g + e];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const double xh = n > 0.0 ? xv[e] / n : 0.0;
      r[e] = xh - cv[e];
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
  const int half = dh / 2;
  const int e = blockIdx.y * 256 + threadIdx.x;  // one rotation pair per thread
  if (e >= Hq * half) return;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  const int pos = ws + (W / K) * j;
  const int nq = Hq * dh;
  const int h = e / half, t = e - h * half;
  const int c0 = h * dh + t, c1 = c0 + half;
  const float* p0 = part + (size_t)m * ldp;
  const size_t sstride = (size_t)M * ldp;
  const float a = sum_splits(p0 + c0, sstride, S);
  const float c = sum_splits(p0 + c1, sstride, S);
  const float cs = rc[(size_t)pos * half + t], sn = rs[(size_t)pos * half + t];
  io<T>::st(q + (size_t)m * nq + c0, a * cs - c * sn);
  io<T>::st(q + (size_t)m * nq + c1, c * cs + a * sn);
}

// ---------------------------------------------------------------------------
// Proxy attention and per-head KL: for query head h, log A[j][w] =
// log-softmax_w(q_j . k_w / sqrt(dh)) over the window keys of h's KV group
// (fp64), KL_h[j] = sum_w A (log A - log A_prev); log A replaces log A_prev.
// The scores are one 16-row tile of cluster queries against 16-key tiles on
// v_mfma_f64_16x16x4_f64 (products of stored values are exact in fp64); lane
// l feeds query/key row l%16 and the dims (dh/4)*(l/16) .. +dh/4, one per
// MFMA, in the same order for both operands.
// ---------------------------------------------------------------------------
// Whether sequence b's drift refresh at this layer is due: every step at
// tau_upd <= 0, on a window's first step, or once tau_upd tokens were decoded
// since the layer's last refresh.
__device__ __forceinline__ bool ps_refresh_due(int b, int ws, int tau_upd, const int32_t* __restrict__ wstart,
                                               const int32_t* __restrict__ n_hist,
                                               const int32_t* __restrict__ upd_hist) {
  return tau_upd <= 0 || wstart[b] != ws || n_hist[b] - upd_hist[b] >= tau_upd;
}

template <typename T>
__global__ __launch_bounds__(256) void ps_attn_kl_kernel(int L, int blk, int W, int K, int Hq, int Hkv, int dh,
                                                         const int32_t* __restrict__ bstart,
                                                         const T* __restrict__ q, const T* __restrict__ Kc,
                                                         double* __restrict__ logA, double* __restrict__ klp,
                                                         int tau_upd, const int32_t* __restrict__ wstart,
                                                         const int32_t* __restrict__ n_hist,
                                                         const int32_t* __restrict__ upd_hist) {
  __shared__ double sc[16 * PS_WMAX];  // [K][W]
  const int b = blockIdx.y, h = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = (h * Hkv) / Hq;
  const int ws = ps_window_start(bstart[b], L, blk, W);
  // without a due refresh the stored attention stays (the KL is not used)
  const bool store = ps_refresh_due(b, ws, tau_upd, wstart, n_hist, upd_hist);
  const int nq = Hq * dh, kq = dh / 4;
  const int r = lane & 15, slot = lane >> 4;
  const T* qrow = q + ((size_t)b * K + min(r, K - 1)) * nq + h * dh + slot * kq;
  const T* kb = Kc + ((size_t)b * Hkv + g) * (size_t)l32_of(L) * dh;
  const double sq = sqrt((double)dh);
  const int TW = (W + 15) / 16;
  // previous log-attention of this wave's rows (j = wv + 4u, keys lane and
  // lane + 64), fetched before the scores so its latency overlaps them
  double prev[4][2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = min(wv + 4 * u, K - 1);
    const double* la = logA + (((size_t)b * K + j) * Hq + h) * W;
    prev[u][0] = la[min(lane, W - 1)];
    prev[u][1] = la[min(lane + 64, W - 1)];
  }
  for (int tw = wv; tw < TW; tw += 4) {
    const int w = tw * 16 + r;
    const int wc = min(w, W - 1);
    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
    // kq is 8, 16 or 32 (dh % 32 == 0, dh <= 128): up to four 8-dim chunks,
    // all loads issued before the MFMAs
    double xa[4][8], xb[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = min(u * 8, kq - 8);
      ld8d(qrow + c, xa[u]);
      ld8d(kb + kc_off(ws + wc, slot * kq + c, dh), xb[u]);
    }
    // chunks past kq are zeroed rather than skipped (a skip let the loads
    // sink into per-chunk branches, each with its own wait); their products
    // add exact zeros
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool live = u * 8 < kq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (r >= K || !live) xa[u][e] = 0.0;
        if (w >= W || !live) xb[u][e] = 0.0;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(xa[u][e], xb[u][e], acc, 0, 0, 0);
    }
    // D register e of lane l: query row l/16 + 4e, key tw*16 + l%16
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = slot + 4 * e, wk = tw * 16 + r;
      if (j < K && wk < W) sc[j * W + wk] = acc[e] / sq;
    }
  }
  __syncthreads();
  // one wave per cluster row: log-softmax, KL against the previous step
  // (W <= 120: each lane holds keys lane and lane + 64)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = wv + 4 * u;
    if (j >= K) break;
    const bool k1 = lane + 64 < W, k0 = lane < W;
    const double s0 = k0 ? sc[j * W + lane] : -INFINITY;
    const double s1 = k1 ? sc[j * W + lane + 64] : -INFINITY;
    const double mx = wave_max(fmax(s0, s1));
    double se = (k0 ? exp(s0 - mx) : 0.0);
    if (k1) se += exp(s1 - mx);
    se = wave_sum(se);
    const double lse = log(se);
    double* la = logA + (((size_t)b * K + j) * Hq + h) * W;
    double kl = 0.0;
    if (k0) {
      const double lv = (s0 - mx) - lse;
      kl += exp(lv) * (lv - prev[u][0]);
      if (store) la[lane] = lv;
    }
    if (k1) {
      const double lv = (s1 - mx) - lse;
      kl += exp(lv) * (lv - prev[u][1]);
      if (store) la[lane + 64] = lv;
    }
    kl = wave_sum(kl);
    if (lane == 0) klp[((size_t)b * Hq + h) * K + j] = kl;
  }
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
                                                        int32_t* __restrict__ idx, int32_t* __restrict__ n_out,
                                                        int32_t* __restrict__ valid_out, int tau_upd,
                                                        const int32_t* __restrict__ n_hist,
                                                        int32_t* __restrict__ upd_hist) {
  __shared__ double kl[16];
  __shared__ int sel[16];
  __shared__ int cnt0;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int bs = bstart[b];
  const int ws = ps_window_start(bs, L, blk, W);
  const bool upd = ps_refresh_due(b, ws, tau_upd, wstart, n_hist, upd_hist);
  const bool valid = upd && wstart[b] == ws;
  if (tid < K) {
    // mean over heads, heads added in order (loads issued 8 at a time)
    double acc = 0.0;
    for (int h0 = 0; h0 < Hq; h0 += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = h0 + u < Hq ? klp[((size_t)b * Hq + h0 + u) * K + tid] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (h0 + u < Hq) acc += v[u];
    }
    kl[tid] = valid ? acc / (double)Hq : 0.0;
    kl_out[(size_t)b * K + tid] = kl[tid];
  }
  __syncthreads();
  if (tid < K) {
    // rank of cluster tid by (drift desc, index asc)
    int rk = 0;
    for (int j = 0; j < K; ++j) rk += (kl[j] > kl[tid]) || (kl[j] == kl[tid] && j < tid);
    sel[tid] = rk < top;
  }
  __syncthreads();
  if (tid < K && sel[tid]) {
    int pos = 0;  // selected clusters listed in index order
    for (int j = 0; j < tid; ++j) pos += sel[j];
    top_out[(size_t)b * top + pos] = tid;
  }
  if (tid == 0) {
    if (upd) {
      wstart[b] = ws;
      upd_hist[b] = n_hist[b];
    }
    valid_out[b] = valid ? 1 : 0;
  }
  // I = current block rows + members of the selected clusters, ascending
  const int row = ws + tid;
  const bool f = tid < W && ((row >= bs && row < bs + blk) || (upd && sel[assign[(size_t)b * W + tid]]));
  const unsigned long long m = __ballot(f);
  const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
  if (tid == 0) cnt0 = __popcll(m);
  __syncthreads();
  const int off = (tid >> 6) ? cnt0 : 0;
  if (f) idx[(size_t)b * L + off + __popcll(m & below)] = row;
  if (tid == 64) n_out[b] = cnt0 + __popcll(m);
}

// ---------------------------------------------------------------------------
// Polestar-Commit (Polestar page, section 2B), one workgroup per sequence:
// wave 0 holds the current block's rows, wave 1 the next block's.  stats:
// [B][2 blk][4] LM-head statistics of both blocks.  A masked current row
// commits at conf >= thr, or when its drift D (its cluster's drift at the last
// layer, defined when drift_valid) exceeds the mean of its earlier drifts in
// this block by more than alpha (thr - conf)^2; if none commits, the most
// confident masked row (lowest position on ties).  When a top cluster has a
// member among the window rows after the block, the next block's masked rows
// with conf >= thr commit too.  History gets the current block's commits then
// the next block's, ascending; entropy gate and block advance as in the
// threshold commit.  Then D is added to the drift history (cleared when the
// block advances) and drift_valid is cleared.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void ps_commit_kernel(
    int L, int blk, int W, int K, int top, double thr, double alpha, double tau, const double* __restrict__ stats,
    const double* __restrict__ kl, const int32_t* __restrict__ assign, const int32_t* __restrict__ top_c,
    int32_t* __restrict__ drift_valid, double* __restrict__ dsum, int32_t* __restrict__ dcnt,
    int32_t* __restrict__ tokens, uint8_t* __restrict__ committed, int32_t* __restrict__ history,
    int32_t* __restrict__ n_history, int32_t* __restrict__ n_new, int32_t* __restrict__ block_start,
    uint8_t* __restrict__ full_next, double* __restrict__ max_entropy) {
  __shared__ int s_hit, s_cnt[2], s_nbs;
  __shared__ double s_e[2];
  __shared__ uint8_t done_row[128];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bs = block_start[b];
  const bool active = bs < L;
  const int ws = ps_window_start(active ? bs : 0, L, blk, W);
  const bool valid = active && drift_valid[b] != 0;
  uint8_t* cm = committed + (size_t)b * L;
  if (wv == 1) {
    // suffix hit: a top cluster among the window rows after the current block
    unsigned tmask = 0u;
    for (int t = 0; t < top; ++t) tmask |= 1u << top_c[(size_t)b * top + t];
    const int first = bs + blk - ws;
    bool h = false;
    for (int r = lane; r < W; r += 64)
      if (r >= first && ((tmask >> assign[(size_t)b * W + r]) & 1u)) h = true;
    const bool any = __ballot(h) != 0ull;
    if (lane == 0) s_hit = (valid && any) ? 1 : 0;
  }
  const int row = bs + wv * blk + lane;
  const bool rv = active && lane < blk && row < L;
  double conf = 0.0, ent = 0.0, D = 0.0;
  int tok = 0;
  bool cand = false;
  if (rv) {
    const double* p = stats + ((size_t)b * 2 * blk + wv * blk + lane) * 4;
    conf = 1.0 / p[2];
    ent = log(p[2]) - p[3] / p[2];
    tok = (int)p[1];
    cand = cm[row] == 0;
  }
  bool pick = false;
  if (wv == 0) {
    int cnt = 0;
    double sm = 0.0;
    if (rv) {
      cnt = dcnt[(size_t)b * blk + lane];
      sm = dsum[(size_t)b * blk + lane];
      if (valid) D = kl[(size_t)b * K + assign[(size_t)b * W + (row - ws)]];
    }
    if (cand) {
      if (conf >= thr) {
        pick = true;
      } else if (valid && cnt > 0) {
        const double delta = D - sm / (double)cnt;
        const double t = thr - conf;
        pick = delta > alpha * (t * t);
      }
    }
    const uint64_t any_pick = __ballot(pick);
    const uint64_t any_cand = __ballot(cand);
    if (any_pick == 0ull && any_cand != 0ull) {
      // most confident candidate, lowest position on ties
      double bc = cand ? conf : -1.0;
      int br = cand ? row : 0x7fffffff;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const double oc = __shfl_xor(bc, o, 64);
        const int orr = __shfl_xor(br, o, 64);
        if (oc > bc || (oc == bc && orr < br)) {
          bc = oc;
          br = orr;
        }
      }
      pick = cand && row == br;
    }
  }
  __syncthreads();
  if (wv == 1) pick = s_hit != 0 && cand && conf >= thr;
  const uint64_t mask = __ballot(pick);
  double e = pick ? ent : 0.0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) e = fmax(e, __shfl_xor(e, o, 64));
  if (lane == 0) {
    s_cnt[wv] = __popcll(mask);
    s_e[wv] = e;
  }
  // rows of both blocks committed after this step (rows past L count as done)
  if (lane < blk) done_row[wv * blk + lane] = (!rv || !cand || pick) ? 1 : 0;
  __syncthreads();
  const int nh = n_history[b];
  if (pick) {
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    tokens[(size_t)b * L + row] = tok;
    cm[row] = 1;
    history[(size_t)b * L + nh + (wv ? s_cnt[0] : 0) + rank] = row;
  }
  if (tid == 0) {
    int nbs = bs;
    if (active) {
      bool cur_done = true;
      for (int j = 0; j < blk; ++j) cur_done = cur_done && done_row[j];
      if (cur_done) {
        nbs = bs + blk;
        if (nbs < L) {
          bool nxt_done = true;
          for (int j = 0; j < blk; ++j) nxt_done = nxt_done && done_row[blk + j];
          if (nxt_done) {
            nbs += blk;
            // later blocks are untouched by this step
            while (nbs < L) {
              bool c = true;
              for (int j = 0; j < blk && nbs + j < L; ++j) c = c && cm[nbs + j] != 0;
              if (!c) break;
              nbs += blk;
            }
          }
        }
      }
    }
    s_nbs = nbs;
    const int cnt = s_cnt[0] + s_cnt[1];
    const double em = fmax(s_e[0], s_e[1]);
    n_history[b] = nh + cnt;
    n_new[b] = cnt;
    max_entropy[b] = em;
    full_next[b] = em > tau ? 1 : 0;
    block_start[b] = nbs;
    drift_valid[b] = 0;
  }
  __syncthreads();
  if (wv == 0 && lane < blk && active) {
    double* sp = dsum + (size_t)b * blk + lane;
    int32_t* cp = dcnt + (size_t)b * blk + lane;
    if (s_nbs != bs) {
      *sp = 0.0;
      *cp = 0;
    } else if (valid && rv) {
      *sp = *sp + D;
      *cp = *cp + 1;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int ps_gram_splits() { return PS_GRAM_SPLITS; }

hipError_t launch_ps_gram(hipStream_t st, bool bf16m, int B, int L, int d, int blk, int W, const int32_t* bstart,
                          const void* H, double* R) {
  if (d % 32 || W > PS_WMAX || W < 1) return hipErrorInvalidValue;
  const int TW = (W + 15) / 16;
  const dim3 grid(TW * (TW + 1) / 2, B, PS_GRAM_SPLITS);
  if (bf16m)
    hipLaunchKernelGGL(ps_gram_kernel<bf16>, grid, dim3(64 * PS_GRAM_WAVES), 0, st, L, d, blk, W, bstart,
                       (const bf16*)H, R);
  else
    hipLaunchKernelGGL(ps_gram_kernel<float>, grid, dim3(64 * PS_GRAM_WAVES), 0, st, L, d, blk, W, bstart,
                       (const float*)H, R);
  return hipGetLastError();
}

hipError_t launch_ps_kmeans(hipStream_t st, int B, int W, int K, int iters, const double* R, int32_t* assign,
                            double* norms, double* coef, int32_t* nsel) {
  if (W > PS_WMAX || W > 128 || K > 16 || K < 1 || W < K) return hipErrorInvalidValue;
  const size_t lds = ((size_t)W * W + K * W + W + 1) * sizeof(double) + (size_t)W * sizeof(int);
  static std::atomic<unsigned long long> attr{0};
  hipError_t ea = once_per_device(attr, [] {
    const size_t mx = ((size_t)PS_WMAX * PS_WMAX + 16 * PS_WMAX + PS_WMAX + 1) * sizeof(double) + PS_WMAX * sizeof(int);
    return hipFuncSetAttribute((const void*)ps_kmeans_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)mx);
  });
  if (ea != hipSuccess) return ea;
  hipLaunchKernelGGL(ps_kmeans_kernel, dim3(B), dim3(PS_KM_THREADS), lds, st, W, K, iters, R, assign, norms, coef,
                     nsel);
  return hipGetLastError();
}

hipError_t launch_ps_centroids(hipStream_t st, bool bf16m, int B, int L, int d, int blk, int W, int K, float eps,
                               int MTt, const int32_t* bstart, const void* H, const double* coef,
                               const double* norms, const float* g1, double* cent, void* A) {
  if (d > 2 * PS_CENT_THREADS * 8 || d % 8) return hipErrorInvalidValue;  // dims per thread: two groups of 8
  if (bf16m)
    hipLaunchKernelGGL(ps_centroid_kernel<bf16>, dim3(K, B), dim3(PS_CENT_THREADS), 0, st, L, d, blk, W, K, eps, MTt, bstart,
                       (const bf16*)H, coef, norms, g1, cent, (bf16*)A);
  else
    hipLaunchKernelGGL(ps_centroid_kernel<float>, dim3(K, B), dim3(PS_CENT_THREADS), 0, st, L, d, blk, W, K, eps, MTt, bstart,
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
  const dim3 grid(M, (Hq * (dh / 2) + 255) / 256);
  if (bf16m)
    hipLaunchKernelGGL(ps_query_kernel<bf16>, grid, dim3(256), 0, st, L, blk, W, K, Hq, dh, S, M, ldp, bstart, part,
                       rc, rs, (bf16*)q);
  else
    hipLaunchKernelGGL(ps_query_kernel<float>, grid, dim3(256), 0, st, L, blk, W, K, Hq, dh, S, M, ldp, bstart,
                       part, rc, rs, (float*)q);
  return hipGetLastError();
}

hipError_t launch_ps_attn_kl(hipStream_t st, bool bf16m, int B, int L, int blk, int W, int K, int Hq, int Hkv,
                             int dh, const int32_t* bstart, const void* q, const void* Kc, double* logA, double* klp,
                             int tau_upd, const int32_t* wstart, const int32_t* n_hist, const int32_t* upd_hist) {
  if (W > PS_WMAX || W < 1 || K > 16 || K < 1 || dh % 32 || dh > 128) return hipErrorInvalidValue;
  if (bf16m)
    hipLaunchKernelGGL(ps_attn_kl_kernel<bf16>, dim3(Hq, B), dim3(256), 0, st, L, blk, W, K, Hq, Hkv, dh, bstart,
                       (const bf16*)q, (const bf16*)Kc, logA, klp, tau_upd, wstart, n_hist, upd_hist);
  else
    hipLaunchKernelGGL(ps_attn_kl_kernel<float>, dim3(Hq, B), dim3(256), 0, st, L, blk, W, K, Hq, Hkv, dh, bstart,
                       (const float*)q, (const float*)Kc, logA, klp, tau_upd, wstart, n_hist, upd_hist);
  return hipGetLastError();
}

hipError_t launch_ps_select(hipStream_t st, int B, int L, int blk, int W, int K, int Hq, int top,
                            const int32_t* bstart, const int32_t* assign, const double* klp, int32_t* wstart,
                            double* kl, int32_t* top_out, int32_t* idx, int32_t* n, int32_t* valid, int tau_upd,
                            const int32_t* n_hist, int32_t* upd_hist) {
  if (W > PS_WMAX || K > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ps_select_kernel, dim3(B), dim3(128), 0, st, L, blk, W, K, Hq, top, bstart, assign, klp, wstart,
                     kl, top_out, idx, n, valid, tau_upd, n_hist, upd_hist);
  return hipGetLastError();
}

hipError_t launch_ps_commit(hipStream_t st, int B, int L, int blk, int W, int K, int top, double thr, double alpha,
                            double tau, const double* stats, const double* kl, const int32_t* assign,
                            const int32_t* top_c, int32_t* drift_valid, double* dsum, int32_t* dcnt,
                            int32_t* tokens, uint8_t* committed, int32_t* history, int32_t* n_history,
                            int32_t* n_new, int32_t* block_start, uint8_t* full_next, double* max_entropy) {
  if (W > PS_WMAX || K > 16 || blk > 64 || top > K) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ps_commit_kernel, dim3(B), dim3(128), 0, st, L, blk, W, K, top, thr, alpha, tau, stats, kl,
                     assign, top_c, drift_valid, dsum, dcnt, tokens, committed, history, n_history, n_new,
                     block_start, full_next, max_entropy);
  return hipGetLastError();
}

}  // namespace dllm
