// SPA-Cache method step 1 ("Singular proxy for adaptive caching in diffusion
// language models"): project each changed row's layer input onto the rank-r
// value subspace, x W_r, and score it by the cosine against the proxy cached
// at the row's last refresh (lowest similarity = most drift).
//
// Every decision-feeding quantity is fp64.  The normalised input's gain g1 is
// applied to x in fp64 (exactly: at most 24+24 significant bits), the basis is
// kept in fp32 as given and widened exactly, and the products are accumulated
// by v_mfma_f64_16x16x4_f64, so the result is the fp64 definition up to the
// order of the fp64 sum.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int PX_KC = 32;      // k per chunk: 8 MFMA steps of 4
constexpr int PX_NCT = 2;      // 16-column tiles per wave
constexpr int PX_TARGET = 1024;  // workgroups to aim for (512 -> 1024: 9.5 -> 8.3 us per layer at L = 1024, d = 4096)
constexpr int PX_SMAX = 32;    // most partial splits

// Basis width as stored: r rounded up to 32, 64 or 128 (zero columns).
int proxy_rpad(int r) { return r <= 32 ? 32 : (r <= 64 ? 64 : 128); }

// Partial splits across workgroups; each workgroup's 4 waves split its K
// range again and are summed in LDS.
static int proxy_splits(int max_rows, int d, int rpad) {
  const int tasks = ((max_rows + 15) / 16) * (rpad / 16 / PX_NCT);
  const int kq = d / PX_KC;  // k chunks
  int s = 1;
  while (s * 2 <= PX_SMAX && kq % (s * 2) == 0 && kq / (s * 2) >= 4 && tasks * s * 2 <= PX_TARGET) s *= 2;
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

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// partial[s][m][j] = sum over k in split s of (x[m][k] g1[k]) W_r[k][j].
// A workgroup owns 16 rows x (16 * PX_NCT) columns and a K range whose 32-k
// chunks its 4 waves split four ways.  In MFMA step t of a 32-k chunk, lane l = i + 16 q
// supplies A[i][q] = x[row i][k0 + 8q + t] g1[k0 + 8q + t] and
// B[q][j] = W_r[k0 + 8q + t][col j] (any assignment of k to the four MFMA
// k-slots sums the same terms), so a lane's A values for a chunk are 8
// consecutive inputs (one 16-byte load) and its B values are 8 consecutive
// fp32 of the packed basis.
template <typename T>
__global__ __launch_bounds__(256) void proxy_partial_kernel(int B, int L, int d, int rpad, int kps, int cap,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ n,
                                                            const T* __restrict__ H,
                                                            const float* __restrict__ g1,
                                                            const float* __restrict__ wp,
                                                            double* __restrict__ partial) {
  constexpr int XV = XVec<T>::N;
  __shared__ f64x4_t red[3][PX_NCT][64];
  const int M = total_rows(n, B, cap);
  const int ncg = rpad / (16 * PX_NCT);
  const int task = blockIdx.x;
  const int rt = task / ncg, cg = task % ncg;
  if (rt * 16 >= M) return;
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 15, q = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = rt * 16 + i;
  // the row's sequence-0 list entry, loaded before anything else (see
  // row_resolve); the row itself is resolved after the first chunk's gain
  // and basis loads are issued
  const int n0 = n[0];
  const int i0 = idx[m < L ? m : L - 1];
  bool valid = false;
  const T* xrow = H + 8 * q;  // rows past M read row 0 and are zeroed
  // this wave's chunks of the workgroup's K range
  const int nch = kps / PX_KC;
  const int c_beg = blockIdx.y * nch + (wv * nch) / 4;
  const int c_end = blockIdx.y * nch + ((wv + 1) * nch) / 4;
  const int nct = rpad / 16;
  f64x4_t acc[PX_NCT];
#pragma unroll
  for (int c = 0; c < PX_NCT; ++c) acc[c] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  // one chunk's raw loads; the next chunk's are in flight during this one's MFMAs
  struct Raw {
    typename XVec<T>::V x[8 / XV];
    float4 g[2];
    float4 w[PX_NCT][2];
  };
  auto fetch_x = [&](int kc, Raw& r) {
    const int k0 = kc * PX_KC;
#pragma unroll
    for (int h = 0; h < 8 / XV; ++h) r.x[h] = *reinterpret_cast<const typename XVec<T>::V*>(xrow + k0 + h * XV);
  };
  auto fetch_gw = [&](int kc, Raw& r) {
    const int k0 = kc * PX_KC;
    r.g[0] = *reinterpret_cast<const float4*>(g1 + k0 + 8 * q);
    r.g[1] = *reinterpret_cast<const float4*>(g1 + k0 + 8 * q + 4);
#pragma unroll
    for (int c = 0; c < PX_NCT; ++c) {
      const float* wsrc = wp + (((size_t)kc * nct + cg * PX_NCT + c) * 64 + lane) * 8;
      r.w[c][0] = *reinterpret_cast<const float4*>(wsrc);
      r.w[c][1] = *reinterpret_cast<const float4*>(wsrc + 4);
    }
  };
  auto mma = [&](const Raw& r) {
    double a[8];
#pragma unroll
    for (int h = 0; h < 8 / XV; ++h) XVec<T>::unpack(r.x[h], a + h * XV);
    const float g[8] = {r.g[0].x, r.g[0].y, r.g[0].z, r.g[0].w, r.g[1].x, r.g[1].y, r.g[1].z, r.g[1].w};
#pragma unroll
    for (int t = 0; t < 8; ++t) a[t] = valid ? a[t] * (double)g[t] : 0.0;
#pragma unroll
    for (int c = 0; c < PX_NCT; ++c) {
      const double w[8] = {r.w[c][0].x, r.w[c][0].y, r.w[c][0].z, r.w[c][0].w,
                           r.w[c][1].x, r.w[c][1].y, r.w[c][1].z, r.w[c][1].w};
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[t], w[t], acc[c], 0, 0, 0);
    }
  };
  auto fetch = [&](int kc, Raw& r) {
    fetch_x(kc, r);
    fetch_gw(kc, r);
  };
  Raw ra, rb;
  if (c_beg < c_end) fetch_gw(c_beg, ra);
  {
    int b, li;
    if (m < M && row_resolve(idx, n, B, L, m, n0, i0, b, li)) {
      valid = true;
      xrow = H + ((size_t)b * L + li) * d + 8 * q;
    }
  }
  if (c_beg < c_end) {
    fetch_x(c_beg, ra);
    for (int c = c_beg; c < c_end; c += 2) {
      fetch(min(c + 1, c_end - 1), rb);
      mma(ra);
      if (c + 1 >= c_end) break;
      fetch(min(c + 2, c_end - 1), ra);
      mma(rb);
    }
  }
  // sum the four waves' K ranges in a fixed order
  if (wv > 0) {
#pragma unroll
    for (int c = 0; c < PX_NCT; ++c) red[wv - 1][c][lane] = acc[c];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int c = 0; c < PX_NCT; ++c) {
#pragma unroll
    for (int w2 = 0; w2 < 3; ++w2) acc[c] += red[w2][c][lane];
    // D register e of lane l holds row l / 16 + 4 e, column l % 16
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mr = rt * 16 + q + 4 * e;
      if (mr < M) partial[((size_t)blockIdx.y * M + mr) * rpad + (cg * PX_NCT + c) * 16 + i] = acc[c][e];
    }
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
  const int m = blockIdx.x;
  const int M = total_rows(n, B, cap);
  if (m >= M) return;
  // the split partials (addressed by the compact row m alone) and the row's
  // sequence-0 list entry are loaded before the row is resolved
  const int n0 = n[0];
  const int i0 = idx[m < L ? m : L - 1];
  const int tid = threadIdx.x, j = tid % RPAD, sg = tid / RPAD;
  const int per = (S + SG - 1) / SG, s0 = sg * per;
  // unconditional loads (the split index clamped), so they are issued
  // together; the sum below takes only the group's own splits
  double t[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int s = min(s0 + q, S - 1);
    t[q] = partial[((size_t)s * M + m) * RPAD + j];
  }
  int b, i;
  if (!row_resolve(idx, n, B, L, m, n0, i0, b, i)) return;
  const size_t row = (size_t)b * L + i;
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
  const int tasks = ((max_rows + 15) / 16) * (rpad / 16 / PX_NCT);
  dim3 grid(tasks, S);
  if (bf16m)
    hipLaunchKernelGGL(proxy_partial_kernel<bf16>, grid, dim3(256), 0, st, B, L, d, rpad, kps, max_rows, idx, n,
                       (const bf16*)H, g1, wr, partial);
  else
    hipLaunchKernelGGL(proxy_partial_kernel<float>, grid, dim3(256), 0, st, B, L, d, rpad, kps, max_rows, idx, n,
                       (const float*)H, g1, wr, partial);
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

// Packed basis: fp32, element (kc, ct, lane l = i + 16 q, t) = W_r[32 kc + 8 q + t][16 ct + i],
// zero for columns >= r.
__global__ void pack_proxy_kernel(int d, int r, int rpad, const float* __restrict__ wr, float* __restrict__ out) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (size_t)d * rpad) return;
  const int t = (int)(e & 7), lane = (int)((e >> 3) & 63);
  const size_t f = e >> 9;  // (kc, ct)
  const int nct = rpad / 16;
  const int ct = (int)(f % nct), kc = (int)(f / nct);
  const int k = kc * 32 + 8 * (lane >> 4) + t, j = ct * 16 + (lane & 15);
  out[e] = j < r ? wr[(size_t)k * r + j] : 0.0f;
}

hipError_t launch_pad_proxy(hipStream_t st, int d, int r, const float* wr, float* out) {
  if (d % 32) return hipErrorInvalidValue;
  const int rpad = proxy_rpad(r);
  const size_t total = (size_t)d * rpad;
  hipLaunchKernelGGL(pack_proxy_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, d, r, rpad, wr,
                     out);
  return hipGetLastError();
}

}  // namespace dllm
