// Proxy basis in the library (SPA-Cache, method step 1: the top-r singular
// vectors and values of the value projection, W_r = U_r S_r).  Init-time
// only.  Randomised subspace iteration in fp64 on the device:
//
//   Q <- orth(random d x p), p = r + oversampling
//   repeat iters times:  Q <- orth(W (W^T Q))
//   Rayleigh-Ritz:       Z = W^T Q,  T = Z^T Z = V diag(lambda) V^T (Jacobi)
//   W_r = Q V_r diag(sqrt(lambda_r))   (the r largest eigenvalues)
//
// orth() is CholeskyQR2: G = Y^T Y, G = L L^T, Y <- Y L^-T, twice.  The
// products are v_mfma_f64_16x16x4_f64 tiles; the small factorisations run in
// one workgroup.  W is read in its storage type and widened exactly.
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace dllm {

typedef double f64x4_b __attribute__((ext_vector_type(4)));

constexpr int BS_PMAX = 136;  // p <= 136: a p x p fp64 matrix fits in LDS

template <typename T> __device__ __forceinline__ double bs_ld(const T* p);
template <> __device__ __forceinline__ double bs_ld<double>(const double* p) { return *p; }
template <> __device__ __forceinline__ double bs_ld<float>(const float* p) { return (double)*p; }
template <> __device__ __forceinline__ double bs_ld<bf16>(const bf16* p) { return (double)bf2f(*p); }

// C[M][N] (ldc) = op(A)[M][K] B[K][N] (ldb), fp64 accumulation.  op(A)[i][k] is
// A[i*lda + k], or A[k*lda + i] when TA.  One wave per 16 x 16 tile of C;
// lane l feeds A row l%16 and B column l%16 with k-slot l/16 of each
// 4-k step; elements outside the matrices are zero.
template <typename T, bool TA>
__global__ __launch_bounds__(256) void bs_gemm_kernel(int M, int N, int K, const T* __restrict__ A, int lda,
                                                      const double* __restrict__ B, int ldb, double* __restrict__ C,
                                                      int ldc) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tiles_m = (M + 15) / 16;
  const int tile = blockIdx.x * 4 + wv;
  if (tile >= tiles_m * ((N + 15) / 16)) return;
  const int i0 = (tile % tiles_m) * 16, j0 = (tile / tiles_m) * 16;
  const int r = lane & 15, kq = lane >> 4;
  const int i = i0 + r, j = j0 + r;
  f64x4_b acc = {0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < K; k0 += 16) {
    double a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + 4 * u + kq;
      const bool kin = k < K;
      a[u] = (kin && i < M) ? bs_ld<T>(TA ? A + (size_t)k * lda + i : A + (size_t)i * lda + k) : 0.0;
      b[u] = (kin && j < N) ? B[(size_t)k * ldb + j] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[u], b[u], acc, 0, 0, 0);
  }
  // D register e of lane l: row l/16 + 4e, column l%16
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int ii = i0 + kq + 4 * e;
    if (ii < M && j < N) C[(size_t)ii * ldc + j] = acc[e];
  }
}

// Cholesky G = L L^T of a p x p SPD matrix (one workgroup), lower factor to L
// (upper part zero).  status[0] = 1 when a pivot is not positive.
__global__ __launch_bounds__(256) void bs_chol_kernel(int p, const double* __restrict__ G, double* __restrict__ Lout,
                                                      int32_t* __restrict__ status) {
  extern __shared__ double Ls[];  // [p][p]
  const int tid = threadIdx.x;
  for (int e = tid; e < p * p; e += 256) Ls[e] = G[e];
  __syncthreads();
  for (int j = 0; j < p; ++j) {
    if (tid == 0) {
      double s = Ls[j * p + j];
      for (int k = 0; k < j; ++k) s -= Ls[j * p + k] * Ls[j * p + k];
      if (!(s > 0.0)) {
        status[0] = 1;
        s = 1e-300;
      }
      Ls[j * p + j] = sqrt(s);
    }
    __syncthreads();
    const double djj = Ls[j * p + j];
    for (int i = j + 1 + tid; i < p; i += 256) {
      double s = Ls[i * p + j];
      for (int k = 0; k < j; ++k) s -= Ls[i * p + k] * Ls[j * p + k];
      Ls[i * p + j] = s / djj;
    }
    __syncthreads();
  }
  for (int e = tid; e < p * p; e += 256) {
    const int i = e / p, k = e - i * p;
    Lout[e] = k <= i ? Ls[e] : 0.0;
  }
}

// Y[i][:] <- Y[i][:] L^-T (each row solves y L^T = y_old by forward
// substitution), one thread per row.
__global__ __launch_bounds__(256) void bs_trsm_kernel(int rows, int p, const double* __restrict__ L,
                                                      double* __restrict__ Y) {
  extern __shared__ double Ls[];  // [p][p]
  for (int e = threadIdx.x; e < p * p; e += 256) Ls[e] = L[e];
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  double* y = Y + (size_t)i * p;
  for (int j = 0; j < p; ++j) {
    double s = y[j];
    for (int k = 0; k < j; ++k) s -= y[k] * Ls[j * p + k];
    y[j] = s / Ls[j * p + j];
  }
}

// Random start: uniform values in [-1, 1) from a 64-bit mix of (i, j).
__global__ void bs_init_kernel(int rows, int p, uint64_t seed, double* __restrict__ Q, int32_t* __restrict__ status) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e == 0) status[0] = 0;  // the factorisations only ever set it
  if (e >= (size_t)rows * p) return;
  uint64_t z = seed + 0x9E3779B97F4A7C15ull * (e + 1);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  Q[e] = (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

// Symmetric eigen-decomposition T = V diag(lambda) V^T of a p x p matrix by
// cyclic Jacobi in parallel (round-robin) order: in each round the p/2 (p
// even) disjoint pairs are rotated together (columns, then rows), `sweeps`
// sweeps of p - 1 rounds.  T is held in LDS; V (p x p) in global memory.
// lambda[j] = the diagonal at the end.
__global__ __launch_bounds__(256) void bs_jacobi_kernel(int p, int sweeps, const double* __restrict__ Tin,
                                                        double* __restrict__ V, double* __restrict__ lambda) {
  extern __shared__ double sm[];
  double* T = sm;                    // [p][p]
  double* cs = T + (size_t)p * p;    // [p/2][2] rotation (c, s) per pair
  int* pr = (int*)(cs + p);          // [p] pair members of this round: (pr[2k], pr[2k+1])
  const int tid = threadIdx.x;
  for (int e = tid; e < p * p; e += 256) {
    T[e] = Tin[e];
    const int i = e / p, k = e - i * p;
    V[e] = i == k ? 1.0 : 0.0;
  }
  const int h = p / 2;
  __syncthreads();
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int rd = 0; rd < p - 1; ++rd) {
      // round-robin tournament: player p-1 fixed, the others rotate
      if (tid < h) {
        const int a = tid == 0 ? p - 1 : (rd + tid) % (p - 1);
        const int b = (rd + p - 1 - tid) % (p - 1);
        const int lo = a < b ? a : b, hi = a < b ? b : a;
        pr[2 * tid] = lo;
        pr[2 * tid + 1] = hi;
        const double app = T[lo * p + lo], aqq = T[hi * p + hi], apq = T[lo * p + hi];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double th = (aqq - app) / (2.0 * apq);
          const double t = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(1.0 + th * th));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        cs[2 * tid] = c;
        cs[2 * tid + 1] = s;
      }
      __syncthreads();
      // columns: T <- T J, V <- V J
      for (int e = tid; e < h * p; e += 256) {
        const int k = e / p, i = e - k * p;
        const int a = pr[2 * k], b = pr[2 * k + 1];
        const double c = cs[2 * k], s = cs[2 * k + 1];
        const double ta = T[i * p + a], tb = T[i * p + b];
        T[i * p + a] = c * ta - s * tb;
        T[i * p + b] = s * ta + c * tb;
        const double va = V[(size_t)i * p + a], vb = V[(size_t)i * p + b];
        V[(size_t)i * p + a] = c * va - s * vb;
        V[(size_t)i * p + b] = s * va + c * vb;
      }
      __syncthreads();
      // rows: T <- J^T T
      for (int e = tid; e < h * p; e += 256) {
        const int k = e / p, i = e - k * p;
        const int a = pr[2 * k], b = pr[2 * k + 1];
        const double c = cs[2 * k], s = cs[2 * k + 1];
        const double ta = T[a * p + i], tb = T[b * p + i];
        T[a * p + i] = c * ta - s * tb;
        T[b * p + i] = s * ta + c * tb;
      }
      __syncthreads();
    }
  }
  for (int j = tid; j < p; j += 256) lambda[j] = T[j * p + j];
}

// B[k][c] = V[k][sel[c]] * sqrt(lambda[sel[c]]) for the r largest eigenvalues
// (descending; lowest index on ties), one workgroup.
__global__ __launch_bounds__(256) void bs_pick_kernel(int p, int r, const double* __restrict__ V,
                                                      const double* __restrict__ lambda, double* __restrict__ Bsel) {
  __shared__ int sel[BS_PMAX];
  const int tid = threadIdx.x;
  if (tid < p) {
    const double v = lambda[tid];
    int rank = 0;
    for (int j = 0; j < p; ++j) rank += (lambda[j] > v) || (lambda[j] == v && j < tid);
    if (rank < r) sel[rank] = tid;
  }
  __syncthreads();
  for (int e = tid; e < p * r; e += 256) {
    const int k = e / r, c = e - k * r;
    const int j = sel[c];
    Bsel[e] = V[(size_t)k * p + j] * sqrt(fmax(lambda[j], 0.0));
  }
}

__global__ void bs_to_f32_kernel(size_t n, const double* __restrict__ src, float* __restrict__ dst) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) dst[e] = (float)src[e];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <typename T, bool TA>
static hipError_t gemm64(hipStream_t st, int M, int N, int K, const T* A, int lda, const double* B, int ldb,
                         double* C, int ldc) {
  const int tiles = ((M + 15) / 16) * ((N + 15) / 16);
  hipLaunchKernelGGL((bs_gemm_kernel<T, TA>), dim3((tiles + 3) / 4), dim3(256), 0, st, M, N, K, A, lda, B, ldb, C,
                     ldc);
  return hipGetLastError();
}

static hipError_t set_lds(const void* f, size_t bytes) {
  return hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Y (rows x p) <- orth(Y) by CholeskyQR2; G, L: p x p scratch.
static hipError_t cholqr2(hipStream_t st, int rows, int p, double* Y, double* G, double* L, int32_t* status) {
  const size_t lds = (size_t)p * p * 8;
  for (int pass = 0; pass < 2; ++pass) {
    hipError_t e = gemm64<double, true>(st, p, p, rows, Y, p, Y, p, G, p);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bs_chol_kernel, dim3(1), dim3(256), lds, st, p, G, L, status);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bs_trsm_kernel, dim3((rows + 255) / 256), dim3(256), lds, st, rows, p, L, Y);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

int proxy_basis_width(int d, int nv, int r) {
  int p = r + 8;
  p = p < d ? p : d;
  p = p < nv ? p : nv;
  p = p < BS_PMAX ? p : BS_PMAX;
  return p & ~1;  // even, for the pairwise Jacobi rounds
}

size_t proxy_basis_workspace_doubles(int d, int nv, int r) {
  const int p = proxy_basis_width(d, nv, r);
  return (size_t)d * p * 2 + (size_t)nv * p + (size_t)p * p * 4 + (size_t)p + (size_t)p * r + 16;
}

template <typename T>
static hipError_t run_basis(hipStream_t st, int d, int nv, int r, int iters, const T* W, double* wr, double* ws,
                            int32_t* status) {
  const int p = proxy_basis_width(d, nv, r);
  double* Q = ws;
  double* Y = Q + (size_t)d * p;
  double* Z = Y + (size_t)d * p;
  double* G = Z + (size_t)nv * p;
  double* L = G + (size_t)p * p;
  double* Tm = L + (size_t)p * p;
  double* V = Tm + (size_t)p * p;
  double* lam = V + (size_t)p * p;
  double* Bs = lam + p;
  hipError_t e;
  static std::atomic<unsigned long long> attr{0};
  e = once_per_device(attr, [] {
    const size_t mx = (size_t)BS_PMAX * BS_PMAX * 8;
    hipError_t r;
    if ((r = set_lds((const void*)bs_chol_kernel, mx)) != hipSuccess) return r;
    if ((r = set_lds((const void*)bs_trsm_kernel, mx)) != hipSuccess) return r;
    return set_lds((const void*)bs_jacobi_kernel, mx + BS_PMAX * 8 + BS_PMAX * 4);
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bs_init_kernel, dim3((unsigned)(((size_t)d * p + 255) / 256)), dim3(256), 0, st, d, p,
                     (uint64_t)0x5EED5EEDull, Q, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = cholqr2(st, d, p, Q, G, L, status)) != hipSuccess) return e;
  for (int it = 0; it < iters; ++it) {
    if ((e = gemm64<T, true>(st, nv, p, d, W, nv, Q, p, Z, p)) != hipSuccess) return e;   // Z = W^T Q
    if ((e = gemm64<T, false>(st, d, p, nv, W, nv, Z, p, Q, p)) != hipSuccess) return e;  // Q = W Z
    if ((e = cholqr2(st, d, p, Q, G, L, status)) != hipSuccess) return e;
  }
  // Rayleigh-Ritz
  if ((e = gemm64<T, true>(st, nv, p, d, W, nv, Q, p, Z, p)) != hipSuccess) return e;        // Z = W^T Q
  if ((e = gemm64<double, true>(st, p, p, nv, Z, p, Z, p, Tm, p)) != hipSuccess) return e;   // T = Z^T Z
  const size_t jl = (size_t)p * p * 8 + (size_t)p * 8 + (size_t)p * 4;
  hipLaunchKernelGGL(bs_jacobi_kernel, dim3(1), dim3(256), jl, st, p, 14, Tm, V, lam);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bs_pick_kernel, dim3(1), dim3(256), 0, st, p, r, V, lam, Bs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return gemm64<double, false>(st, d, r, p, Q, p, Bs, r, wr, r);  // W_r = Q Bsel
}

// Fixed workspace of the allocation-free derivation: a file-scope device
// array (one copy per device, held until the process ends) of
// PROXY_BASIS_STATIC_DOUBLES workspace doubles followed by the status word.
// Host code never passes the array's name to a kernel: its device address,
// looked up once per device, is kept in g_static_ws.
static __device__ __align__(256) double scratch[PROXY_BASIS_STATIC_DOUBLES + 32];
static std::mutex g_static_mu;
static double* g_static_ws[64] = {};

hipError_t proxy_basis_static_setup(int dev) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (g_static_ws[dev]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != dev) return hipErrorInvalidDevice;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_static_ws[dev] = (double*)ptr;
  return hipSuccess;
}

double* proxy_basis_static_ws(int dev) {
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_static_mu);
  return g_static_ws[dev];
}

hipError_t launch_f64_to_f32(hipStream_t st, size_t n, const double* src, float* dst) {
  hipLaunchKernelGGL(bs_to_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, src, dst);
  return hipGetLastError();
}

hipError_t launch_proxy_basis(hipStream_t st, bool bf16m, int d, int nv, int r, int iters, const void* W, double* wr,
                              double* ws, int32_t* status) {
  if (r < 1 || r > 128 || r > d || r > nv || iters < 0) return hipErrorInvalidValue;
  if (proxy_basis_width(d, nv, r) < r) return hipErrorInvalidValue;
  if (bf16m) return run_basis<bf16>(st, d, nv, r, iters, (const bf16*)W, wr, ws, status);
  return run_basis<float>(st, d, nv, r, iters, (const float*)W, wr, ws, status);
}

}  // namespace dllm
