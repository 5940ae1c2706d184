// Dense contractions of the sparse layer on the gathered rows: out = A W with
// A [M][K] (the M selected rows, compact) and W [K][N] the layer weight.
//
// bf16: v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The sparse step's M
// (tens to a few hundred rows) is far below the machine balance, so the
// weights are streamed from HBM exactly once: a workgroup owns a 128-column
// slab (4 waves x 32 columns) and every row of a row block, the activation
// chunk is staged in LDS (double buffered) and shared by the 4 waves, and the
// next chunk's weight fragments are loaded while the current one is
// multiplied.  Weights are pre-packed into MFMA B-fragment order so that
// every lane issues one 16-byte load per fragment and a wave's column tile is
// one contiguous stream.  Split-K partials [S][M][N] are summed in a fixed
// order by the epilogue kernels.  Workgroups sharing an A range are placed on
// the same XCD (workgroup i runs on XCD i % 8).
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Packing.  Fragment (nt, kt) of W [K][N] holds, for lane l and j < 8,
// W[kt*16 + 8*(l/32) + j][nt*32 + l%32]; fragments are stored nt-major.
// Source column tile t (32 columns) of a Nsrc-wide source goes to packed
// column col0 + t*tile_stride.
// ---------------------------------------------------------------------------
__global__ void pack_bf16_kernel(int K, int Nsrc, const uint16_t* __restrict__ src, int ld_src,
                                 uint16_t* __restrict__ dst, int col0, int tile_stride) {
  const int KT = K >> 4;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // (t, kt, lane)
  const size_t total = (size_t)(Nsrc >> 5) * KT * 64;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const size_t f = gid >> 6;
  const int kt = (int)(f % KT);
  const int t = (int)(f / KT);
  const int scol = t * 32 + (lane & 31);
  const int dcol = col0 + t * tile_stride + (lane & 31);
  const int nt = dcol >> 5;
  uint16_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = src[(size_t)(kt * 16 + 8 * (lane >> 5) + j) * ld_src + scol];
  uint4 w;
  w.x = v[0] | ((uint32_t)v[1] << 16);
  w.y = v[2] | ((uint32_t)v[3] << 16);
  w.z = v[4] | ((uint32_t)v[5] << 16);
  w.w = v[6] | ((uint32_t)v[7] << 16);
  reinterpret_cast<uint4*>(dst)[((size_t)nt * KT + kt) * 64 + lane] = w;
}

hipError_t launch_pack_bf16(hipStream_t st, int K, int Nsrc, const uint16_t* src, int ld_src, uint16_t* dst,
                            int col0, int tile_stride) {
  const size_t total = (size_t)(Nsrc >> 5) * (K >> 4) * 64;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, K, Nsrc, src,
                     ld_src, dst, col0, tile_stride);
  return hipGetLastError();
}

// fp32: row-major [K][Ndst], same column placement.
__global__ void pack_f32_kernel(int K, int Nsrc, const float* __restrict__ src, int ld_src, float* __restrict__ dst,
                                int Ndst, int col0, int tile_stride) {
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (size_t)K * Nsrc) return;
  const int k = (int)(gid / Nsrc), c = (int)(gid % Nsrc);
  const int dcol = col0 + (c >> 5) * tile_stride + (c & 31);
  dst[(size_t)k * Ndst + dcol] = src[(size_t)k * ld_src + c];
}

hipError_t launch_pack_f32(hipStream_t st, int K, int Nsrc, const float* src, int ld_src, float* dst, int Ndst,
                           int col0, int tile_stride) {
  const size_t total = (size_t)K * Nsrc;
  hipLaunchKernelGGL(pack_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, K, Nsrc, src,
                     ld_src, dst, Ndst, col0, tile_stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM.
// ---------------------------------------------------------------------------
template <int MT, int KS>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ Wp,
                                                           float* __restrict__ out,
                                                           const int32_t* __restrict__ n_sel, int B, int K, int N,
                                                           int kps, int row_blocks, int n_slabs, int total, int cap) {
  extern __shared__ u32x4 lds[];
  constexpr int BUF = MT * KS * 64;           // 16-byte entries per buffer
  constexpr int PPT = (MT * KS * 64) / 256;   // A pieces per thread
  const int G = gridDim.x;
  const int w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  if (w >= total) return;
  const int slab = w % n_slabs;
  const int t2 = w / n_slabs;
  const int rb = t2 % row_blocks;
  const int split = t2 / row_blocks;
  const int M = total_rows(n_sel, B, cap);
  const int r0 = rb * 32 * MT;
  if (r0 >= M) return;
  const int mt_n = min(MT, (M - r0 + 31) >> 5);
  const int rows_n = mt_n * 32;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int nt = slab * 4 + wv;
  const bool wvalid = nt < (N >> 5);
  const int k0 = split * kps;
  const int nchunks = kps / (16 * KS);
  const int KT = K >> 4;
  const u32x4* wbase = reinterpret_cast<const u32x4*>(Wp) + ((size_t)(wvalid ? nt : 0) * KT + (k0 >> 4)) * 64 + lane;

  f32x16_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;

  u32x4 wcur[KS], wnext[KS];
  u32x4 areg[PPT];

  auto load_w = [&](int c, u32x4* dst) {
    if (wvalid) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[ks] = __builtin_nontemporal_load(wbase + (size_t)(c * KS + ks) * 64);
    }
  };
  auto load_a = [&](int c) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int piece = tid + p * 256;
      const int row = piece / (2 * KS), kp = piece % (2 * KS);
      if (row < rows_n)
        areg[p] = *reinterpret_cast<const u32x4*>(A + (size_t)(r0 + row) * K + k0 + c * 16 * KS + kp * 8);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PPT; ++p) {
      const int piece = tid + p * 256;
      const int row = piece / (2 * KS), kp = piece % (2 * KS);
      if (row < rows_n) {
        const int mt = row >> 5, rr = row & 31, ks = kp >> 1, hf = kp & 1;
        lds[buf * BUF + (mt * KS + ks) * 64 + rr + 32 * hf] = areg[p];
      }
    }
  };

  load_w(0, wcur);
  load_a(0);
  store_a(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_w(c + 1, wnext);
      load_a(c + 1);
    }
    if (wvalid) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, wcur[ks]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mt_n) {
            const bf16x8_t aa = __builtin_bit_cast(bf16x8_t, lds[buf * BUF + (mt * KS + ks) * 64 + lane]);
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, bb, acc[mt], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_a(buf ^ 1);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wcur[ks] = wnext[ks];
  }
  if (!wvalid) return;
  const int ncol = nt * 32 + (lane & 31);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < mt_n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = r0 + mt * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (m < M) out[((size_t)split * M + m) * N + ncol] = acc[mt][i];
      }
    }
  }
}

constexpr int GEMM_KS = 4;

template <int MT>
static hipError_t launch_mt(hipStream_t st, int grid, const uint16_t* A, const uint16_t* Wp, float* out,
                            const int32_t* n_sel, int B, int K, int N, int kps, int row_blocks, int n_slabs,
                            int total, int cap) {
  static bool attr_set = false;
  const size_t lds = (size_t)2 * MT * GEMM_KS * 64 * 16;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<MT, GEMM_KS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<MT, GEMM_KS>), dim3(grid), dim3(256), lds, st, A, Wp, out, n_sel, B, K, N,
                     kps, row_blocks, n_slabs, total, cap);
  return hipGetLastError();
}

static int mt_for_rows(int max_rows) {
  const int t = (max_rows + 31) / 32;
  if (t <= 1) return 1;
  if (t <= 2) return 2;
  if (t <= 4) return 4;
  if (t <= 6) return 6;
  if (t <= 8) return 8;
  if (t <= 10) return 10;
  return 8;  // row-blocked
}

int gemm_bf16_pick_splits(int max_rows, int K, int N, int n_cu) {
  const int MT = mt_for_rows(max_rows);
  const int row_blocks = (max_rows + 32 * MT - 1) / (32 * MT);
  const int n_slabs = (N + 127) / 128;
  const int base = n_slabs * row_blocks;
  const double wbytes = (double)K * N * 2.0 * row_blocks;
  double best = 1e300;
  int best_s = 1;
  for (int s = 1; s <= 64; s *= 2) {
    if (K % (s * 16 * GEMM_KS) != 0) break;
    const int waves = (base * s + n_cu - 1) / n_cu;
    const double eff = (double)base * s / ((double)waves * n_cu);
    const double cost = wbytes / eff + 0.5 * 2.0 * 4.0 * s * (double)max_rows * N;
    if (cost < best * 0.999) {
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

hipError_t launch_gemm_bf16(hipStream_t st, int max_rows, int B, int K, int N, const uint16_t* A,
                            const uint16_t* Wp, const int32_t* n_sel, float* out, int splits) {
  if (max_rows <= 0) return hipSuccess;
  const int MT = mt_for_rows(max_rows);
  const int row_blocks = (max_rows + 32 * MT - 1) / (32 * MT);
  const int n_slabs = (N + 127) / 128;
  const int kps = K / splits;
  if (kps * splits != K || kps % (16 * GEMM_KS) != 0) return hipErrorInvalidValue;
  const int total = n_slabs * row_blocks * splits;
  const int grid = (total + 7) / 8 * 8;
  switch (MT) {
    case 1: return launch_mt<1>(st, grid, A, Wp, out, n_sel, B, K, N, kps, row_blocks, n_slabs, total, max_rows);
    case 2: return launch_mt<2>(st, grid, A, Wp, out, n_sel, B, K, N, kps, row_blocks, n_slabs, total, max_rows);
    case 4: return launch_mt<4>(st, grid, A, Wp, out, n_sel, B, K, N, kps, row_blocks, n_slabs, total, max_rows);
    case 6: return launch_mt<6>(st, grid, A, Wp, out, n_sel, B, K, N, kps, row_blocks, n_slabs, total, max_rows);
    case 8: return launch_mt<8>(st, grid, A, Wp, out, n_sel, B, K, N, kps, row_blocks, n_slabs, total, max_rows);
    default: return launch_mt<10>(st, grid, A, Wp, out, n_sel, B, K, N, kps, row_blocks, n_slabs, total, max_rows);
  }
}

// ---------------------------------------------------------------------------
// fp32 GEMM (fp32 models): 64x64 tiles, 4x4 outputs per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                       const int32_t* __restrict__ n_sel, int B, int K, int N,
                                                       int cap, float* __restrict__ out) {
  __shared__ float As[16][64 + 4];
  __shared__ float Ws[16][64 + 4];
  const int M = total_rows(n_sel, B, cap);
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  if (m0 >= M) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int kk = e & 15, mm = e >> 4;
      As[kk][mm] = (m0 + mm < M && k0 + kk < K) ? A[(size_t)(m0 + mm) * K + k0 + kk] : 0.f;
      const int kk2 = e >> 6, nn = e & 63;
      Ws[kk2][nn] = (n0 + nn < N && k0 + kk2 < K) ? W[(size_t)(k0 + kk2) * N + n0 + nn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = Ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nn = n0 + tx * 4 + j;
      if (nn < N) out[(size_t)m * N + nn] = acc[i][j];
    }
  }
}

hipError_t launch_gemm_f32(hipStream_t st, int max_rows, int B, int K, int N, const float* A, const float* W,
                           const int32_t* n_sel, float* out) {
  if (max_rows <= 0) return hipSuccess;
  dim3 grid((N + 63) / 64, (max_rows + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, A, W, n_sel, B, K, N, max_rows, out);
  return hipGetLastError();
}

}  // namespace dllm
