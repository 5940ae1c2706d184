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
// one contiguous stream.  Split-K partials [S][cap][N] (cap: the launch's row
// capacity, so that a row's partial addresses do not depend on the selected
// row count) are summed in a fixed order by the epilogue kernels.  Workgroups sharing an A range are placed on
// the same XCD (workgroup i runs on XCD i % 8).
#include <type_traits>

#include "common.h"
#include "kernels.h"

#include <hip/hip_ext.h>

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Packing.  Fragment (nt, kt) of W [K][N] holds, for lane l and j < 8,
// W[kt*16 + 8*(l/32) + j][nt*32 + l%32]; fragments are stored nt-major.
// Source column group t (gw = 32 or 16 columns) of a Nsrc-wide source goes to
// packed columns col0 + t*tile_stride .. + gw - 1 (inside one 32-column tile).
// ---------------------------------------------------------------------------
__global__ void pack_bf16_kernel(int K, int Nsrc, const uint16_t* __restrict__ src, int ld_src,
                                 uint16_t* __restrict__ dst, int col0, int tile_stride, int gw) {
  const int KT = K >> 4;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // (t, kt, lane)
  const size_t total = (size_t)(Nsrc / gw) * KT * 64;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const int c = lane & 31;
  if (c >= gw) return;
  const size_t f = gid >> 6;
  const int kt = (int)(f % KT);
  const int t = (int)(f / KT);
  const int scol = t * gw + c;
  const int dcol = col0 + t * tile_stride + c;
  const int nt = dcol >> 5;
  uint16_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = src[(size_t)(kt * 16 + 8 * (lane >> 5) + j) * ld_src + scol];
  uint4 w;
  w.x = v[0] | ((uint32_t)v[1] << 16);
  w.y = v[2] | ((uint32_t)v[3] << 16);
  w.z = v[4] | ((uint32_t)v[5] << 16);
  w.w = v[6] | ((uint32_t)v[7] << 16);
  reinterpret_cast<uint4*>(dst)[((size_t)nt * KT + kt) * 64 + (dcol & 31) + 32 * (lane >> 5)] = w;
}

hipError_t launch_pack_bf16(hipStream_t st, int K, int Nsrc, const uint16_t* src, int ld_src, uint16_t* dst,
                            int col0, int tile_stride, int gw) {
  if ((gw != 32 && gw != 16) || Nsrc % gw != 0 || (col0 & 31) + gw > 32) return hipErrorInvalidValue;
  const size_t total = (size_t)(Nsrc / gw) * (K >> 4) * 64;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, K, Nsrc, src,
                     ld_src, dst, col0, tile_stride, gw);
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
//
// Workgroup = 4 waves, a slab of COLS column tiles of 32 (128 or 96 columns)
// and a row block of 4*MTW row tiles; wave w owns row tiles w, w+4, ... of the
// block and all the slab's column tiles, so each A fragment it loads (straight
// from the packed activations, 16 B per lane) feeds COLS MFMAs.  The slab's
// weight fragments are loaded once per workgroup (wave w loads column tile w;
// with 3 columns wave 3 repeats wave 2's loads, which hit in L2, and its LDS
// slot is not read) and shared through a double-buffered LDS stage.  96-column
// slabs serve shapes whose 128-column workgroups leave much of the last round
// of the chip empty.  Both operands are prefetched two chunks ahead in
// registers, so the HBM weight stream overlaps the MFMAs of earlier chunks.
// EPI 0 writes fp32 split-K partials out[split][m][n] ([S][cap][N]); EPI 1 (one split)
// applies SwiGLU to the gate/up pairs inside each 32-column tile (16 gate then
// 16 up columns) and writes the packed bf16 activation of the next GEMM.
// ---------------------------------------------------------------------------
template <int MTW, int KS, int EPI, int COLS>
__global__ __launch_bounds__(256, (MTW * KS <= 4) ? 2 : 1) void gemm_bf16_kernel(const u32x4* __restrict__ Ap, int MTt,
                                                           const u32x4* __restrict__ Wp, float* __restrict__ out,
                                                           uint16_t* __restrict__ act, int MTt_out,
                                                           const int32_t* __restrict__ n_sel, int B, int K, int N,
                                                           int kps, int row_blocks, int n_slabs, int total, int cap) {
  extern __shared__ u32x4 wl[];  // [2][KS][4][64]
  constexpr int WBUF = KS * 4 * 64;
  const int G = gridDim.x;
  const int w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  if (w >= total) return;
  const int slab = w % n_slabs;
  const int t2 = w / n_slabs;
  const int rb = t2 % row_blocks;
  const int split = t2 / row_blocks;
  const int M = total_rows(n_sel, B, cap);
  const int mt_base = rb * 4 * MTW;
  if (mt_base * 32 >= M) return;
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int NT = N >> 5;
  const int nt0 = slab * COLS;
  const int KT = K >> 4;
  const int kt0 = (split * kps) >> 4;
  const int nchunks = kps / (16 * KS);
  const int m_tiles = (M + 31) >> 5;
  bool tv[MTW];
#pragma unroll
  for (int j = 0; j < MTW; ++j) tv[j] = mt_base + wv + 4 * j < m_tiles;
  // Every load below is unconditional so that the compiler's wait counts keep
  // the prefetched chunks in flight: invalid tiles are clamped to a valid one
  // and the (at most three) chunks read past the end of a range land in the
  // padding that every weight and activation buffer carries.
  const int ntw = min(nt0 + min(wv, COLS - 1), NT - 1);
  const u32x4* wsrc = Wp + ((size_t)ntw * KT + kt0) * 64 + lane;
  const u32x4* asrc[MTW];
#pragma unroll
  for (int j = 0; j < MTW; ++j)
    asrc[j] = Ap + (size_t)kt0 * MTt * 64 + (size_t)min(mt_base + wv + 4 * j, m_tiles - 1) * 64 + lane;
  const size_t astep = (size_t)KS * MTt * 64;  // one chunk of A, in 16-byte units

  f32x16_t acc[MTW][COLS];
#pragma unroll
  for (int j = 0; j < MTW; ++j)
#pragma unroll
    for (int nt = 0; nt < COLS; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][nt][i] = 0.f;

  u32x4 wA[KS], wB[KS];
  u32x4 aA[MTW][KS], aB[MTW][KS];

  auto load_w = [&](int c, u32x4* dst) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = __builtin_nontemporal_load(wsrc + (size_t)(c * KS + ks) * 64);
  };
  auto load_a = [&](int c, u32x4 (*dst)[KS]) {
#pragma unroll
    for (int j = 0; j < MTW; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) dst[j][ks] = asrc[j][(size_t)c * astep + (size_t)ks * MTt * 64];
  };
  auto store_w = [&](const u32x4* src, int buf) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) wl[buf * WBUF + (ks * 4 + wv) * 64 + lane] = src[ks];
  };
  // nv: std::integral_constant<int, v> = the wave's first v row tiles hold
  // rows and the rest none (no per-tile test in the loop), or -1: test each
  // tile
  auto compute = [&](int buf, u32x4 (*a)[KS], auto nv) {
    // all B fragments of the chunk first, so one LDS latency covers them all
    u32x4 b[KS][COLS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < COLS; ++nt) b[ks][nt] = wl[buf * WBUF + (ks * 4 + nt) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        if constexpr (decltype(nv)::value < 0) {
          if (!tv[j]) continue;  // a row tile past the rows (wave-uniform): no MFMAs
        } else if (j >= decltype(nv)::value) {
          continue;
        }
        const bf16x8_t aa = __builtin_bit_cast(bf16x8_t, a[j][ks]);
#pragma unroll
        for (int nt = 0; nt < COLS; ++nt)
          acc[j][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, __builtin_bit_cast(bf16x8_t, b[ks][nt]),
                                                               acc[j][nt], 0, 0, 0);
      }
  };

  // nchunks is even (the host guarantees it)
  load_w(0, wA);
  load_w(1, wB);
  load_a(0, aA);
  store_w(wA, 0);
  load_a(1, aB);
  load_w(2, wA);
  __syncthreads();
  auto main_loop = [&](auto nv) {
    for (int c = 0; c < nchunks; c += 2) {
      // A(c) in aA, W(c) in LDS 0, W(c+1) in wB, W(c+2) in wA
      compute(0, aA, nv);
      store_w(wB, 1);
      load_a(c + 2, aA);
      load_w(c + 3, wB);
      __syncthreads();
      // A(c+1) in aB, W(c+1) in LDS 1, W(c+2) in wA
      compute(1, aB, nv);
      store_w(wA, 0);
      load_a(c + 3, aB);
      load_w(c + 4, wA);
      __syncthreads();
    }
  };
  // 384-row blocks: one loop per count of row tiles that hold rows (the
  // tiles are in row order, so they are the first ones).  256-row blocks keep
  // one loop that tests each tile (a second copy measured slower there, 23.1
  // -> 23.6 ms per full-pass step, against 6 % faster GEMMs at 384).
  if constexpr (MTW == 3) {
    const int nvalid = (int)tv[0] + (int)tv[1] + (int)tv[2];
    if (nvalid == 3)
      main_loop(std::integral_constant<int, 3>{});
    else if (nvalid == 2)
      main_loop(std::integral_constant<int, 2>{});
    else if (nvalid == 1)
      main_loop(std::integral_constant<int, 1>{});
    else
      main_loop(std::integral_constant<int, 0>{});
  } else {
    main_loop(std::integral_constant<int, -1>{});
  }

  if constexpr (EPI == 0) {
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      if (!tv[j]) continue;
      const int mrow = (mt_base + wv + 4 * j) * 32 + (lane >> 5) * 4;
#pragma unroll
      for (int nt = 0; nt < COLS; ++nt) {
        if (nt0 + nt >= NT) continue;
        const int ncol = (nt0 + nt) * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = mrow + (i >> 2) * 8 + (i & 3);
          if (m < M) out[((size_t)split * cap + m) * N + ncol] = acc[j][nt][i];
        }
      }
    }
  } else {
    // each 32-column tile holds 16 gate columns (lanes l % 32 < 16) and the
    // matching 16 up columns (lane l + 16): intermediate column 16 T + l % 16
#pragma unroll
    for (int j = 0; j < MTW; ++j) {
      if (!tv[j]) continue;
      const int mrow = (mt_base + wv + 4 * j) * 32 + (lane >> 5) * 4;
#pragma unroll
      for (int nt = 0; nt < COLS; ++nt) {
        if (nt0 + nt >= NT) continue;
        const int f = (nt0 + nt) * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = mrow + (i >> 2) * 8 + (i & 3);
          const float g = acc[j][nt][i], u = __shfl_xor(acc[j][nt][i], 16, 64);
          if (!(lane & 16) && m < M) act[apack_off(m, f, MTt_out)] = f2bf(silu_fast(g) * u);
        }
      }
    }
  }
}

// Row tiles per wave: 384-row blocks (3) unless 256-row blocks (2, two
// workgroups per CU) leave fewer padded row tiles (measured: a 1024-row full
// pass -21 %, 2624 rows +8 % with 256-row blocks).
static int mtw_for_rows(int max_rows) {
  if (max_rows <= 128) return 1;
  if (max_rows <= 256) return 2;
  const int t = (max_rows + 31) / 32;
  const int b3 = (t + 11) / 12, b2 = (t + 7) / 8;
  return t * 12 * b3 > t * 8 * b2 ? 2 : 3;  // t/(8 b2) > t/(12 b3)
}
// k16 steps per chunk: 2 for 2 row tiles per wave (fewer registers: two
// waves per SIMD), else 4.
static int ks_for(int mtw) { return mtw == 2 ? 2 : 4; }

template <int MTW, int KS, int EPI, int COLS>
static hipError_t launch_cfg(hipStream_t st, int grid, const void* A, int MTt, const void* Wp, float* out,
                             uint16_t* act, int MTt_out, const int32_t* n_sel, int B, int K, int N, int kps,
                             int row_blocks, int n_slabs, int total, int cap, LaunchEvents ev) {
  static std::atomic<unsigned long long> attr_set{0};
  const size_t lds = (size_t)2 * KS * 4 * 64 * 16;
  hipError_t ea = once_per_device(attr_set, [&] {
    return hipFuncSetAttribute((const void*)gemm_bf16_kernel<MTW, KS, EPI, COLS>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (ea != hipSuccess) return ea;
  if (ev.start)
    hipExtLaunchKernelGGL((gemm_bf16_kernel<MTW, KS, EPI, COLS>), dim3(grid), dim3(256), lds, st, ev.start, ev.stop,
                          0, (const u32x4*)A, MTt, (const u32x4*)Wp, out, act, MTt_out, n_sel, B, K, N, kps,
                          row_blocks, n_slabs, total, cap);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<MTW, KS, EPI, COLS>), dim3(grid), dim3(256), lds, st, (const u32x4*)A, MTt,
                       (const u32x4*)Wp, out, act, MTt_out, n_sel, B, K, N, kps, row_blocks, n_slabs, total, cap);
  return hipGetLastError();
}

// Elements of padding every packed weight / activation buffer needs past its
// end: the pipeline reads up to three 64-wide k chunks beyond a range.
size_t gemm_pad_elems(int rows_tiles) { return (size_t)3 * 4 * (size_t)(rows_tiles > 0 ? rows_tiles : 1) * 512; }

// Relative cost of a 96-column slab per unit of work (each activation
// fragment feeds 3 MFMAs instead of 4), fitted to measurements: at 3 row
// tiles per wave, 11 rounds of 96-column workgroups ran 5 % slower than 9
// rounds of 128-column ones (2624 rows, 37888 columns), and one round of
// 96-column workgroups (256 of them) 7 % faster than 192 128-column ones
// (about 380 rows, 24576 and 12288 columns).  At 2 row tiles per wave two
// workgroups share a CU and fill the idle SIMDs of a partial round by
// themselves: there 96-column slabs were 9 % slower (1024 rows), so they
// are not used.
constexpr double BF16_COLS3_COST = 1.2;

// Cost of a (column tiles per workgroup, K splits) choice: the weight stream
// at the occupancy its rounds of workgroups achieve, plus the split partials'
// round trip; infinite where the split does not divide K in whole chunk pairs.
static double bf16_cost(int max_rows, int K, int N, int n_cu, int cols, int s) {
  const int mtw = mtw_for_rows(max_rows);
  const int ks = ks_for(mtw);
  if (K % (s * 32 * ks) != 0) return 1e300;  // an even number of chunks per split
  const int row_blocks = (max_rows + 128 * mtw - 1) / (128 * mtw);
  const int n_slabs = ((N >> 5) + cols - 1) / cols;
  const int base = n_slabs * row_blocks;
  const int slots = mtw * ks <= 4 ? 2 * n_cu : n_cu;  // workgroups resident at once (two when they fit)
  const int rounds = (base * s + slots - 1) / slots;
  const double eff = (double)base * s / ((double)rounds * slots);
  const double wbytes = (double)K * N * 2.0;
  return wbytes / eff * (cols == 3 ? BF16_COLS3_COST : 1.0) +
         (s > 1 ? 2.0 * 4.0 * s * (double)max_rows * N : 0.0);
}

int gemm_bf16_pick_splits(int max_rows, int K, int N, int n_cu) {
  double best = 1e300;
  int best_s = 1;
  for (int s = 1; s <= 32; s *= 2) {
    if (K % (s * 32 * ks_for(mtw_for_rows(max_rows))) != 0) break;
    const double c3 = mtw_for_rows(max_rows) != 3 ? 1e300 : bf16_cost(max_rows, K, N, n_cu, 3, s);
    const double cost = std::min(bf16_cost(max_rows, K, N, n_cu, 4, s), c3);
    if (cost < best * 0.999) {
      best = cost;
      best_s = s;
    }
  }
  return best_s;
}

int gemm_bf16_pick_cols(int max_rows, int K, int N, int n_cu, int splits) {
  if (mtw_for_rows(max_rows) != 3) return 4;  // 96-column slabs pay off at 3 row tiles per wave only
  return bf16_cost(max_rows, K, N, n_cu, 3, splits) < bf16_cost(max_rows, K, N, n_cu, 4, splits) ? 3 : 4;
}

hipError_t launch_gemm_bf16(hipStream_t st, int max_rows, int B, int K, int N, const uint16_t* A, int MTt,
                            const uint16_t* Wp, const int32_t* n_sel, float* out, int splits, uint16_t* act,
                            int MTt_out, int cols, LaunchEvents ev) {
  if (max_rows <= 0) return hipSuccess;
  if (cols != 3 && cols != 4) return hipErrorInvalidValue;
  const int mtw = mtw_for_rows(max_rows);
  const int ks = ks_for(mtw);
  const int row_blocks = (max_rows + 128 * mtw - 1) / (128 * mtw);
  const int n_slabs = ((N >> 5) + cols - 1) / cols;
  const int kps = K / splits;
  if (kps * splits != K || kps % (32 * ks) != 0) return hipErrorInvalidValue;
  if (act != nullptr && (splits != 1 || N % 64 != 0)) return hipErrorInvalidValue;
  const int total = n_slabs * row_blocks * splits;
  const int grid = (total + 7) / 8 * 8;
#define GL(MTW, KS, EPI, C)                                                                                   \
  launch_cfg<MTW, KS, EPI, C>(st, grid, A, MTt, Wp, out, act, MTt_out, n_sel, B, K, N, kps, row_blocks, n_slabs, \
                              total, max_rows, ev)
  if (cols == 3 && mtw != 3) return hipErrorInvalidValue;
  if (act == nullptr) {
    if (mtw == 1) return GL(1, 4, 0, 4);
    if (mtw == 2) return GL(2, 2, 0, 4);
    return cols == 3 ? GL(3, 4, 0, 3) : GL(3, 4, 0, 4);
  }
  if (mtw == 1) return GL(1, 4, 1, 4);
  if (mtw == 2) return GL(2, 2, 1, 4);
  return cols == 3 ? GL(3, 4, 1, 3) : GL(3, 4, 1, 4);
#undef GL
}

// ---------------------------------------------------------------------------
// Weight-streaming bf16 GEMM for up to 288 rows (9 row tiles).
//
// Workgroup = 4 waves and a 128-column slab (COLS = 4); wave w owns column
// tile w of the slab and every row tile.  COLS = 3 (96-column slabs, for up to
// three row tiles where N/128 slabs times the K splits leave CUs idle, e.g. a
// 12288-column QKV at two splits or a 24576-column fused gate|up: 192
// workgroups, against 256 with 96-column slabs): waves 0..2 own the three
// column tiles and wave 3 only shares the activation DMA, its waits and the
// barriers.  Each wave streams its own weight tile straight
// from HBM into a register ring of 16 k16 steps (no LDS on the weight path).
// The activation chunk (64 k, all row tiles) goes from global memory straight
// into LDS by DMA (global_load_lds_dwordx4: no registers, no ds_write), into a
// ring of NS chunk slots requested NS-1 chunks ahead, and is shared by the 4
// waves; the next step's activation fragments are read from LDS while the
// current step multiplies.
//
// The DMA is issued from inline asm so that the compiler does not make every
// later LDS read wait for it; its completion is waited for explicitly.  vmcnt
// retires in issue order, and the order of the memory operations inside a
// step is pinned by scheduling barriers, so the number of operations issued
// after the request of chunk c+1 is a compile-time constant (DMA_AFTER): a
// wait down to that count (minus a margin) followed by a workgroup barrier
// makes chunk c+1 visible to every wave before its first fragment is read.
// The compiler's own waits for the weight ring see only the weight loads, so
// they wait at least as long as needed.  EPI as above.
// ---------------------------------------------------------------------------
constexpr int GS_KC = 4;  // k16 steps per activation chunk
constexpr int GS_MAXMT = 9;

template <int MT>
struct StreamShape {
  static constexpr int NS = 4;  // activation ring slots (chunks)
  static constexpr int P = NS - 1;             // chunks requested ahead
  static constexpr int NW = 4;  // chunks per weight-ring turn (ring depth GS_KC * NW steps)
  // VMEM operations issued after the request of chunk c+1 (step 0 of chunk
  // c+1-P, before that step's weight refill) until the wait at the end of
  // step GS_KC-2 of chunk c: the rest of that chunk's refills, MT requests and
  // GS_KC refills for each chunk in between, MT requests and GS_KC-1 refills in
  // chunk c.
  static constexpr int DMA_AFTER = GS_KC + (P - 2) * (MT + GS_KC) + MT + (GS_KC - 1);
  static constexpr int WAIT = DMA_AFTER - 2;
  static constexpr size_t LDS = (size_t)NS * GS_KC * MT * 64 * 16;
  static_assert(WAIT >= 0 && WAIT < 64, "vmcnt field");
  static_assert(LDS <= 160 * 1024, "LDS");
};

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(n) lgkmcnt(0) (expcnt untouched)
#define GS_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14) | (7 << 4)))

// IDLE: wave 3 of a 96-column slab, which owns no column tile and only shares
// the activation DMA, its waits and the barriers
template <int MT, int EPI, int COLS, bool IDLE>
__device__ __forceinline__ void gemm_stream_body(const u32x4* __restrict__ Ap, int MTt, const u32x4* __restrict__ Wp,
                                                 float* __restrict__ out, uint16_t* __restrict__ act, int MTt_out,
                                                 const int32_t* __restrict__ n_sel, int B, int K, int N, int kps,
                                                 int n_slabs, int total, int cap) {
  static_assert(COLS == 4 || (COLS == 3 && EPI != 2), "96-column slabs: partials or SwiGLU");
  using S = StreamShape<MT>;
  constexpr int NS = S::NS, P = S::P;
  extern __shared__ u32x4 lds[];  // activation ring: [NS][GS_KC][MT][64]
  constexpr int ABUF = GS_KC * MT * 64;
  const int G = gridDim.x;
  const int w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  if (w >= total) return;
  const int slab = w % n_slabs, split = w / n_slabs;
  const int M = total_rows(n_sel, B, cap);
  if (M <= 0) return;
  const int m_tiles = (M + 31) >> 5;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NT = N >> 5, KT = K >> 4;
  const int nt = min(slab * COLS + wv, NT - 1);
  const int kt0 = (split * kps) >> 4;
  constexpr int GS_NW = S::NW;
  constexpr int GS_D = GS_KC * GS_NW;  // weight ring depth (k16 steps)
  const int nsteps = kps >> 4, nch = nsteps / GS_KC, nsup = nsteps / GS_D;

  const u32x4* wsrc = Wp + ((size_t)nt * KT + kt0) * 64 + lane;
  // chunk c: wave wv requests step wv of the chunk for every row tile (row
  // tiles past M repeat the last one; chunks past the range repeat the last).
  // Fragment base in scalar registers, lane byte offset in one VGPR; the DMA
  // writes lane l's 16 bytes at m0 + 16 l.  An M0 write needs one wait state
  // before an LDS DMA (the compiler's hazard pass does not look inside asm).
  const unsigned voff = (unsigned)lane * 16u;
  auto request_a = [&](int c) {
    const int cc = min(c, nch - 1);
    const int slot = c % NS;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is only ever set here
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4* g = Ap + ((size_t)(kt0 + wv + cc * GS_KC) * MTt + min(mt, m_tiles - 1)) * 64;
      const unsigned l = (unsigned)(uintptr_t)(lds_void_t*)&lds[slot * ABUF + (wv * MT + mt) * 64];
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(l)),
                   "v"(voff), "s"(uniform_ptr(g))
                   : "memory", "m0");
    }
#pragma clang diagnostic pop
  };
  auto read_af = [&](int c, int st, u32x4* dst) {
    const int slot = c % NS;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) dst[mt] = lds[slot * ABUF + (st * MT + mt) * 64 + lane];
  };

  // VMEM operations after the request of chunk c+1 until the wait: on an
  // idle wave only the requests of chunks c+2 .. c+P-1 ((P - 1) MT), less
  // the same margin of two
  constexpr int WAIT = IDLE ? (S::P - 1) * MT - 2 : S::WAIT;
  static_assert(WAIT >= 0 && WAIT < 64, "vmcnt field");
  f32x16_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;

#pragma unroll
  for (int c = 0; c < P; ++c) request_a(c);
  u32x4 wr[GS_D];  // slot j holds step s with s % GS_D == j
  if constexpr (!IDLE) {
#pragma unroll
    for (int j = 0; j < GS_D; ++j) wr[j] = __builtin_nontemporal_load(wsrc + (size_t)min(j, nsteps - 1) * 64);
  }
  GS_WAIT_VM_LGKM0(0);
  __builtin_amdgcn_s_barrier();
  u32x4 af[2][MT];
  if constexpr (!IDLE) read_af(0, 0, af[0]);
  for (int sc = 0; sc < nsup; ++sc) {
#pragma unroll
    for (int cc = 0; cc < GS_NW; ++cc) {
      const int c = sc * GS_NW + cc;
#pragma unroll
      for (int st = 0; st < GS_KC; ++st) {
        const int j = cc * GS_KC + st;
        const int s = c * GS_KC + st;
        if constexpr (!IDLE) {
          // the next step's activation fragments are read while this step multiplies
          if (st + 1 < GS_KC) read_af(c, st + 1, af[(j + 1) & 1]);
          else read_af(c + 1, 0, af[(j + 1) & 1]);
          const bf16x8_t b = __builtin_bit_cast(bf16x8_t, wr[j]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[j & 1][mt]), b,
                                                              acc[mt], 0, 0, 0);
          // one fragment read for the next step between consecutive MFMAs
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // slot (c+P) % NS held chunk c-1, which every wave finished reading
        // before the barrier of chunk c-1
        if (st == 0) request_a(c + P);
        __builtin_amdgcn_sched_barrier(0);
        // refill the slot only after its last use, so the new load can take
        // the same registers (no copy of an in-flight load at the back edge)
        if constexpr (!IDLE) wr[j] = __builtin_nontemporal_load(wsrc + (size_t)min(s + GS_D, nsteps - 1) * 64);
        __builtin_amdgcn_sched_barrier(0);
        if (st == GS_KC - 2) {
          // this wave's requests for chunk c+1 have landed and its reads of
          // chunk c are complete; after the barrier, for every wave
          GS_WAIT_VM_LGKM0(WAIT);
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  GS_WAIT_VM_LGKM0(0);  // no request may still be writing LDS

  if constexpr (!IDLE) {
    if constexpr (EPI == 2) {
      // LM-head row statistics of this 128-column vocabulary slab (the logits
      // are never written): per row the max logit, its lowest column, and in
      // fp64 S = sum e^{z-max}, T = sum e^{z-max} (z-max), into
      // out (as double) [row][slab][4]
      __builtin_amdgcn_s_barrier();  // every wave is done with the ring
      constexpr int ZLD = 129;       // padded row of the slab's logits in LDS
      float* zs = reinterpret_cast<float*>(lds);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int mrow = mt * 32 + (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i) zs[(mrow + (i >> 2) * 8 + (i & 3)) * ZLD + wv * 32 + (lane & 31)] = acc[mt][i];
      }
      __syncthreads();
      // four threads per row, 32 columns each, combined in a fixed order; 64
      // rows per pass
      const int q = tid & 3;
      for (int r0 = 0; r0 < MT * 32; r0 += 64) {
        const int rr = r0 + (tid >> 2);
        const float* zr = zs + min(rr, MT * 32 - 1) * ZLD + q * 32;
        float best = zr[0];
        int bidx = 0;
        for (int c = 1; c < 32; ++c)
          if (zr[c] > best) {  // increasing column order keeps the lowest index
            best = zr[c];
            bidx = c;
          }
        bidx += slab * 128 + q * 32;
#pragma unroll
        for (int o = 1; o <= 2; o <<= 1) {
          const float ov = __shfl_xor(best, o, 64);
          const int oi = __shfl_xor(bidx, o, 64);
          if (ov > best || (ov == best && oi < bidx)) {
            best = ov;
            bidx = oi;
          }
        }
        const double mx = (double)best;
        double sa = 0.0, ta = 0.0;
        for (int c = 0; c < 32; ++c) {
          const double dz = (double)zr[c] - mx;
          const double e = exp(dz);
          sa += e;
          ta += e * dz;
        }
#pragma unroll
        for (int o = 1; o <= 2; o <<= 1) {  // commutative pairs: every lane of the row gets the same sums
          sa += __shfl_xor(sa, o, 64);
          ta += __shfl_xor(ta, o, 64);
        }
        if (q == 0 && rr < MT * 32 && rr < M) {
          double* p = reinterpret_cast<double*>(out) + ((size_t)rr * n_slabs + slab) * 4;
          p[0] = mx;
          p[1] = (double)bidx;
          p[2] = sa;
          p[3] = ta;
        }
      }
    } else if constexpr (EPI == 0) {
      const int ncol = nt * 32 + (lane & 31);
      if (slab * COLS + wv < NT) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int mrow = mt * 32 + (lane >> 5) * 4;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = mrow + (i >> 2) * 8 + (i & 3);
            if (m < M) out[((size_t)split * cap + m) * N + ncol] = acc[mt][i];
          }
        }
      }
    } else {
      // gate columns in lanes l % 32 < 16 of the tile, the matching up columns
      // in lane l + 16: intermediate column 16 nt + l % 16
      if (slab * COLS + wv < NT) {
        const int f = nt * 16 + (lane & 15);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int mrow = mt * 32 + (lane >> 5) * 4;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int m = mrow + (i >> 2) * 8 + (i & 3);
            const float g = acc[mt][i], u = __shfl_xor(acc[mt][i], 16, 64);
            if (!(lane & 16) && m < M) act[apack_off(m, f, MTt_out)] = f2bf(silu_fast(g) * u);
          }
        }
      }
    }
  }
}

template <int MT, int EPI, int COLS>
__global__ __launch_bounds__(256, 1) void gemm_stream_kernel(const u32x4* __restrict__ Ap, int MTt,
                                                       const u32x4* __restrict__ Wp, float* __restrict__ out,
                                                       uint16_t* __restrict__ act, int MTt_out,
                                                       const int32_t* __restrict__ n_sel, int B, int K, int N,
                                                       int kps, int n_slabs, int total, int cap) {
  if constexpr (COLS == 3) {
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 3) {
      gemm_stream_body<MT, EPI, COLS, true>(Ap, MTt, Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs, total, cap);
      return;
    }
  }
  gemm_stream_body<MT, EPI, COLS, false>(Ap, MTt, Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs, total, cap);
}

#undef GS_WAIT_VM_LGKM0

template <int MT, int EPI, int COLS = 4>
static hipError_t stream_cfg(hipStream_t st, int grid, const void* A, int MTt, const void* Wp, float* out,
                             uint16_t* act, int MTt_out, const int32_t* n_sel, int B, int K, int N, int kps,
                             int n_slabs, int total, int cap, LaunchEvents ev) {
  static std::atomic<unsigned long long> attr_set{0};
  // the statistics epilogue keeps the slab's logits in LDS ([MT*32][129] fp32)
  constexpr size_t zlds = (size_t)MT * 32 * 129 * 4;
  const size_t lds = (EPI == 2 && zlds > StreamShape<MT>::LDS) ? zlds : StreamShape<MT>::LDS;
  hipError_t ea = once_per_device(attr_set, [&] {
    return hipFuncSetAttribute((const void*)gemm_stream_kernel<MT, EPI, COLS>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (ea != hipSuccess) return ea;
  if (ev.start)
    hipExtLaunchKernelGGL((gemm_stream_kernel<MT, EPI, COLS>), dim3(grid), dim3(256), lds, st, ev.start, ev.stop, 0,
                          (const u32x4*)A, MTt, (const u32x4*)Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs,
                          total, cap);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<MT, EPI, COLS>), dim3(grid), dim3(256), lds, st, (const u32x4*)A, MTt,
                       (const u32x4*)Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs, total, cap);
  return hipGetLastError();
}

static int stream_mt(int max_rows) {
  const int t = (max_rows + 31) / 32;
  return t <= GS_MAXMT ? (t < 1 ? 1 : t) : -1;
}

// Split count for the streaming kernel: K must split into multiples of 256;
// the largest split whose workgroup count still fits the chip in one pass (one
// per CU).  0 when the shape does not suit the kernel (more than 288 rows, or
// more row tiles than the activation buffer holds).
int gemm_stream_pick_splits(int max_rows, int K, int N, int n_cu, bool fused, int MTt) {
  const int mt = stream_mt(max_rows);
  if (mt < 0 || mt > MTt || N % 128 != 0 || K % 256 != 0) return 0;
  if (fused) return 1;
  const int n_slabs = N / 128;
  int best = 1;
  for (int s = 2; s <= 32 && s <= K / 256; ++s)
    if ((K / 256) % s == 0 && n_slabs * s <= n_cu) best = s;
  return best;
}

// Fraction of the CUs a launch of `wgs` one-per-CU workgroups keeps busy,
// over its rounds.
static double cu_fill(int wgs, int n_cu) {
  const int rounds = (wgs + n_cu - 1) / n_cu;
  return rounds > 0 ? (double)wgs / ((double)rounds * n_cu) : 0.0;
}

int gemm_stream3_pick_splits(int max_rows, int K, int N, int n_cu, bool fused, int MTt) {
  const int mt = stream_mt(max_rows);
  // up to three row tiles (wave 3 then only shares the activation DMA, and
  // every weight fragment is loaded once): measured faster where the weight
  // stream bounds the GEMM; with rows of its own wave 3 re-reads the three
  // weight tiles and the layout loses from four row tiles on
  if (mt < 0 || mt > 3 || mt > MTt || N % 96 != 0 || K % 256 != 0) return 0;
  const int n3 = N / 96;
  int s3 = 1;
  if (!fused)
    for (int s = 2; s <= 32 && s <= K / 256; ++s)
      if ((K / 256) % s == 0 && n3 * s <= n_cu) s3 = s;
  // only where the 96-column slabs fill more of the chip than the 128-column ones
  const int s4 = gemm_stream_pick_splits(max_rows, K, N, n_cu, fused, MTt);
  const double f4 = s4 > 0 ? cu_fill((N / 128) * s4, n_cu) : 0.0;
  return cu_fill(n3 * s3, n_cu) > f4 + 1e-9 ? s3 : 0;
}

hipError_t launch_gemm_stream3(hipStream_t st, int max_rows, int B, int K, int N, const uint16_t* A, int MTt,
                               const uint16_t* Wp, const int32_t* n_sel, float* out, int splits, uint16_t* act,
                               int MTt_out, LaunchEvents ev) {
  if (max_rows <= 0) return hipSuccess;
  const int mt = stream_mt(max_rows);
  if (mt < 0 || mt > MTt || N % 96 != 0 || splits < 1) return hipErrorInvalidValue;
  const int n_slabs = N / 96;
  const int kps = K / splits;
  if (kps * splits != K || kps % (16 * GS_KC * 4) != 0) return hipErrorInvalidValue;
  if (act != nullptr && splits != 1) return hipErrorInvalidValue;
  const int total = n_slabs * splits;
  const int grid = (total + 7) / 8 * 8;
#define GS3(MT_)                                                                                                  \
  case MT_:                                                                                                       \
    return act ? stream_cfg<MT_, 1, 3>(st, grid, A, MTt, Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs, total, \
                                     max_rows, ev)                                                                \
               : stream_cfg<MT_, 0, 3>(st, grid, A, MTt, Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs, total, \
                                     max_rows, ev);
  switch (mt) {
    GS3(1) GS3(2) GS3(3)
    default: return hipErrorInvalidValue;
  }
#undef GS3
}

hipError_t launch_gemm_stream_stats(hipStream_t st, int max_rows, int K, int N, const uint16_t* A, int MTt,
                                    const uint16_t* Wp, const int32_t* n_sel, double* part, LaunchEvents ev) {
  if (max_rows <= 0) return hipSuccess;
  const int mt = stream_mt(max_rows);
  if (mt < 1 || mt > MTt || N % 128 != 0 || K % 256 != 0) return hipErrorInvalidValue;
  const int n_slabs = N / 128;
  const int grid = (n_slabs + 7) / 8 * 8;
#define GSS(MT_)                                                                                                 \
  case MT_:                                                                                                      \
    return stream_cfg<MT_, 2>(st, grid, A, MTt, Wp, (float*)part, nullptr, 0, n_sel, 1, K, N, K, n_slabs, n_slabs, \
                              max_rows, ev);
  switch (mt) {
    GSS(1) GSS(2) GSS(3) GSS(4) GSS(5) GSS(6) GSS(7) GSS(8) GSS(9)
    default: return hipErrorInvalidValue;
  }
#undef GSS
}

hipError_t launch_gemm_stream(hipStream_t st, int max_rows, int B, int K, int N, const uint16_t* A, int MTt,
                              const uint16_t* Wp, const int32_t* n_sel, float* out, int splits, uint16_t* act,
                              int MTt_out, LaunchEvents ev) {
  if (max_rows <= 0) return hipSuccess;
  const int mt = stream_mt(max_rows);
  if (mt < 0 || mt > MTt || N % 128 != 0 || splits < 1) return hipErrorInvalidValue;
  const int n_slabs = N / 128;
  const int kps = K / splits;
  if (kps * splits != K || kps % (16 * GS_KC * 4) != 0) return hipErrorInvalidValue;
  if (act != nullptr && splits != 1) return hipErrorInvalidValue;
  const int total = n_slabs * splits;
  const int grid = (total + 7) / 8 * 8;
#define GSL(MT_)                                                                                                  \
  case MT_:                                                                                                       \
    return act ? stream_cfg<MT_, 1>(st, grid, A, MTt, Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs, total, \
                                    max_rows, ev)                                                                 \
               : stream_cfg<MT_, 0>(st, grid, A, MTt, Wp, out, act, MTt_out, n_sel, B, K, N, kps, n_slabs, total, \
                                    max_rows, ev);
  // one column tile per wave up to 9 row tiles; more rows go to the
  // row-blocked kernel (measured faster from 10 row tiles on)
  switch (mt) {
    GSL(1) GSL(2) GSL(3) GSL(4) GSL(5) GSL(6) GSL(7) GSL(8) GSL(9)
    default: return hipErrorInvalidValue;
  }
#undef GSL
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
                           const int32_t* n_sel, float* out, LaunchEvents ev) {
  if (max_rows <= 0) return hipSuccess;
  dim3 grid((N + 63) / 64, (max_rows + 63) / 64);
  if (ev.start)
    hipExtLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, ev.start, ev.stop, 0, A, W, n_sel, B, K, N, max_rows,
                          out);
  else
    hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, st, A, W, n_sel, B, K, N, max_rows, out);
  return hipGetLastError();
}

}  // namespace dllm
