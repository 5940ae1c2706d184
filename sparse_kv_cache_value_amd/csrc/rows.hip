// Row bookkeeping, gathers, norms and GEMM epilogues of the sparse layer.
//
// Sparse execution (SPA-Cache, method step 3): only the selected rows I are
// gathered, normed and projected; their new keys/values are scattered into
// the cache before attention, and the layer output is written back only at I.
#include "common.h"
#include "kernels.h"

namespace dllm {

// ---------------------------------------------------------------------------
// Forced rows (EntropyCache step 3: current mask block + k most recent
// decoded tokens; Polestar: current block), the rows whose token changed since
// the last step (the layer-0 rows to refresh) and this step's full flags.
// One workgroup per sequence.
// ---------------------------------------------------------------------------
__global__ void prep_kernel(int L, int block_len, int rule, int recent_k, int mode,
                            const int32_t* __restrict__ history, const int32_t* __restrict__ n_history,
                            const int32_t* __restrict__ n_new, const int32_t* __restrict__ block_start,
                            const uint8_t* __restrict__ full_next, uint8_t* __restrict__ forced,
                            uint8_t* __restrict__ step_full, int32_t* __restrict__ idx0,
                            int32_t* __restrict__ n0) {
  const int b = blockIdx.x;
  const int nh = n_history[b];
  const int bs = block_start[b];
  const int full = mode == 1 ? 1 : (mode == 2 ? 0 : (full_next[b] ? 1 : 0));
  if (forced != nullptr) {
    for (int i = threadIdx.x; i < L; i += blockDim.x)
      forced[(size_t)b * L + i] = (rule >= 1 && i >= bs && i < bs + block_len) ? 1 : 0;
    __syncthreads();
    if (rule == 2) {
      const int nr = min(recent_k, nh);
      for (int j = threadIdx.x; j < nr; j += blockDim.x) {
        const int p = history[(size_t)b * L + nh - 1 - j];
        if (p >= 0 && p < L) forced[(size_t)b * L + p] = 1;
      }
    }
  }
  if (idx0 != nullptr) {
    if (full) {
      for (int i = threadIdx.x; i < L; i += blockDim.x) idx0[(size_t)b * L + i] = i;
      if (threadIdx.x == 0) n0[b] = L;
    } else {
      const int nn = min(n_new[b], nh);
      for (int j = threadIdx.x; j < nn; j += blockDim.x) idx0[(size_t)b * L + j] = history[(size_t)b * L + nh - nn + j];
      if (threadIdx.x == 0) n0[b] = nn;
    }
  }
  if (step_full != nullptr && threadIdx.x == 0) step_full[b] = (uint8_t)full;
}

hipError_t launch_prep(hipStream_t st, int B, int L, int block_len, int rule, int recent_k, int mode,
                       const int32_t* history, const int32_t* n_history, const int32_t* n_new,
                       const int32_t* block_start, const uint8_t* full_next, uint8_t* forced,
                       uint8_t* step_full, int32_t* idx0, int32_t* n0) {
  hipLaunchKernelGGL(prep_kernel, dim3(B), dim3(256), 0, st, L, block_len, rule, recent_k, mode, history,
                     n_history, n_new, block_start, full_next, forced, step_full, idx0, n0);
  return hipGetLastError();
}

hipError_t launch_forced(hipStream_t st, int B, int L, int block_len, int rule, int recent_k,
                         const int32_t* history, const int32_t* n_history, const int32_t* block_start,
                         uint8_t* forced) {
  hipLaunchKernelGGL(prep_kernel, dim3(B), dim3(256), 0, st, L, block_len, rule, recent_k, 2, history,
                     n_history, (const int32_t*)nullptr, block_start, (const uint8_t*)nullptr, forced,
                     (uint8_t*)nullptr, (int32_t*)nullptr, (int32_t*)nullptr);
  return hipGetLastError();
}

__global__ void all_rows_kernel(int L, int32_t* __restrict__ idx, int32_t* __restrict__ n) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < L; i += blockDim.x) idx[(size_t)b * L + i] = i;
  if (threadIdx.x == 0) n[b] = L;
}

hipError_t launch_all_rows(hipStream_t st, int B, int L, int32_t* idx, int32_t* n) {
  hipLaunchKernelGGL(all_rows_kernel, dim3(B), dim3(256), 0, st, L, idx, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Layer-0 input of the listed rows: the embedding of the row's token.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void embed_kernel(int B, int L, int d, int V, const int32_t* __restrict__ idx,
                             const int32_t* __restrict__ n, const int32_t* __restrict__ tokens,
                             const T* __restrict__ embed, T* __restrict__ h0) {
  int b, i;
  if (!row_of(idx, n, B, L, blockIdx.x, b, i)) return;
  const int tok = tokens[(size_t)b * L + i];
  T* dst = h0 + ((size_t)b * L + i) * d;
  if (tok < 0 || tok >= V) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) dst[c] = T(0);
    return;
  }
  const T* src = embed + (size_t)tok * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) dst[c] = src[c];
}

hipError_t launch_embed(hipStream_t st, bool bf16m, int max_rows, int B, int L, int d, int V,
                        const int32_t* idx, const int32_t* n, const int32_t* tokens, const void* embed,
                        void* h0) {
  if (max_rows <= 0) return hipSuccess;
  if (bf16m)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(max_rows), dim3(256), 0, st, B, L, d, V, idx, n, tokens,
                       (const bf16*)embed, (bf16*)h0);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(max_rows), dim3(256), 0, st, B, L, d, V, idx, n, tokens,
                       (const float*)embed, (float*)h0);
  return hipGetLastError();
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float4 v) {
  uint2 u;
  u.x = pack2bf(v.x, v.y);
  u.y = pack2bf(v.z, v.w);
  *reinterpret_cast<uint2*>(p) = u;
}

__device__ __forceinline__ float4 sum_splits4(const float* __restrict__ p, size_t stride, int S) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += 8) {
    float4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      t[j] = (s0 + j < S) ? *reinterpret_cast<const float4*>(p + (size_t)(s0 + j) * stride) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) {
        acc.x += t[j].x; acc.y += t[j].y; acc.z += t[j].z; acc.w += t[j].w;
      }
  }
  return acc;
}

// ---------------------------------------------------------------------------
// Gather + RMSNorm (fp32 statistics) of the selected rows into compact A.
// One workgroup per row; each thread holds up to RV groups of 8 consecutive
// values in registers between the statistics and the normalised store.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(RT) void gather_norm_kernel(int B, int L, int d, float eps, int MTt,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ n,
                                                          const T* __restrict__ H, const float* __restrict__ g,
                                                          T* __restrict__ A) {
  __shared__ float red[RT / 64];
  int b, i;
  const int m = blockIdx.x;
  if (!row_of(idx, n, B, L, m, b, i)) return;
  norm_row_store<T>(H + ((size_t)b * L + i) * d, d, eps, g, A, m, MTt, red);
}

// The same rows, one per wave (4 rows per workgroup), for launches of many
// rows: no workgroup barrier and an eighth of the workgroups.  Each lane
// stands in for the 8 threads l + 64 w of gather_norm_kernel's workgroup
// and keeps their partial sums apart, so that the sum of squares is added
// in the same order (each virtual wave's shuffle tree, then the 8 wave
// totals in wave order) and the result is bit-identical.
constexpr int GN_ROWS = 4;             // rows (waves) per workgroup
constexpr int GN_WAVE_MIN_ROWS = 1024;  // launches from this many rows use it

template <typename T, int RVN>  // RVN: the groups of 8 per virtual thread that d needs (1 up to d = RT * 8)
__global__ __launch_bounds__(GN_ROWS * 64) void gather_norm_rows_kernel(int B, int L, int d, float eps, int MTt,
                                                                       const int32_t* __restrict__ idx,
                                                                       const int32_t* __restrict__ n,
                                                                       const T* __restrict__ H,
                                                                       const float* __restrict__ g,
                                                                       T* __restrict__ A) {
  constexpr int VW = RT / 64;  // virtual waves of gather_norm_kernel's workgroup
  const int lane = threadIdx.x & 63;
  const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * GN_ROWS + (threadIdx.x >> 6));
  int b, i;
  if (!row_of(idx, n, B, L, m, b, i)) return;
  const T* x = H + ((size_t)b * L + i) * d;
  float v[VW][RVN][8];
  float part[VW];
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    part[w] = 0.f;
#pragma unroll
    for (int r = 0; r < RVN; ++r) {
      const int c8 = (lane + 64 * w + r * RT) * 8;
      if (c8 < d) {
        load8<T>(x + c8, v[w][r]);
#pragma unroll
        for (int e = 0; e < 8; ++e) part[w] += v[w][r][e] * v[w][r][e];
      }
    }
  }
  // virtual wave w's total as its lane 0 would have it, then the totals in order
  float ss = 0.f;
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    const float t = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wave_sum(part[w]))));
    ss = w == 0 ? t : ss + t;
  }
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int w = 0; w < VW; ++w)
#pragma unroll
    for (int r = 0; r < RVN; ++r) {
      const int c8 = (lane + 64 * w + r * RT) * 8;
      if (c8 < d) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = v[w][r][e] * inv * g[c8 + e];
        store_a8(A, m, c8, MTt, d, o);
      }
    }
}

hipError_t launch_gather_norm(hipStream_t st, bool bf16m, int max_rows, int B, int L, int d, float eps, int MTt,
                              const int32_t* idx, const int32_t* n, const void* H, const float* g,
                              void* A) {
  if (max_rows <= 0) return hipSuccess;
  if (max_rows >= GN_WAVE_MIN_ROWS) {
    const dim3 grid((max_rows + GN_ROWS - 1) / GN_ROWS);
#define GNR(TT, RR)                                                                                        \
  hipLaunchKernelGGL((gather_norm_rows_kernel<TT, RR>), grid, dim3(GN_ROWS * 64), 0, st, B, L, d, eps, MTt, idx, n, \
                     (const TT*)H, g, (TT*)A)
    if (bf16m) {
      if (d <= RT * 8) GNR(bf16, 1); else GNR(bf16, RV);
    } else {
      if (d <= RT * 8) GNR(float, 1); else GNR(float, RV);
    }
#undef GNR
    return hipGetLastError();
  }
  if (bf16m)
    hipLaunchKernelGGL(gather_norm_kernel<bf16>, dim3(max_rows), dim3(RT), 0, st, B, L, d, eps, MTt, idx, n,
                       (const bf16*)H, g, (bf16*)A);
  else
    hipLaunchKernelGGL(gather_norm_kernel<float>, dim3(max_rows), dim3(RT), 0, st, B, L, d, eps, MTt, idx, n,
                       (const float*)H, g, (float*)A);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// QKV epilogue: sum split partials, rotate-half RoPE on q and k at the row's
// position (cos/sin tables [L][dh/2]), write q (compact) and scatter k, v into
// the cache rows [b][g][i][:].
//
// Split partials of every GEMM are laid out [S][cap][N] (cap = the launch's
// row capacity), so their addresses depend on the compact row m only: a
// thread issues all its partial loads together with the row-list loads and
// only then waits, once, for the row's position.  S is a template parameter
// (1, 2, 4, 8) so the loads are unconditional; other counts take the
// runtime-S path (S = 0).
// ---------------------------------------------------------------------------
template <typename T, int S>
__global__ __launch_bounds__(256) void qkv_epilogue_kernel(int B, int L, int Hq, int Hkv, int dh, int Srt, int cap,
                                                           const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ n,
                                                           const float* __restrict__ part,
                                                           const float* __restrict__ rc,
                                                           const float* __restrict__ rs, T* __restrict__ q,
                                                           T* __restrict__ Kc, T* __restrict__ Vc) {
  const int m = blockIdx.x;
  const int n0 = n[0];
  const int i0 = idx[m < L ? m : L - 1];
  const int nq = Hq * dh, nv = Hkv * dh, N = nq + 2 * nv, half = dh / 2;
  const size_t sstride = (size_t)cap * N;
  const float* p0 = part + (size_t)m * N;
  // item p: rotary quad p (four consecutive pairs (j, j + dh/2) of one q or k
  // head) and value quad p (four consecutive value columns)
  const int qph = half / 4, nquads = (Hq + Hkv) * qph, nvq = nv / 4;
  const int items = nquads > nvq ? nquads : nvq;
  const int t0 = blockIdx.y * 256 + threadIdx.x, tstep = 256 * gridDim.y;
  constexpr int SA = S ? S : 1;
  float4 ta[SA], tc[SA], tv[SA];
  auto issue = [&](int p) {
    if constexpr (S) {
      const int pq = p < nquads ? p : 0, pv = p < nvq ? p : 0;
      const int head = pq / qph, c0 = head * dh + (pq - head * qph) * 4;
      load_splits4<S>(p0 + c0, sstride, ta);
      load_splits4<S>(p0 + c0 + half, sstride, tc);
      load_splits4<S>(p0 + nq + nv + pv * 4, sstride, tv);
    }
  };
  if (t0 < items) issue(t0);
  int b, i;
  if (!row_resolve(idx, n, B, L, m, n0, i0, b, i)) return;
  for (int p = t0; p < items; p += tstep) {
    if (p != t0) issue(p);
    if (p < nquads) {
      const int head = p / qph, j = (p - head * qph) * 4;
      const int c0 = head * dh + j, c1 = c0 + half;
      const float4 cs = *reinterpret_cast<const float4*>(rc + (size_t)i * half + j);
      const float4 sn = *reinterpret_cast<const float4*>(rs + (size_t)i * half + j);
      float4 a, c;
      if constexpr (S) {
        a = add_splits4<S>(ta);
        c = add_splits4<S>(tc);
      } else {
        a = sum_splits4(p0 + c0, sstride, Srt);
        c = sum_splits4(p0 + c1, sstride, Srt);
      }
      const float4 r0 = make_float4(a.x * cs.x - c.x * sn.x, a.y * cs.y - c.y * sn.y, a.z * cs.z - c.z * sn.z,
                                    a.w * cs.w - c.w * sn.w);
      const float4 r1 = make_float4(c.x * cs.x + a.x * sn.x, c.y * cs.y + a.y * sn.y, c.z * cs.z + a.z * sn.z,
                                    c.w * cs.w + a.w * sn.w);
      if (head < Hq) {
        store4<T>(q + (size_t)m * nq + c0, r0);
        store4<T>(q + (size_t)m * nq + c1, r1);
      } else {
        // four consecutive dimensions are adjacent in the fragment layout
        T* kb = Kc + ((size_t)b * Hkv + (head - Hq)) * (size_t)l32_of(L) * dh;
        store4<T>(kb + kc_off(i, j, dh), r0);
        store4<T>(kb + kc_off(i, j + half, dh), r1);
      }
    }
    if (p < nvq) {
      const int c4 = p * 4;
      float4 v;
      if constexpr (S) v = add_splits4<S>(tv);
      else v = sum_splits4(p0 + nq + nv + c4, sstride, Srt);
      const int g = c4 / dh, t = c4 - g * dh;
      // values are row-major: the quad is one contiguous piece of the key's row
      T* vb = Vc + ((size_t)b * Hkv + g) * (size_t)l32_of(L) * dh;
      store4<T>(vb + (size_t)i * dh + t, v);
    }
  }
}

template <typename T>
static hipError_t qkv_epi_cfg(hipStream_t st, int max_rows, int B, int L, int Hq, int Hkv, int dh, int S,
                              const int32_t* idx, const int32_t* n, const float* part, const float* rc,
                              const float* rs, T* q, T* Kc, T* Vc) {
  const dim3 grid(max_rows, 4), blk(256);
#define QE(SS) hipLaunchKernelGGL((qkv_epilogue_kernel<T, SS>), grid, blk, 0, st, B, L, Hq, Hkv, dh, S, max_rows, idx, \
                                  n, part, rc, rs, q, Kc, Vc)
  switch (S) {
    case 1: QE(1); break;
    case 2: QE(2); break;
    case 4: QE(4); break;
    case 8: QE(8); break;
    default: QE(0); break;
  }
#undef QE
  return hipGetLastError();
}

hipError_t launch_qkv_epilogue(hipStream_t st, bool bf16m, int max_rows, int B, int L, int Hq, int Hkv,
                               int dh, int S, const int32_t* idx, const int32_t* n, const float* part,
                               const float* rope_cos, const float* rope_sin, void* q_out, void* Kc,
                               void* Vc) {
  if (max_rows <= 0) return hipSuccess;
  if (bf16m)
    return qkv_epi_cfg<bf16>(st, max_rows, B, L, Hq, Hkv, dh, S, idx, n, part, rope_cos, rope_sin, (bf16*)q_out,
                             (bf16*)Kc, (bf16*)Vc);
  return qkv_epi_cfg<float>(st, max_rows, B, L, Hq, Hkv, dh, S, idx, n, part, rope_cos, rope_sin, (float*)q_out,
                            (float*)Kc, (float*)Vc);
}

// ---------------------------------------------------------------------------
// Output projection epilogue: h' = x + o W_o (fp32, split partials summed in
// order), then the FFN norm into the next GEMM's input.  The partial loads
// are issued before the row's position is known (split layout [S][cap][d]).
// ---------------------------------------------------------------------------
template <typename T, int S>
__global__ __launch_bounds__(RT) void o_epilogue_kernel(int B, int L, int d, int Srt, int cap, float eps, int MTt,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ n,
                                                         const float* __restrict__ part,
                                                         const T* __restrict__ H, const float* __restrict__ g2,
                                                         float* __restrict__ hprime, T* __restrict__ A2) {
  __shared__ float red[RT / 64];
  const int m = blockIdx.x;
  const int n0 = n[0];
  const int i0 = idx[m < L ? m : L - 1];
  const size_t sstride = (size_t)cap * d;
  const float* p0 = part + (size_t)m * d;
  constexpr int SA = S ? S : 1;
  float4 t[RV][2][SA];
  if constexpr (S) {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const int c8 = (threadIdx.x + r * RT) * 8;
      if (r == 0 || c8 < d) {
        const int cc = c8 < d ? c8 : 0;
        load_splits4<S>(p0 + cc, sstride, t[r][0]);
        load_splits4<S>(p0 + cc + 4, sstride, t[r][1]);
      }
    }
  }
  int b, i;
  if (!row_resolve(idx, n, B, L, m, n0, i0, b, i)) return;
  const T* x = H + ((size_t)b * L + i) * d;
  float* hp = hprime + (size_t)m * d;
  float v[RV][8];
  float ss = 0.f;
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    const int c8 = (threadIdx.x + r * RT) * 8;
    if (c8 < d) {
      load8<T>(x + c8, v[r]);
      float4 a, c;
      if constexpr (S) {
        a = add_splits4<S>(t[r][0]);
        c = add_splits4<S>(t[r][1]);
      } else {
        a = sum_splits4(p0 + c8, sstride, Srt);
        c = sum_splits4(p0 + c8 + 4, sstride, Srt);
      }
      v[r][0] += a.x; v[r][1] += a.y; v[r][2] += a.z; v[r][3] += a.w;
      v[r][4] += c.x; v[r][5] += c.y; v[r][6] += c.z; v[r][7] += c.w;
      *reinterpret_cast<float4*>(hp + c8) = make_float4(v[r][0], v[r][1], v[r][2], v[r][3]);
      *reinterpret_cast<float4*>(hp + c8 + 4) = make_float4(v[r][4], v[r][5], v[r][6], v[r][7]);
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
      for (int e = 0; e < 8; ++e) o[e] = v[r][e] * inv * g2[c8 + e];
      store_a8(A2, m, c8, MTt, d, o);
    }
  }
}

// The same rows, one per wave (GN_ROWS per workgroup), for launches of many
// rows and a split count fixed at compile time: each lane stands in for the
// 8 threads l + 64 w of o_epilogue_kernel's workgroup, so every value and the
// order of the sum of squares are the same and the outputs bit-identical.
template <typename T, int S, int RVN>
__global__ __launch_bounds__(GN_ROWS * 64) void o_epilogue_rows_kernel(int B, int L, int d, int cap, float eps,
                                                                      int MTt, const int32_t* __restrict__ idx,
                                                                      const int32_t* __restrict__ n,
                                                                      const float* __restrict__ part,
                                                                      const T* __restrict__ H,
                                                                      const float* __restrict__ g2,
                                                                      float* __restrict__ hprime,
                                                                      T* __restrict__ A2) {
  constexpr int VW = RT / 64;
  const int lane = threadIdx.x & 63;
  const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * GN_ROWS + (threadIdx.x >> 6));
  if (m >= cap) return;
  const int n0 = n[0];
  const int i0 = idx[m < L ? m : L - 1];
  const size_t sstride = (size_t)cap * d;
  const float* p0 = part + (size_t)m * d;
  // the partials, before the row's position is known (clamped, unconditional)
  float4 t[VW][RVN][2][S];
#pragma unroll
  for (int w = 0; w < VW; ++w)
#pragma unroll
    for (int r = 0; r < RVN; ++r) {
      const int c8 = (lane + 64 * w + r * RT) * 8;
      const int cc = c8 < d ? c8 : 0;
      load_splits4<S>(p0 + cc, sstride, t[w][r][0]);
      load_splits4<S>(p0 + cc + 4, sstride, t[w][r][1]);
    }
  int b, i;
  if (!row_resolve(idx, n, B, L, m, n0, i0, b, i)) return;
  const T* x = H + ((size_t)b * L + i) * d;
  float* hp = hprime + (size_t)m * d;
  float v[VW][RVN][8];
  float pt[VW];
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    pt[w] = 0.f;
#pragma unroll
    for (int r = 0; r < RVN; ++r) {
      const int c8 = (lane + 64 * w + r * RT) * 8;
      if (c8 < d) {
        load8<T>(x + c8, v[w][r]);
        const float4 a = add_splits4<S>(t[w][r][0]), c = add_splits4<S>(t[w][r][1]);
        v[w][r][0] += a.x; v[w][r][1] += a.y; v[w][r][2] += a.z; v[w][r][3] += a.w;
        v[w][r][4] += c.x; v[w][r][5] += c.y; v[w][r][6] += c.z; v[w][r][7] += c.w;
        *reinterpret_cast<float4*>(hp + c8) = make_float4(v[w][r][0], v[w][r][1], v[w][r][2], v[w][r][3]);
        *reinterpret_cast<float4*>(hp + c8 + 4) = make_float4(v[w][r][4], v[w][r][5], v[w][r][6], v[w][r][7]);
#pragma unroll
        for (int e = 0; e < 8; ++e) pt[w] += v[w][r][e] * v[w][r][e];
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    const float tw = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wave_sum(pt[w]))));
    ss = w == 0 ? tw : ss + tw;
  }
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int w = 0; w < VW; ++w)
#pragma unroll
    for (int r = 0; r < RVN; ++r) {
      const int c8 = (lane + 64 * w + r * RT) * 8;
      if (c8 < d) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = v[w][r][e] * inv * g2[c8 + e];
        store_a8(A2, m, c8, MTt, d, o);
      }
    }
}

template <typename T>
static hipError_t o_epi_cfg(hipStream_t st, int max_rows, int B, int L, int d, int S, float eps, int MTt,
                            const int32_t* idx, const int32_t* n, const float* part, const T* H, const float* g2,
                            float* hprime, T* A2) {
  // (one or two splits: with four the partials alone take 128 registers)
  if (max_rows >= GN_WAVE_MIN_ROWS && d <= RT * 8 && (S == 1 || S == 2)) {
    const dim3 grid((max_rows + GN_ROWS - 1) / GN_ROWS);
#define OR(SS)                                                                                                   \
  hipLaunchKernelGGL((o_epilogue_rows_kernel<T, SS, 1>), grid, dim3(GN_ROWS * 64), 0, st, B, L, d, max_rows, eps, MTt, \
                     idx, n, part, H, g2, hprime, A2)
    if (S == 1) OR(1); else OR(2);
#undef OR
    return hipGetLastError();
  }
#define OE(SS) hipLaunchKernelGGL((o_epilogue_kernel<T, SS>), dim3(max_rows), dim3(RT), 0, st, B, L, d, S, max_rows, \
                                  eps, MTt, idx, n, part, H, g2, hprime, A2)
  switch (S) {
    case 1: OE(1); break;
    case 2: OE(2); break;
    case 4: OE(4); break;
    case 8: OE(8); break;
    default: OE(0); break;
  }
#undef OE
  return hipGetLastError();
}

hipError_t launch_o_epilogue(hipStream_t st, bool bf16m, int max_rows, int B, int L, int d, int S,
                             float eps, int MTt, const int32_t* idx, const int32_t* n, const float* part,
                             const void* H, const float* g2, float* hprime, void* A2) {
  if (max_rows <= 0) return hipSuccess;
  if (bf16m)
    return o_epi_cfg<bf16>(st, max_rows, B, L, d, S, eps, MTt, idx, n, part, (const bf16*)H, g2, hprime, (bf16*)A2);
  return o_epi_cfg<float>(st, max_rows, B, L, d, S, eps, MTt, idx, n, part, (const float*)H, g2, hprime, (float*)A2);
}

// ---------------------------------------------------------------------------
// SwiGLU (fp32 models): act = SiLU(gate) * up.  The fused fp32 gate|up weight
// interleaves the two by 32-column tiles: packed tile 2t is gate tile t, tile
// 2t+1 is up tile t.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(int B, int F, int S, int cap, const int32_t* __restrict__ n,
                                                     const float* __restrict__ part, T* __restrict__ act) {
  const int M = total_rows(n, B, cap);
  const int m = blockIdx.y;
  if (m >= M) return;
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const int N = 2 * F;
  const size_t sstride = (size_t)cap * N;
  const int cg = (f >> 5) * 64 + (f & 31);
  const float gv = sum_splits(part + (size_t)m * N + cg, sstride, S);
  const float uv = sum_splits(part + (size_t)m * N + cg + 32, sstride, S);
  const float sl = gv / (1.0f + expf(-gv));
  io<T>::st(act + (size_t)m * F + f, sl * uv);
}

hipError_t launch_swiglu(hipStream_t st, bool bf16m, int max_rows, int B, int F, int S, const int32_t* n,
                         const float* part, void* act) {
  if (max_rows <= 0) return hipSuccess;
  dim3 grid((F + 255) / 256, max_rows);
  if (bf16m)
    hipLaunchKernelGGL(swiglu_kernel<bf16>, grid, dim3(256), 0, st, B, F, S, max_rows, n, part, (bf16*)act);
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, grid, dim3(256), 0, st, B, F, S, max_rows, n, part, (float*)act);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Down-projection epilogue: out = h' + act W_down, written back at the row's
// slot of the next layer's input; the row's proxy reference is refreshed.
// The partial and h' loads are issued before the row's position is known.
// ---------------------------------------------------------------------------
template <typename T, int S>
__global__ __launch_bounds__(256) void down_epilogue_kernel(int B, int L, int d, int r, int Srt, int cap,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ n,
                                                            const float* __restrict__ part,
                                                            const float* __restrict__ hprime,
                                                            T* __restrict__ Hout, const double* __restrict__ pcur,
                                                            double* __restrict__ pref, double* __restrict__ score) {
  const int m = blockIdx.x;
  const int n0 = n[0];
  const int i0 = idx[m < L ? m : L - 1];
  const size_t sstride = (size_t)cap * d;
  const float* hp = hprime + (size_t)m * d;
  const float* p0 = part + (size_t)m * d;
  const int t0 = (blockIdx.y * 256 + threadIdx.x) * 4, tstep = 256 * gridDim.y * 4;
  constexpr int SA = S ? S : 1;
  float4 t[SA], h;
  if constexpr (S)
    if (t0 < d) {
      h = *reinterpret_cast<const float4*>(hp + t0);
      load_splits4<S>(p0 + t0, sstride, t);
    }
  int b, i;
  if (!row_resolve(idx, n, B, L, m, n0, i0, b, i)) return;
  const size_t row = (size_t)b * L + i;
  T* o = Hout + row * d;
  for (int c4 = t0; c4 < d; c4 += tstep) {
    float4 a;
    if (S && c4 == t0) {
      if constexpr (S) a = add_splits4<S>(t);
    } else {
      a = sum_splits4(p0 + c4, sstride, Srt);
      h = *reinterpret_cast<const float4*>(hp + c4);
    }
    store4<T>(o + c4, make_float4(h.x + a.x, h.y + a.y, h.z + a.z, h.w + a.w));
  }
  if (blockIdx.y != 0 || !pref) return;
  for (int j = threadIdx.x; j < r; j += 256) pref[row * r + j] = pcur[row * r + j];
  if (threadIdx.x == 0) score[row] = 0.0;
}

template <typename T>
static hipError_t down_epi_cfg(hipStream_t st, int max_rows, int B, int L, int d, int r, int S, const int32_t* idx,
                               const int32_t* n, const float* part, const float* hprime, T* H_out,
                               const double* pcur, double* pref, double* score) {
  const dim3 grid(max_rows, 4), blk(256);
#define DE(SS) hipLaunchKernelGGL((down_epilogue_kernel<T, SS>), grid, blk, 0, st, B, L, d, r, S, max_rows, idx, n, \
                                  part, hprime, H_out, pcur, pref, score)
  switch (S) {
    case 1: DE(1); break;
    case 2: DE(2); break;
    case 4: DE(4); break;
    case 8: DE(8); break;
    default: DE(0); break;
  }
#undef DE
  return hipGetLastError();
}

hipError_t launch_down_epilogue(hipStream_t st, bool bf16m, int max_rows, int B, int L, int d, int r,
                                int S, const int32_t* idx, const int32_t* n, const float* part,
                                const float* hprime, void* H_out, const double* pcur, double* pref,
                                double* score) {
  if (max_rows <= 0) return hipSuccess;
  if (bf16m)
    return down_epi_cfg<bf16>(st, max_rows, B, L, d, r, S, idx, n, part, hprime, (bf16*)H_out, pcur, pref, score);
  return down_epi_cfg<float>(st, max_rows, B, L, d, r, S, idx, n, part, hprime, (float*)H_out, pcur, pref, score);
}

}  // namespace dllm
