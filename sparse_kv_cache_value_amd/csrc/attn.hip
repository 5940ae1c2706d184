// Bidirectional attention of the selected (sparse) queries over every cached
// row (SPA-Cache method step 3: the sparse queries attend over the partially
// updated KV cache; dLLM attention is non-causal, so there is no mask).
// Query head h reads KV head floor(h * Hkv / Hq).
//
// Cache layouts: K [B][Hkv][L][dh] (post-RoPE), V [B][Hkv][L/4][dh][4] -- four
// consecutive keys of one head dimension are adjacent, so a lane's PV operand
// (4 keys x 2 runs of one dimension) is two 8-byte loads.
//
// bf16, dh in {64, 128}, L % 32 == 0: MFMA flash attention.  A workgroup owns
// 32 query rows of one sequence and one head; its 4 waves split the keys and
// each keeps an online softmax (fp32) over 32-key tiles, computing
// S^T = K Q^T (so a query's scores sit in one lane pair and the row max/sum need
// one cross-lane exchange) and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16.
// The four partial results are merged in LDS in a fixed order.  Otherwise a
// reference kernel (one wave per query row and head).
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

size_t attn_partial_floats(int, int, int, int) { return 0; }

__device__ __forceinline__ size_t vt4_off(int j, int t, int dh) {
  return ((size_t)(j >> 2) * dh + t) * 4 + (j & 3);
}

template <typename T>
__global__ __launch_bounds__(64) void attn_ref_kernel(int B, int L, int Hq, int Hkv, int dh, float scale,
                                                      const int32_t* __restrict__ idx, const int32_t* __restrict__ n,
                                                      const T* __restrict__ q, const T* __restrict__ Kc,
                                                      const T* __restrict__ Vc, T* __restrict__ out, int MTt) {
  extern __shared__ float sm[];
  float* qs = sm;       // [dh]
  float* ps = sm + dh;  // [L]
  int b, i;
  const int m = blockIdx.x, h = blockIdx.y;
  if (!row_of(idx, n, B, L, m, b, i)) return;
  const int lane = threadIdx.x;
  const int g = (h * Hkv) / Hq;
  const T* qr = q + (size_t)m * Hq * dh + (size_t)h * dh;
  for (int t = lane; t < dh; t += 64) qs[t] = io<T>::ld(qr + t);
  __syncthreads();
  const T* K = Kc + ((size_t)b * Hkv + g) * L * dh;
  const T* V = Vc + ((size_t)b * Hkv + g) * L * dh;
  float mx = -INFINITY;
  for (int j = lane; j < L; j += 64) {
    const T* kr = K + (size_t)j * dh;
    float s = 0.f;
    for (int t = 0; t < dh; ++t) s = fmaf(qs[t], io<T>::ld(kr + t), s);
    s *= scale;
    ps[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = lane; j < L; j += 64) {
    const float e = expf(ps[j] - mx);
    ps[j] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  __syncthreads();
  const float inv = 1.0f / sum;
  for (int t = lane; t < dh; t += 64) {
    float acc = 0.f;
    for (int j = 0; j < L; ++j) acc = fmaf(ps[j], io<T>::ld(V + vt4_off(j, t, dh)), acc);
    store_a1(out, m, h * dh + t, MTt, Hq * dh, acc * inv);
  }
}

constexpr int ATT_NW = 4;

template <int DH>
__global__ __launch_bounds__(ATT_NW * 64) void attn_mfma_kernel(int B, int L, int Hq, int Hkv, float sl2e, int cap,
                                                                const int32_t* __restrict__ n,
                                                                const bf16* __restrict__ q,
                                                                const bf16* __restrict__ Kc,
                                                                const bf16* __restrict__ Vc,
                                                                bf16* __restrict__ out, int MTt) {
  constexpr int KS = DH / 16;  // k-steps of S^T
  constexpr int DT = DH / 32;  // d-tiles of O^T
  __shared__ float ms[ATT_NW][32], ls[ATT_NW][32];
  __shared__ f32x16_t ox[2][DT][64];
  const int h = blockIdx.y;
  // query tile -> (sequence, first compact row)
  int T = blockIdx.x, b = -1, off = 0, nb = 0;
  for (int bb = 0; bb < B; ++bb) {
    const int c = min(max(n[bb], 0), L);
    const int nt = (c + 31) >> 5;
    if (T < nt) {
      b = bb;
      nb = c;
      break;
    }
    T -= nt;
    off += c;
  }
  if (b < 0) return;
  const int r0 = off + 32 * T;
  if (r0 >= cap) return;
  const int nqv = min(min(32, nb - 32 * T), cap - r0);
  const int g = (h * Hkv) / Hq;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, hlf = lane >> 5, ln = lane & 31;

  // Q^T fragments (B operand): lane holds q[r0 + ln][h*DH + ks*16 + 8*hlf + 0..7]
  u32x4 qf[KS];
  const bool qv = ln < nqv;
  const bf16* qrow = q + (size_t)(r0 + ln) * Hq * DH + (size_t)h * DH + 8 * hlf;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = qv ? *reinterpret_cast<const u32x4*>(qrow + ks * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  const bf16* Kb = Kc + ((size_t)b * Hkv + g) * L * DH;
  const bf16* Vb = Vc + ((size_t)b * Hkv + g) * L * DH;
  const int ntiles = L >> 5;
  const int t_beg = (wv * ntiles) / ATT_NW, t_end = ((wv + 1) * ntiles) / ATT_NW;

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kt = t_beg; kt < t_end; ++kt) {
    const int key0 = kt * 32;
    u32x4 kf[KS];
    const bf16* krow = Kb + (size_t)(key0 + ln) * DH + 8 * hlf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const u32x4*>(krow + ks * 16);
    // V^T fragments: d = dt*32 + ln, keys kk*16 + hlf*4 + {0..3} and kk*16 + 8 + hlf*4 + {0..3}
    u32x2 vlo[2][DT], vhi[2][DT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int g1 = (key0 >> 2) + kk * 4 + hlf;
        vlo[kk][dt] = *reinterpret_cast<const u32x2*>(Vb + ((size_t)g1 * DH + dt * 32 + ln) * 4);
        vhi[kk][dt] = *reinterpret_cast<const u32x2*>(Vb + ((size_t)(g1 + 2) * DH + dt * 32 + ln) * 4);
      }
    f32x16_t s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]),
                                                  __builtin_bit_cast(bf16x8_t, qf[ks]), s, 0, 0, 0);
    float mt = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * sl2e;
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float p[16], rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = exp2f(s[i] * sl2e - m_new);
      rs += p[i];
    }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 pf;
      pf.x = (uint32_t)f2bf(p[8 * kk + 0]) | ((uint32_t)f2bf(p[8 * kk + 1]) << 16);
      pf.y = (uint32_t)f2bf(p[8 * kk + 2]) | ((uint32_t)f2bf(p[8 * kk + 3]) << 16);
      pf.z = (uint32_t)f2bf(p[8 * kk + 4]) | ((uint32_t)f2bf(p[8 * kk + 5]) << 16);
      pf.w = (uint32_t)f2bf(p[8 * kk + 6]) | ((uint32_t)f2bf(p[8 * kk + 7]) << 16);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pf);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 va{vlo[kk][dt].x, vlo[kk][dt].y, vhi[kk][dt].x, vhi[kk][dt].y};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va), pb, o[dt], 0, 0, 0);
      }
    }
  }

  // merge the waves' partial softmax states in a fixed order
  if (lane < 32) {
    ms[wv][ln] = m_run;
    ls[wv][ln] = l_run;
  }
  __syncthreads();
  float mg = ms[0][ln];
#pragma unroll
  for (int w2 = 1; w2 < ATT_NW; ++w2) mg = fmaxf(mg, ms[w2][ln]);
  float lg = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < ATT_NW; ++w2) lg += ls[w2][ln] * exp2f(ms[w2][ln] - mg);
  const float f = exp2f(m_run - mg);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] *= f;
  if (wv >= 2) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ox[wv - 2][dt][lane] = o[dt];
  }
  __syncthreads();
  if (wv < 2) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] += ox[wv][dt][lane];
  }
  __syncthreads();
  if (wv == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ox[0][dt][lane] = o[dt];
  }
  __syncthreads();
  if (wv != 0) return;
  const float inv = 1.0f / lg;
  const int m = r0 + ln;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    o[dt] += ox[0][dt][lane];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float mine[4], part[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mine[e] = o[dt][q4 * 4 + e] * inv;
        part[e] = __shfl_xor(mine[e], 32, 64);
      }
      if ((q4 & 1) == hlf && qv) {
        float v8[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v8[e] = hlf ? part[e] : mine[e];
          v8[4 + e] = hlf ? mine[e] : part[e];
        }
        store_a8(out, m, h * DH + dt * 32 + q4 * 8, MTt, Hq * DH, v8);
      }
    }
  }
}

hipError_t launch_attention(hipStream_t st, bool bf16m, int max_rows, int B, int L, int Hq, int Hkv, int dh,
                            const int32_t* idx, const int32_t* n, const void* q, const void* Kc, const void* Vc,
                            float* partial, void* out, int MTt) {
  (void)partial;
  if (max_rows <= 0) return hipSuccess;
  const float scale = 1.0f / sqrtf((float)dh);
  if (bf16m && (dh == 128 || dh == 64) && L % 32 == 0) {
    const float sl2e = scale * 1.4426950408889634f;
    dim3 grid((max_rows + 31) / 32 + B, Hq);
    if (dh == 128)
      hipLaunchKernelGGL(attn_mfma_kernel<128>, grid, dim3(ATT_NW * 64), 0, st, B, L, Hq, Hkv, sl2e, max_rows, n,
                         (const bf16*)q, (const bf16*)Kc, (const bf16*)Vc, (bf16*)out, MTt);
    else
      hipLaunchKernelGGL(attn_mfma_kernel<64>, grid, dim3(ATT_NW * 64), 0, st, B, L, Hq, Hkv, sl2e, max_rows, n,
                         (const bf16*)q, (const bf16*)Kc, (const bf16*)Vc, (bf16*)out, MTt);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(dh + L) * sizeof(float);
  dim3 grid(max_rows, Hq);
  if (bf16m)
    hipLaunchKernelGGL(attn_ref_kernel<bf16>, grid, dim3(64), lds, st, B, L, Hq, Hkv, dh, scale, idx, n,
                       (const bf16*)q, (const bf16*)Kc, (const bf16*)Vc, (bf16*)out, MTt);
  else
    hipLaunchKernelGGL(attn_ref_kernel<float>, grid, dim3(64), lds, st, B, L, Hq, Hkv, dh, scale, idx, n,
                       (const float*)q, (const float*)Kc, (const float*)Vc, (float*)out, MTt);
  return hipGetLastError();
}

}  // namespace dllm
