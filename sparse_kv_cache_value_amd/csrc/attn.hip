// Bidirectional attention of the selected (sparse) queries over every cached
// row (SPA-Cache method step 3: the sparse queries attend over the partially
// updated KV cache; dLLM attention is non-causal, so no mask).  Query head h
// reads KV head floor(h * Hkv / Hq).
//
// Reference kernel: one wave per (query row, head); scores with lanes over
// keys, fp32 softmax, output with lanes over the head dimension.
#include "common.h"
#include "kernels.h"

namespace dllm {

size_t attn_partial_floats(int, int, int, int) { return 0; }

template <typename T>
__global__ __launch_bounds__(64) void attn_ref_kernel(int B, int L, int Hq, int Hkv, int dh, float scale,
                                                      const int32_t* __restrict__ idx, const int32_t* __restrict__ n,
                                                      const T* __restrict__ q, const T* __restrict__ Kc,
                                                      const T* __restrict__ Vc, T* __restrict__ out) {
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
  T* o = out + (size_t)m * Hq * dh + (size_t)h * dh;
  for (int t = lane; t < dh; t += 64) {
    float acc = 0.f;
    for (int j = 0; j < L; ++j) acc = fmaf(ps[j], io<T>::ld(V + (size_t)j * dh + t), acc);
    io<T>::st(o + t, acc * inv);
  }
}

hipError_t launch_attention(hipStream_t st, bool bf16m, int max_rows, int B, int L, int Hq, int Hkv, int dh,
                            const int32_t* idx, const int32_t* n, const void* q, const void* Kc, const void* Vc,
                            float* partial, void* out) {
  (void)partial;
  if (max_rows <= 0) return hipSuccess;
  const float scale = 1.0f / sqrtf((float)dh);
  const size_t lds = (size_t)(dh + L) * sizeof(float);
  dim3 grid(max_rows, Hq);
  if (bf16m)
    hipLaunchKernelGGL(attn_ref_kernel<bf16>, grid, dim3(64), lds, st, B, L, Hq, Hkv, dh, scale, idx, n,
                       (const bf16*)q, (const bf16*)Kc, (const bf16*)Vc, (bf16*)out);
  else
    hipLaunchKernelGGL(attn_ref_kernel<float>, grid, dim3(64), lds, st, B, L, Hq, Hkv, dh, scale, idx, n,
                       (const float*)q, (const float*)Kc, (const float*)Vc, (float*)out);
  return hipGetLastError();
}

}  // namespace dllm
