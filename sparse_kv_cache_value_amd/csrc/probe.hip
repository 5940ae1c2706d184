// Achievable streaming-read bandwidth of the device (diagnostics): the
// denominator the measured kernels are compared with besides the published
// HBM peak.  Each workgroup streams its own contiguous share of a buffer with
// 16-byte nontemporal loads, D loads in flight per thread.
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef unsigned int u32x4_p __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void stream_probe_kernel(const u32x4_p* __restrict__ src, size_t per_wg16,
                                                           unsigned* __restrict__ out) {
  const u32x4_p* p = src + (size_t)blockIdx.x * per_wg16 + threadIdx.x;
  u32x4_p acc = {0u, 0u, 0u, 0u};
  for (size_t i = 0; i < per_wg16; i += 256 * D) {
    u32x4_p v[D];
#pragma unroll
    for (int d = 0; d < D; ++d) v[d] = __builtin_nontemporal_load(p + i + (size_t)d * 256);
#pragma unroll
    for (int d = 0; d < D; ++d) acc ^= v[d];
  }
  // a data-dependent store keeps the loads alive
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) out[blockIdx.x] = acc.x;
}

size_t stream_probe_quantum(int grid, int depth) { return (size_t)grid * 256 * depth * 16; }

hipError_t launch_stream_probe(hipStream_t st, int grid, int depth, const void* buf, size_t bytes, unsigned* out) {
  const size_t q = stream_probe_quantum(grid, depth);
  if (bytes < q || bytes % q) return hipErrorInvalidValue;
  const size_t per = bytes / 16 / grid;
  if (depth == 4)
    hipLaunchKernelGGL(stream_probe_kernel<4>, dim3(grid), dim3(256), 0, st, (const u32x4_p*)buf, per, out);
  else if (depth == 8)
    hipLaunchKernelGGL(stream_probe_kernel<8>, dim3(grid), dim3(256), 0, st, (const u32x4_p*)buf, per, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dllm
