// Per-layer index set I (SPA-Cache method steps 1-2; EntropyCache step 3).
//
// Forced rows (current mask block, recent decoded tokens) are always in I;
// the remaining max(k, |F|) - |F| rows are the non-forced rows with the
// largest drift score, ties to the lower index.  One 256-thread workgroup
// per sequence; thread t owns the contiguous rows [t*E, t*E + E).  The k-th
// largest score is found by an exact MSB-first radix select over the fp64
// bit patterns (non-negative doubles order like their unsigned bits), stopping
// as soon as the bucket holding the cut is taken whole; rows equal to the
// threshold on the resolved bits are ranked by an index-order scan, and the
// selected rows are compacted in ascending order by a second scan.  When no
// more candidates have a non-zero score than are needed (zero drift marks rows
// whose input did not change), the cut is zero and no radix pass runs.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int SEL_T = 256;  // 4 waves: cheap barriers between the radix passes
constexpr int SEL_W = SEL_T / 64;
constexpr int SEL_EMAX = 32;  // L <= 8192

// Exclusive prefix sum over the block (thread order); *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < SEL_W; ++i) {
    const int s = wsum[i];
    if (i < w) before += s;
    tot += s;
  }
  *total = tot;
  return before + inc - v;
}

__device__ __forceinline__ uint64_t score_key(double s) {
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? 0ull : u;  // -0.0 (and negatives, which drift never yields) rank as +0
}

// EM: rows held per thread, the smallest of 4/8/16/32 that covers ceil(L/256).
template <int EM>
__global__ __launch_bounds__(SEL_T) void select_kernel(int L, int k, const double* __restrict__ score,
                                                       const uint8_t* __restrict__ forced,
                                                       const uint8_t* __restrict__ full,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ n_out) {
  __shared__ int hist[256];
  __shared__ int wsum[SEL_W];
  __shared__ int pick[3];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int E = (L + SEL_T - 1) / SEL_T;
  const int i0 = tid * E;
  const double* s = score + (size_t)b * L;
  const uint8_t* fr = forced ? forced + (size_t)b * L : nullptr;

  uint64_t key[EM];
  int cls[EM];  // 0 = candidate, 1 = forced, 2 = past the end
  int nf = 0, nz = 0;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int i = i0 + e;
    key[e] = 0;
    cls[e] = 2;
    if (e < E && i < L) {
      cls[e] = (fr && fr[i]) ? 1 : 0;
      key[e] = score_key(s[i]);
      nf += cls[e] == 1;
      nz += cls[e] == 0 && key[e] != 0;
    }
  }
  // forced rows (low 16 bits) and candidates of non-zero score (high bits),
  // both <= L <= 8192, in one scan
  int packed;
  (void)block_excl_scan(nf | (nz << 16), wsum, &packed);
  const int nF = packed & 0xFFFF, nnz = packed >> 16;
  const bool all_rows = full && full[b];
  const int keff = all_rows ? L : min(max(k, nF), L);
  const int need = keff - nF;       // rows to take by score
  const int ncand = L - nF;
  // mode: 0 none by score, 1 all candidates, 2 radix threshold
  const int mode = need <= 0 ? 0 : (need >= ncand ? 1 : 2);
  uint64_t thr = 0;
  int take_eq = 0;
  if (mode == 2 && need >= nnz) {
    // the cut falls among the zero scores (rows whose input did not change):
    // every non-zero candidate is taken, then zeros by index
    take_eq = need - nnz;
  } else if (mode == 2) {
    uint64_t prefix = 0, pmask = 0;
    int rem = need;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        // the leading digits of nearby scores mostly agree: when every
        // participating lane of the wave has the same digit, one lane adds the
        // count (LDS atomics to one address serialise)
        const bool part = cls[e] == 0 && (key[e] & pmask) == prefix;
        const int dg = (int)((key[e] >> shift) & 255);
        const unsigned long long bal = __ballot(part);
        if (bal == 0ull) continue;
        const int lead = __ffsll((long long)bal) - 1;
        const int d0 = __shfl(dg, lead, 64);
        if (__all(!part || dg == d0)) {
          if ((threadIdx.x & 63) == lead) atomicAdd(&hist[d0], __popcll(bal));
        } else if (part) {
          atomicAdd(&hist[dg], 1);
        }
      }
      __syncthreads();
      if (tid < 64) {
        int c[4], ls = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = hist[255 - (4 * tid + q)];
          ls += c[q];
        }
        int inc = ls;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(inc, o, 64);
          if (tid >= o) inc += t;
        }
        int acc = inc - ls;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (acc < rem && rem <= acc + c[q]) {
            pick[0] = 255 - (4 * tid + q);
            pick[1] = acc;
            pick[2] = rem == acc + c[q];  // the digit's rows are all taken: the cut is exact
          }
          acc += c[q];
        }
      }
      __syncthreads();
      const int digit = pick[0];
      const bool done = pick[2];
      rem -= pick[1];
      prefix |= (uint64_t)digit << shift;
      pmask |= 0xFFull << shift;
      __syncthreads();
      if (done) break;  // uniform: every thread read the same flag
    }
    thr = prefix;
    take_eq = rem;  // rows whose masked key equals thr to take, lowest index first
    // compare on the resolved high bits only: below the last pass every row
    // sharing the prefix is either all taken or ranked by index
#pragma unroll
    for (int e = 0; e < EM; ++e) key[e] &= pmask;
  }
  // rank of each equal-to-threshold candidate in index order
  int neq = 0;
  if (mode == 2) {
#pragma unroll
    for (int e = 0; e < EM; ++e) neq += (cls[e] == 0 && key[e] == thr);
  }
  int tot_eq;
  int eq_before = block_excl_scan(neq, wsum, &tot_eq);
  bool sel[EM];
  int nsel = 0;
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    bool v = false;
    if (cls[e] == 1) {
      v = true;
    } else if (cls[e] == 0) {
      if (mode == 1) {
        v = true;
      } else if (mode == 2) {
        if (key[e] > thr) v = true;
        else if (key[e] == thr) {
          v = eq_before < take_eq;
          ++eq_before;
        }
      }
    }
    sel[e] = v;
    nsel += v;
  }
  int total;
  int pos = block_excl_scan(nsel, wsum, &total);
  int32_t* out = idx + (size_t)b * L;
#pragma unroll
  for (int e = 0; e < EM; ++e)
    if (sel[e]) out[pos++] = i0 + e;
  if (tid == 0) n_out[b] = total;
}

hipError_t launch_select(hipStream_t st, int B, int L, int k, const double* score, const uint8_t* forced,
                         const uint8_t* full, int32_t* idx, int32_t* n) {
  if (L > SEL_T * SEL_EMAX) return hipErrorInvalidValue;
  if (L <= SEL_T * 4)
    hipLaunchKernelGGL(select_kernel<4>, dim3(B), dim3(SEL_T), 0, st, L, k, score, forced, full, idx, n);
  else if (L <= SEL_T * 8)
    hipLaunchKernelGGL(select_kernel<8>, dim3(B), dim3(SEL_T), 0, st, L, k, score, forced, full, idx, n);
  else if (L <= SEL_T * 16)
    hipLaunchKernelGGL(select_kernel<16>, dim3(B), dim3(SEL_T), 0, st, L, k, score, forced, full, idx, n);
  else
    hipLaunchKernelGGL(select_kernel<32>, dim3(B), dim3(SEL_T), 0, st, L, k, score, forced, full, idx, n);
  return hipGetLastError();
}

}  // namespace dllm
