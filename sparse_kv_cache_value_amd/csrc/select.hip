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
//
// Fused with the gather (one sequence, up to SG_MAX_ROWS rows): every
// workgroup of the gather grid runs the same selection for itself, then
// normalises the selected row at its own compact position m (workgroup 0 also
// writes the index list).  The selections are identical, so the launch of the
// selection kernel and its round trip through memory go away.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int SEL_T = 256;  // 4 waves: cheap barriers between the radix passes
constexpr int SEL_EMAX = 32;  // L <= 8192

// Exclusive prefix sum over the block (thread order); *total gets the sum.
template <int NW>
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
  for (int i = 0; i < NW; ++i) {
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

// The selection of one sequence by a workgroup of NT threads.  s and fr are
// the sequence's scores and forced flags (fr may be null); a set *full_flag
// (full_flag may be null) takes every row.  Thread t owns rows [i0, i0 + E), E = ceil(L / NT) <= EM.  On
// return sel[e] marks its selected rows, pos is the compact position of its
// first selected row and total the size of the set.  With m_exit >= 0 it
// returns false (uniformly, before any radix pass) when the set has at most
// m_exit rows.
template <int NT, int EM>
__device__ __forceinline__ bool select_rows(int L, int k, const double* __restrict__ s,
                                            const uint8_t* __restrict__ fr, const uint8_t* __restrict__ full_flag, int m_exit,
                                            int* hist, int* wsum, int* pick, int& i0, bool (&sel)[EM],
                                            int& pos, int& total) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int E = (L + NT - 1) / NT;
  i0 = tid * E;

  uint64_t key[EM];
  int cls[EM];  // 0 = candidate, 1 = forced, 2 = past the end
  int nf = 0, nz = 0;
  // every score and forced flag loaded unconditionally (index clamped), so
  // the loads are issued together rather than one round trip each
  // (without a forced list the flags are read from the scores' bytes, in
  // bounds, and ignored)
  const bool has_fr = fr != nullptr;
  const uint8_t* frp = has_fr ? fr : reinterpret_cast<const uint8_t*>(s);
  double sv[EM];
  uint8_t fv[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int ii = min(i0 + e, L - 1);
    sv[e] = s[ii];
    fv[e] = frp[ii];
  }
  // the full-pass flag (null: none), read with the scores
  const bool has_full = full_flag != nullptr;
  const uint8_t fullv = (has_full ? full_flag : frp)[0];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int i = i0 + e;
    key[e] = 0;
    cls[e] = 2;
    if (e < E && i < L) {
      cls[e] = (has_fr && fv[e]) ? 1 : 0;
      key[e] = score_key(sv[e]);
      nf += cls[e] == 1;
      nz += cls[e] == 0 && key[e] != 0;
    }
  }
  // forced rows (low 16 bits) and candidates of non-zero score (high bits),
  // both <= L <= 8192, in one scan
  int packed;
  (void)block_excl_scan<NW>(nf | (nz << 16), wsum, &packed);
  const int nF = packed & 0xFFFF, nnz = packed >> 16;
  const bool all_rows = has_full && fullv != 0;
  const int keff = all_rows ? L : min(max(k, nF), L);
  if (m_exit >= 0 && m_exit >= keff) return false;  // the set is keff rows
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
  int eq_before = block_excl_scan<NW>(neq, wsum, &tot_eq);
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
  pos = block_excl_scan<NW>(nsel, wsum, &total);
  return true;
}

// EM: rows held per thread, the smallest of 4/8/16/32 that covers ceil(L/256).
template <int EM>
__global__ __launch_bounds__(SEL_T) void select_kernel(int L, int k, const double* __restrict__ score,
                                                       const uint8_t* __restrict__ forced,
                                                       const uint8_t* __restrict__ full,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ n_out) {
  __shared__ int hist[256];
  __shared__ int wsum[SEL_T / 64];
  __shared__ int pick[3];
  const int b = blockIdx.x;
  int i0, pos, total;
  bool sel[EM];
  (void)select_rows<SEL_T, EM>(L, k, score + (size_t)b * L, forced ? forced + (size_t)b * L : nullptr,
                               full ? full + b : nullptr, -1, hist, wsum, pick, i0, sel, pos, total);
  int32_t* out = idx + (size_t)b * L;
#pragma unroll
  for (int e = 0; e < EM; ++e)
    if (sel[e]) out[pos++] = i0 + e;
  if (threadIdx.x == 0) n_out[b] = total;
}

// Selection of the one sequence fused with the gather: workgroup m selects,
// then normalises the selected row at compact position m into A (the same
// arithmetic as the gather kernel); workgroup 0 writes the index list and the
// count.  Workgroups past the set size stop after the first scan.
template <typename T, int EM>
__global__ __launch_bounds__(RT) void select_gather_kernel(int L, int d, float eps, int MTt, int k,
                                                           const double* __restrict__ score,
                                                           const uint8_t* __restrict__ forced,
                                                           const uint8_t* __restrict__ full,
                                                           const T* __restrict__ H, const float* __restrict__ g,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ n_out,
                                                           T* __restrict__ A) {
  __shared__ int hist[256];
  __shared__ int wsum[RT / 64];
  __shared__ int pick[3];
  __shared__ int row;
  __shared__ float red[RT / 64];
  const int m = blockIdx.x;
  int i0, pos, total;
  bool sel[EM];
  if (!select_rows<RT, EM>(L, k, score, forced, full, m == 0 ? -1 : m, hist, wsum, pick, i0, sel, pos,
                           total))
    return;
  int p = pos;
#pragma unroll
  for (int e = 0; e < EM; ++e)
    if (sel[e]) {
      if (m == 0) idx[p] = i0 + e;
      if (p == m) row = i0 + e;
      ++p;
    }
  if (m == 0 && threadIdx.x == 0) n_out[0] = total;
  if (m >= total) return;  // uniform: only workgroup 0 of an empty set
  __syncthreads();
  norm_row_store<T>(H + (size_t)row * d, d, eps, g, A, m, MTt, red);
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

hipError_t launch_select_gather(hipStream_t st, bool bf16m, int max_rows, int L, int d, float eps, int MTt, int k,
                                const double* score, const uint8_t* forced, const uint8_t* full, const void* H,
                                const float* g, int32_t* idx, int32_t* n, void* A) {
  if (max_rows < 1 || max_rows > SG_MAX_ROWS || L < 1 || L > RT * 16 || d > RT * 8 * RV || d % 8)
    return hipErrorInvalidValue;
#define SG_LAUNCH(T, EM)                                                                                     \
  hipLaunchKernelGGL((select_gather_kernel<T, EM>), dim3(max_rows), dim3(RT), 0, st, L, d, eps, MTt, k, score, \
                     forced, full, (const T*)H, g, idx, n, (T*)A)
#define SG_EM(T)                      \
  if (L <= RT * 2) SG_LAUNCH(T, 2);   \
  else if (L <= RT * 4) SG_LAUNCH(T, 4); \
  else if (L <= RT * 8) SG_LAUNCH(T, 8); \
  else SG_LAUNCH(T, 16)
  if (bf16m) {
    SG_EM(bf16);
  } else {
    SG_EM(float);
  }
#undef SG_EM
#undef SG_LAUNCH
  return hipGetLastError();
}

}  // namespace dllm
