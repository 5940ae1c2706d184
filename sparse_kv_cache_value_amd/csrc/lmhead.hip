// LM head statistics, the static-threshold commit and the entropy gate.
//
// EntropyCache (section 2): decode the new tokens from the logits and take
// the maximum entropy of their distributions, an O(V) quantity; if it exceeds
// tau the next step runs a full pass.  Parallel decoding with a static
// confidence threshold (Polestar section 1; TSPD/CE problem statement) commits
// every masked token whose top-1 probability clears the threshold.
//
// Per row the statistics are m = max z, the lowest argmax, S = sum e^{z-m} and
// T = sum e^{z-m}(z-m) (fp64); confidence = 1/S and entropy = ln S - T/S.
// Slabs of the vocabulary are reduced independently and merged in a fixed
// order, so the result does not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace dllm {

constexpr int LM_SLAB = 4096;

int lm_stats_slabs(int V) { return (V + LM_SLAB - 1) / LM_SLAB; }

// A[m] = bf16/f32( RMSNorm_fp64(H_N[b][block_start[b] + j]) * g ), m = b*blk + j.
template <typename T>
__global__ __launch_bounds__(256) void lm_gather_kernel(int B, int L, int blk, int d, float eps, int MTt,
                                                        const int32_t* __restrict__ block_start,
                                                        const T* __restrict__ H, const float* __restrict__ g,
                                                        T* __restrict__ A, int32_t* __restrict__ n_rows) {
  __shared__ double red[4];
  const int m = blockIdx.x;
  const int b = m / blk, j = m - b * blk;
  if (m == 0 && threadIdx.x == 0) n_rows[0] = B * blk;
  const int row = block_start[b] + j;
  if (block_start[b] >= L || row >= L) {
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c8 = threadIdx.x * 8; c8 < d; c8 += 256 * 8) store_a8(A, m, c8, MTt, d, z);
    return;
  }
  const T* x = H + ((size_t)b * L + row) * d;
  double ss = 0.0;
  for (int c = threadIdx.x; c < d; c += 256) {
    const double v = (double)io<T>::ld(x + c);
    ss += v * v;
  }
  ss = block_sum<4>(ss, red);
  const double den = sqrt(ss / (double)d + (double)eps);
  for (int c8 = threadIdx.x * 8; c8 < d; c8 += 256 * 8) {
    float v[8];
#pragma unroll
    for (int j2 = 0; j2 < 8; ++j2) v[j2] = (float)((double)io<T>::ld(x + c8 + j2) / den * (double)g[c8 + j2]);
    store_a8(A, m, c8, MTt, d, v);
  }
}

hipError_t launch_lm_gather(hipStream_t st, bool bf16m, int B, int L, int blk, int d, float eps, int MTt,
                            const int32_t* block_start, const void* H, const float* g, void* A, int32_t* n_rows) {
  if (bf16m)
    hipLaunchKernelGGL(lm_gather_kernel<bf16>, dim3(B * blk), dim3(256), 0, st, B, L, blk, d, eps, MTt, block_start,
                       (const bf16*)H, g, (bf16*)A, n_rows);
  else
    hipLaunchKernelGGL(lm_gather_kernel<float>, dim3(B * blk), dim3(256), 0, st, B, L, blk, d, eps, MTt, block_start,
                       (const float*)H, g, (float*)A, n_rows);
  return hipGetLastError();
}

// One (row, vocabulary slab): part[(m*S + sl)*4 + {0..3}] = {max, argmax, S, T}.
__global__ __launch_bounds__(256) void lm_slab_kernel(int V, int n_slabs, const float* __restrict__ logits,
                                                      double* __restrict__ part) {
  __shared__ float bv[4];
  __shared__ int bi[4];
  __shared__ double red[4];
  const int m = blockIdx.x, sl = blockIdx.y;
  const int c0 = sl * LM_SLAB, c1 = min(V, c0 + LM_SLAB);
  const float* z = logits + (size_t)m * V;
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  for (int c = c0 + threadIdx.x; c < c1; c += 256) {
    const float v = z[c];
    if (v > best) {  // columns visited in increasing order: keeps the lowest index
      best = v;
      bidx = c;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bidx, o, 64);
    if (ov > best || (ov == best && oi < bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    bv[w] = best;
    bi[w] = bidx;
  }
  __syncthreads();
  best = bv[0];
  bidx = bi[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (bv[i] > best || (bv[i] == best && bi[i] < bidx)) {
      best = bv[i];
      bidx = bi[i];
    }
  const double mx = (double)best;
  double s = 0.0, t = 0.0;
  for (int c = c0 + threadIdx.x; c < c1; c += 256) {
    const double dz = (double)z[c] - mx;
    const double e = exp(dz);
    s += e;
    t += e * dz;
  }
  s = block_sum<4>(s, red);
  t = block_sum<4>(t, red);
  if (threadIdx.x == 0) {
    double* p = part + ((size_t)m * n_slabs + sl) * 4;
    p[0] = mx;
    p[1] = (double)bidx;
    p[2] = s;
    p[3] = t;
  }
}

__global__ void lm_merge_kernel(int M, int n_slabs, const double* __restrict__ part, double* __restrict__ stats) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  const double* p = part + (size_t)m * n_slabs * 4;
  double mx = p[0], am = p[1];
  for (int s = 1; s < n_slabs; ++s)
    if (p[s * 4] > mx) {
      mx = p[s * 4];
      am = p[s * 4 + 1];
    }
  double S = 0.0, T = 0.0;
  for (int s = 0; s < n_slabs; ++s) {
    const double dm = p[s * 4] - mx;
    const double f = exp(dm);
    S += f * p[s * 4 + 2];
    T += f * (p[s * 4 + 3] + dm * p[s * 4 + 2]);
  }
  double* o = stats + (size_t)m * 4;
  o[0] = mx;
  o[1] = am;
  o[2] = S;
  o[3] = T;
}

// (max, argmax, S, T) of b merged into a, both relative to their own max;
// symmetric in a and b (floating-point addition commutes), so both lanes of a
// butterfly exchange end with the same bits.  A max of -inf marks no data.
__device__ __forceinline__ void lm_combine(double& mx, double& am, double& S, double& T, double omx, double oam,
                                           double oS, double oT) {
  if (omx == -INFINITY) return;
  if (mx == -INFINITY) {
    mx = omx;
    am = oam;
    S = oS;
    T = oT;
    return;
  }
  const double m = fmax(mx, omx);
  const double da = mx - m, db = omx - m;
  const double fa = exp(da), fb = exp(db);
  const double Sn = S * fa + oS * fb;
  const double Tn = (T + da * S) * fa + (oT + db * oS) * fb;
  if (omx > mx || (omx == mx && oam < am)) am = oam;
  mx = m;
  S = Sn;
  T = Tn;
}

__global__ __launch_bounds__(64) void lm_merge_wide_kernel(int n_slabs, const double* __restrict__ part,
                                                           double* __restrict__ stats) {
  const int m = blockIdx.x, lane = threadIdx.x;
  const double* p = part + (size_t)m * n_slabs * 4;
  double mx = -INFINITY, am = 0.0, S = 0.0, T = 0.0;
  for (int s = lane; s < n_slabs; s += 64) lm_combine(mx, am, S, T, p[s * 4], p[s * 4 + 1], p[s * 4 + 2], p[s * 4 + 3]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double omx = __shfl_xor(mx, o, 64), oam = __shfl_xor(am, o, 64);
    const double oS = __shfl_xor(S, o, 64), oT = __shfl_xor(T, o, 64);
    lm_combine(mx, am, S, T, omx, oam, oS, oT);
  }
  if (lane == 0) {
    double* out = stats + (size_t)m * 4;
    out[0] = mx;
    out[1] = am;
    out[2] = S;
    out[3] = T;
  }
}

hipError_t launch_lm_merge_wide(hipStream_t st, int M, int n_slabs, const double* part, double* stats) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(lm_merge_wide_kernel, dim3(M), dim3(64), 0, st, n_slabs, part, stats);
  return hipGetLastError();
}

hipError_t launch_lm_stats(hipStream_t st, int M, int V, const float* logits, double* part, double* stats,
                           int n_slabs) {
  hipLaunchKernelGGL(lm_slab_kernel, dim3(M, n_slabs), dim3(256), 0, st, V, n_slabs, logits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_merge_kernel, dim3((M + 63) / 64), dim3(64), 0, st, M, n_slabs, part, stats);
  return hipGetLastError();
}

// One wave per sequence; lane j is block row j.
__global__ __launch_bounds__(64) void commit_kernel(int L, int blk, double thr, double tau,
                                                    const double* __restrict__ stats, int32_t* __restrict__ tokens,
                                                    uint8_t* __restrict__ committed, int32_t* __restrict__ history,
                                                    int32_t* __restrict__ n_history, int32_t* __restrict__ n_new,
                                                    int32_t* __restrict__ block_start,
                                                    uint8_t* __restrict__ full_next,
                                                    double* __restrict__ max_entropy) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int bs = block_start[b];
  const int row = bs + lane;
  const bool valid = bs < L && lane < blk && row < L;
  uint8_t* cm = committed + (size_t)b * L;
  double conf = 0.0, ent = 0.0;
  int tok = 0;
  bool cand = false;
  if (valid) {
    const double* p = stats + ((size_t)b * blk + lane) * 4;
    conf = 1.0 / p[2];
    ent = log(p[2]) - p[3] / p[2];
    tok = (int)p[1];
    cand = cm[row] == 0;
  }
  bool pick = cand && conf >= thr;
  const uint64_t any_pick = __ballot(pick);
  const uint64_t any_cand = __ballot(cand);
  if (any_pick == 0 && any_cand != 0) {
    // most confident candidate, lowest position on ties
    double bc = cand ? conf : -1.0;
    int br = cand ? row : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double oc = __shfl_xor(bc, o, 64);
      const int orr = __shfl_xor(br, o, 64);
      if (oc > bc || (oc == bc && orr < br)) {
        bc = oc;
        br = orr;
      }
    }
    pick = cand && row == br;
  }
  const uint64_t mask = __ballot(pick);
  const int cnt = __popcll(mask);
  const int nh = n_history[b];
  if (pick) {
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    tokens[(size_t)b * L + row] = tok;
    cm[row] = 1;
    history[(size_t)b * L + nh + rank] = row;
  }
  double e = pick ? ent : 0.0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) e = fmax(e, __shfl_xor(e, o, 64));
  // block advance: the current block is now full iff every valid row is committed
  const bool done_row = !valid || !cand || pick;
  const uint64_t full_mask = __ballot(lane < blk ? done_row : true);
  int nbs = bs;
  if (bs < L && full_mask == ~0ull) {
    nbs = bs + blk;
    while (nbs < L) {
      bool c = true;
      for (int jj = lane; jj < blk; jj += 64) {
        const int rr = nbs + jj;
        if (rr < L && cm[rr] == 0) c = false;
      }
      if (__ballot(!c) != 0) break;
      nbs += blk;
    }
  }
  if (lane == 0) {
    n_history[b] = nh + cnt;
    n_new[b] = cnt;
    max_entropy[b] = e;
    full_next[b] = e > tau ? 1 : 0;
    block_start[b] = nbs;
  }
}

hipError_t launch_commit(hipStream_t st, int B, int L, int blk, double thr, double tau, const double* stats,
                         int32_t* tokens, uint8_t* committed, int32_t* history, int32_t* n_history, int32_t* n_new,
                         int32_t* block_start, uint8_t* full_next, double* max_entropy) {
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(64), 0, st, L, blk, thr, tau, stats, tokens, committed, history,
                     n_history, n_new, block_start, full_next, max_entropy);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Threshold commit with Confidence Extrapolation (TSPD + CE page, method
// section 2).  Lane j is block row j.  Each still-masked row's confidence
// feeds a constant-velocity Kalman filter (fp64; first observation: state
// (c, 0), covariance diag(r, p_v0); later: predict with
// F = [[1,1],[0,1]], Q = q [[1/4,1/2],[1/2,1]], then update with H = [1,0]
// and noise r).  A masked row commits at conf >= thr, or early when its
// left-context coverage (share of the block rows to its left committed
// before this step; 1 for the first row) is >= gamma and for some
// h = 1..horizon the forecast mean - kappa sd (covariance propagated h steps)
// is >= thr.  Fallback, history, entropy gate and block advance as in
// commit_kernel; the block's filter states are dropped when it advances.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void ce_commit_kernel(int L, int blk, double thr, double tau, int horizon, double q,
                                                       double r, double p_v0, double kappa, double gamma,
                                                       const double* __restrict__ stats, double* __restrict__ kf,
                                                       int32_t* __restrict__ has, int32_t* __restrict__ tokens,
                                                       uint8_t* __restrict__ committed, int32_t* __restrict__ history,
                                                       int32_t* __restrict__ n_history, int32_t* __restrict__ n_new,
                                                       int32_t* __restrict__ block_start,
                                                       uint8_t* __restrict__ full_next,
                                                       double* __restrict__ max_entropy) {
  // every product and sum rounded on its own, in the order written (no fused
  // multiply-add), as the filter equations are stated
#pragma clang fp contract(off)
  const int b = blockIdx.x, lane = threadIdx.x;
  const int bs = block_start[b];
  const int row = bs + lane;
  const bool valid = bs < L && lane < blk && row < L;
  uint8_t* cm = committed + (size_t)b * L;
  double conf = 0.0, ent = 0.0;
  int tok = 0;
  bool cand = false;
  if (valid) {
    const double* p = stats + ((size_t)b * blk + lane) * 4;
    conf = 1.0 / p[2];
    ent = log(p[2]) - p[3] / p[2];
    tok = (int)p[1];
    cand = cm[row] == 0;
  }
  // filter update of the masked rows
  double* ks = kf + ((size_t)b * blk + lane) * 5;
  int32_t* hs = has + (size_t)b * blk + lane;
  double x0 = 0.0, x1 = 0.0, a = 0.0, bb = 0.0, d = 0.0;
  if (cand) {
    if (*hs == 0) {
      x0 = conf;
      x1 = 0.0;
      a = r;
      bb = 0.0;
      d = p_v0;
    } else {
      x0 = ks[0];
      x1 = ks[1];
      a = ks[2];
      bb = ks[3];
      d = ks[4];
      // predict
      x0 = x0 + x1;
      a = a + 2.0 * bb + d + q / 4.0;
      bb = bb + d + q / 2.0;
      d = d + q;
      // update
      const double S = a + r;
      const double k0 = a / S, k1 = bb / S;
      const double y = conf - x0;
      x0 = x0 + k0 * y;
      x1 = x1 + k1 * y;
      const double a2 = a - k0 * a, b2 = bb - k0 * bb, d2 = d - k1 * bb;
      a = a2;
      bb = b2;
      d = d2;
    }
    ks[0] = x0;
    ks[1] = x1;
    ks[2] = a;
    ks[3] = bb;
    ks[4] = d;
    *hs = 1;
  }
  // left-context coverage from the rows committed before this step
  const uint64_t before = __ballot(valid && !cand);
  const int left = __popcll(before & ((1ull << lane) - 1ull));
  const double coverage = lane == 0 ? 1.0 : (double)left / (double)lane;
  bool pick = false;
  if (cand) {
    if (conf >= thr) {
      pick = true;
    } else if (coverage >= gamma) {
      double pa = a, pb = bb, pd = d;
      for (int h = 1; h <= horizon; ++h) {
        const double na = pa + 2.0 * pb + pd + q / 4.0, nb = pb + pd + q / 2.0, nd = pd + q;
        pa = na;
        pb = nb;
        pd = nd;
        if (x0 + (double)h * x1 - kappa * sqrt(pa) >= thr) pick = true;
      }
    }
  }
  const uint64_t any_pick = __ballot(pick);
  const uint64_t any_cand = __ballot(cand);
  if (any_pick == 0 && any_cand != 0) {
    double bc = cand ? conf : -1.0;
    int br = cand ? row : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double oc = __shfl_xor(bc, o, 64);
      const int orr = __shfl_xor(br, o, 64);
      if (oc > bc || (oc == bc && orr < br)) {
        bc = oc;
        br = orr;
      }
    }
    pick = cand && row == br;
  }
  const uint64_t mask = __ballot(pick);
  const int cnt = __popcll(mask);
  const int nh = n_history[b];
  if (pick) {
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    tokens[(size_t)b * L + row] = tok;
    cm[row] = 1;
    history[(size_t)b * L + nh + rank] = row;
  }
  double e = pick ? ent : 0.0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) e = fmax(e, __shfl_xor(e, o, 64));
  const bool done_row = !valid || !cand || pick;
  const uint64_t full_mask = __ballot(lane < blk ? done_row : true);
  int nbs = bs;
  if (bs < L && full_mask == ~0ull) {
    nbs = bs + blk;
    while (nbs < L) {
      bool c = true;
      for (int jj = lane; jj < blk; jj += 64) {
        const int rr = nbs + jj;
        if (rr < L && cm[rr] == 0) c = false;
      }
      if (__ballot(!c) != 0) break;
      nbs += blk;
    }
  }
  if (nbs != bs && lane < blk) *hs = 0;  // the block's filter states end with it
  if (lane == 0) {
    n_history[b] = nh + cnt;
    n_new[b] = cnt;
    max_entropy[b] = e;
    full_next[b] = e > tau ? 1 : 0;
    block_start[b] = nbs;
  }
}

hipError_t launch_ce_commit(hipStream_t st, int B, int L, int blk, double thr, double tau, int horizon, double q,
                            double r, double p_v0, double kappa, double gamma, const double* stats, double* kf,
                            int32_t* has, int32_t* tokens, uint8_t* committed, int32_t* history, int32_t* n_history,
                            int32_t* n_new, int32_t* block_start, uint8_t* full_next, double* max_entropy) {
  if (blk > 64 || horizon < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ce_commit_kernel, dim3(B), dim3(64), 0, st, L, blk, thr, tau, horizon, q, r, p_v0, kappa, gamma,
                     stats, kf, has, tokens, committed, history, n_history, n_new, block_start, full_next,
                     max_entropy);
  return hipGetLastError();
}

// out = {sequences run full, tokens committed, sequences still active, 0} then the max entropy.
__global__ void step_result_kernel(int B, int L, const uint8_t* __restrict__ step_full,
                                   const int32_t* __restrict__ n_new, const int32_t* __restrict__ block_start,
                                   const double* __restrict__ max_entropy, int32_t* __restrict__ out) {
  if (threadIdx.x != 0) return;
  int nf = 0, nc = 0, na = 0;
  double me = 0.0;
  for (int b = 0; b < B; ++b) {
    nf += step_full ? step_full[b] : 0;
    nc += n_new[b];
    na += block_start[b] < L;
    me = fmax(me, max_entropy[b]);
  }
  out[0] = nf;
  out[1] = nc;
  out[2] = na;
  out[3] = 0;
  *reinterpret_cast<double*>(out + 4) = me;
}

hipError_t launch_step_result(hipStream_t st, int B, const uint8_t* step_full, const int32_t* n_new,
                              const int32_t* block_start, const double* max_entropy, int L, void* out) {
  hipLaunchKernelGGL(step_result_kernel, dim3(1), dim3(64), 0, st, B, L, step_full, n_new, block_start,
                     max_entropy, (int32_t*)out);
  return hipGetLastError();
}

}  // namespace dllm
