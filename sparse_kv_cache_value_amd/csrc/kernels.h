// Host-side launchers of the libdllm kernels.  Every launcher enqueues on
// `st` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dllm {

// ---- row bookkeeping (rows.hip) ----
// forced set + layer-0 changed rows + per-sequence full flags of this step.
// mode: 0 auto (full_next), 1 full, 2 sparse.
hipError_t launch_prep(hipStream_t st, int B, int L, int block_len, int rule, int recent_k, int mode,
                       const int32_t* history, const int32_t* n_history, const int32_t* n_new,
                       const int32_t* block_start, const uint8_t* full_next, uint8_t* forced,
                       uint8_t* step_full, int32_t* idx0, int32_t* n0);
hipError_t launch_forced(hipStream_t st, int B, int L, int block_len, int rule, int recent_k,
                         const int32_t* history, const int32_t* n_history, const int32_t* block_start,
                         uint8_t* forced);
hipError_t launch_all_rows(hipStream_t st, int B, int L, int32_t* idx, int32_t* n);
hipError_t launch_embed(hipStream_t st, bool bf16, int max_rows, int B, int L, int d, int V,
                        const int32_t* idx, const int32_t* n, const int32_t* tokens, const void* embed,
                        void* h0);
// A[m] = RMSNorm(H[row m]) * g  (fp32 statistics), rows from idx/n.
hipError_t launch_gather_norm(hipStream_t st, bool bf16, int max_rows, int B, int L, int d, float eps, int MTt,
                              const int32_t* idx, const int32_t* n, const void* H, const float* g,
                              void* A);
// q/k RoPE + K/V scatter from QKV partials [S][max_rows][nq + 2 nv].
hipError_t launch_qkv_epilogue(hipStream_t st, bool bf16, int max_rows, int B, int L, int Hq, int Hkv,
                               int dh, int S, const int32_t* idx, const int32_t* n, const float* part,
                               const float* rope_cos, const float* rope_sin, void* q_out, void* Kc,
                               void* Vc);
// h' = x + sum_s part; A2 = RMSNorm(h') * g2.
hipError_t launch_o_epilogue(hipStream_t st, bool bf16, int max_rows, int B, int L, int d, int S,
                             float eps, int MTt, const int32_t* idx, const int32_t* n, const float* part,
                             const void* H, const float* g2, float* hprime, void* A2);
// act = SiLU(gate) * up from fp32 gate|up partials interleaved by 32 columns.
hipError_t launch_swiglu(hipStream_t st, bool bf16, int max_rows, int B, int F, int S, const int32_t* n,
                         const float* part, void* act);
// H_out[row] = h' + sum_s part; proxy_ref[row] = proxy_cur[row]; score[row] = 0.
hipError_t launch_down_epilogue(hipStream_t st, bool bf16, int max_rows, int B, int L, int d, int r,
                                int S, const int32_t* idx, const int32_t* n, const float* part,
                                const float* hprime, void* H_out, const double* pcur, double* pref,
                                double* score);

// ---- proxy and drift (proxy.hip) ----
// Capacity of the split partial buffer needed for max_rows rows (doubles).
size_t proxy_partial_doubles(int max_rows, int d, int r);
// Stored basis width: r rounded up to 32, 64 or 128.
int proxy_rpad(int r);
// C[row] = (H[row] * g1) W_r and score[row] = drift(C, proxy_ref[row]) for the
// listed rows; wr is the padded fp32 basis [d][proxy_rpad(r)].
hipError_t launch_proxy_drift(hipStream_t st, bool bf16, int max_rows, int B, int L, int d, int r,
                              const int32_t* idx, const int32_t* n, const void* H, const float* g1,
                              const float* wr, double* partial, double* pcur, const double* pref, double* score);
// out[d][rpad] = W_r [d][r] with zero columns appended.
hipError_t launch_pad_proxy(hipStream_t st, int d, int r, const float* wr, float* out);

// ---- selection (select.hip) ----
hipError_t launch_select(hipStream_t st, int B, int L, int k, const double* score, const uint8_t* forced,
                         const uint8_t* full, int32_t* idx, int32_t* n);
// One sequence: the selection fused with the gather + RMSNorm of the selected
// rows into compact A (as launch_gather_norm with B = 1); grid max_rows
// workgroups, each running the selection itself, so max_rows is kept small.
constexpr int SG_MAX_ROWS = 512;
hipError_t launch_select_gather(hipStream_t st, bool bf16, int max_rows, int L, int d, float eps, int MTt, int k,
                                const double* score, const uint8_t* forced, const uint8_t* full, const void* H,
                                const float* g, int32_t* idx, int32_t* n, void* A);

// ---- GEMMs (gemm.hip) ----
// Optional event pair stamped by the GEMM launch itself (hipExtLaunchKernel:
// the kernel's own begin and end, no marker packets around it); diagnostics.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
// out[s][m][n] = sum_{k in split s} A[m][k] W[k][n] for m < sum(n_sel).
hipError_t launch_gemm_f32(hipStream_t st, int max_rows, int B, int K, int N, const float* A,
                           const float* W, const int32_t* n_sel, float* out, LaunchEvents ev = {});
// bf16 weights pre-packed by launch_pack_bf16; `splits` from gemm_bf16_pick_splits,
// `cols` (column tiles per workgroup: 4, or 3 at 384-row blocks) from gemm_bf16_pick_cols.
// A is packed (apack_off) with MTt row tiles.  act != NULL (one split, N a
// multiple of 64, each 32-column tile holding 16 gate then the matching 16 up
// columns) writes SwiGLU(gate, up) as a packed bf16 [M][N/2] activation with
// MTt_out row tiles instead of out.
hipError_t launch_gemm_bf16(hipStream_t st, int max_rows, int B, int K, int N, const uint16_t* A, int MTt,
                            const uint16_t* Wp, const int32_t* n_sel, float* out, int splits, uint16_t* act,
                            int MTt_out, int cols, LaunchEvents ev = {});
int gemm_bf16_pick_splits(int max_rows, int K, int N, int n_cu);
int gemm_bf16_pick_cols(int max_rows, int K, int N, int n_cu, int splits);
// Streaming variant for up to 288 rows (N % 128 == 0, K % 256 == 0); `splits`
// from gemm_stream_pick_splits (0 there = use launch_gemm_bf16).
int gemm_stream_pick_splits(int max_rows, int K, int N, int n_cu, bool fused, int MTt);
hipError_t launch_gemm_stream(hipStream_t st, int max_rows, int B, int K, int N, const uint16_t* A, int MTt,
                              const uint16_t* Wp, const int32_t* n_sel, float* out, int splits, uint16_t* act,
                              int MTt_out, LaunchEvents ev = {});
// The same on 96-column slabs (three column tiles per workgroup, the fourth
// wave sharing only the activation DMA), for up to three row tiles and where
// they fill more of the chip (N a multiple of 96): the split count, or 0 to
// use launch_gemm_stream.
int gemm_stream3_pick_splits(int max_rows, int K, int N, int n_cu, bool fused, int MTt);
hipError_t launch_gemm_stream3(hipStream_t st, int max_rows, int B, int K, int N, const uint16_t* A, int MTt,
                               const uint16_t* Wp, const int32_t* n_sel, float* out, int splits, uint16_t* act,
                               int MTt_out, LaunchEvents ev = {});
// The LM head on up to 288 rows without logits: per row and 128-column slab
// (max, lowest argmax, S, T) into part [rows][N/128][4] (fp64); merge with
// launch_lm_merge_wide.
hipError_t launch_gemm_stream_stats(hipStream_t st, int max_rows, int K, int N, const uint16_t* A, int MTt,
                                    const uint16_t* Wp, const int32_t* n_sel, double* part, LaunchEvents ev = {});
// Padding (elements) a packed buffer needs past its end: for weights pass 1,
// for packed activations the buffer's row-tile count.
size_t gemm_pad_elems(int rows_tiles);
// Pack source columns [0, Nsrc) of a row-major [K][ld_src] weight: source
// column group t (gw columns: 32, or 16 for bf16) lands at packed column
// col0 + t*tile_stride.  bf16: MFMA B-fragment tiles; fp32: row-major [K][Ndst].
hipError_t launch_pack_bf16(hipStream_t st, int K, int Nsrc, const uint16_t* src, int ld_src, uint16_t* dst,
                            int col0, int tile_stride, int gw = 32);
hipError_t launch_pack_f32(hipStream_t st, int K, int Nsrc, const float* src, int ld_src, float* dst, int Ndst,
                           int col0, int tile_stride);

// ---- attention (attn.hip) ----
// out: the GEMM input of the output projection ([M][Hq*dh], packed for bf16
// with MTt row tiles).
hipError_t launch_attention(hipStream_t st, bool bf16, int max_rows, int B, int L, int Hq, int Hkv, int dh,
                            const int32_t* idx, const int32_t* n, const void* q, const void* Kc,
                            const void* Vc, void* out, int MTt);

// ---- LM head and commit (lmhead.hip) ----
hipError_t launch_lm_gather(hipStream_t st, bool bf16, int B, int L, int blk, int d, float eps, int MTt,
                            const int32_t* block_start, const void* H, const float* g, void* A,
                            int32_t* n_rows);
hipError_t launch_lm_stats(hipStream_t st, int M, int V, const float* logits, double* part,
                           double* stats, int n_slabs);
int lm_stats_slabs(int V);
// Merge of per-slab statistics part [M][n_slabs][4] into stats [M][4] (one
// wave per row, fixed order).
hipError_t launch_lm_merge_wide(hipStream_t st, int M, int n_slabs, const double* part, double* stats);
hipError_t launch_commit(hipStream_t st, int B, int L, int blk, double thr, double tau,
                         const double* stats, int32_t* tokens, uint8_t* committed, int32_t* history,
                         int32_t* n_history, int32_t* n_new, int32_t* block_start, uint8_t* full_next,
                         double* max_entropy);
// Threshold commit with Confidence Extrapolation; kf [B][blk][5], has [B][blk].
hipError_t launch_ce_commit(hipStream_t st, int B, int L, int blk, double thr, double tau, int horizon, double q,
                            double r, double p_v0, double kappa, double gamma, const double* stats, double* kf,
                            int32_t* has, int32_t* tokens, uint8_t* committed, int32_t* history, int32_t* n_history,
                            int32_t* n_new, int32_t* block_start, uint8_t* full_next, double* max_entropy);
// out: {n_full, n_committed, n_active, pad} int32 then max entropy as double (24 bytes).
hipError_t launch_step_result(hipStream_t st, int B, const uint8_t* step_full, const int32_t* n_new,
                              const int32_t* block_start, const double* max_entropy, int L, void* out);

// ---- Polestar-Cache drift path (polestar.hip) ----
// R: Gram split partials [B][ps_gram_splits()][W][W], added by the k-means.
int ps_gram_splits();
hipError_t launch_ps_gram(hipStream_t st, bool bf16, int B, int L, int d, int blk, int W, const int32_t* bstart,
                          const void* H, double* R);
hipError_t launch_ps_kmeans(hipStream_t st, int B, int W, int K, int iters, const double* R, int32_t* assign,
                            double* norms, double* coef, int32_t* nsel);
hipError_t launch_ps_centroids(hipStream_t st, bool bf16, int B, int L, int d, int blk, int W, int K, float eps,
                               int MTt, const int32_t* bstart, const void* H, const double* coef,
                               const double* norms, const float* g1, double* cent, void* A);
hipError_t launch_ps_codes(hipStream_t st, bool bf16, int B, int L, int d, int blk, int W, int K,
                           const int32_t* bstart, const void* H, const double* norms, const int32_t* assign,
                           const double* cent, uint8_t* codes, uint8_t* scales);
hipError_t launch_ps_queries(hipStream_t st, bool bf16, int B, int L, int blk, int W, int K, int Hq, int dh, int S,
                             int ldp, const int32_t* bstart, const float* part, const float* rc, const float* rs,
                             void* q);
// logA is replaced only for sequences whose drift refresh is due (tau_upd,
// the layer's window start and n_history at its last refresh).
hipError_t launch_ps_attn_kl(hipStream_t st, bool bf16, int B, int L, int blk, int W, int K, int Hq, int Hkv,
                             int dh, const int32_t* bstart, const void* q, const void* Kc, double* logA, double* klp,
                             int tau_upd, const int32_t* wstart, const int32_t* n_hist, const int32_t* upd_hist);
hipError_t launch_ps_select(hipStream_t st, int B, int L, int blk, int W, int K, int Hq, int top,
                            const int32_t* bstart, const int32_t* assign, const double* klp, int32_t* wstart,
                            double* kl, int32_t* top_out, int32_t* idx, int32_t* n, int32_t* valid, int tau_upd,
                            const int32_t* n_hist, int32_t* upd_hist);
// Polestar-Commit; stats [B][2 blk][4] (current and next block), blk <= 64.
hipError_t launch_ps_commit(hipStream_t st, int B, int L, int blk, int W, int K, int top, double thr, double alpha,
                            double tau, const double* stats, const double* kl, const int32_t* assign,
                            const int32_t* top_c, int32_t* drift_valid, double* dsum, int32_t* dcnt,
                            int32_t* tokens, uint8_t* committed, int32_t* history, int32_t* n_history,
                            int32_t* n_new, int32_t* block_start, uint8_t* full_next, double* max_entropy);

// ---- proxy basis derivation (basis.hip) ----
// Subspace width p (r + oversampling, even, <= 136) and the fp64 workspace
// launch_proxy_basis needs.
int proxy_basis_width(int d, int nv, int r);
size_t proxy_basis_workspace_doubles(int d, int nv, int r);
// Allocation-free derivation: a fixed device array per device of this many
// workspace doubles (32 MiB; every shape with d, nv <= 8192 and r <= 128
// fits), then 32 more doubles whose first word is the status.
constexpr size_t PROXY_BASIS_STATIC_DOUBLES = (size_t)4 << 20;
// Looks the array's device address up on device `dev` (which must be
// current) once; later calls return at once.
hipError_t proxy_basis_static_setup(int dev);
// The address for `dev`, or NULL before its set-up.
double* proxy_basis_static_ws(int dev);
// wr [d][r] fp64 = U_r S_r of W [d][nv] (storage dtype) by randomised
// subspace iteration (iters power steps) and Rayleigh-Ritz; status[0] is set
// to 1 when a Cholesky pivot was not positive (rank-deficient subspace).
hipError_t launch_proxy_basis(hipStream_t st, bool bf16, int d, int nv, int r, int iters, const void* W, double* wr,
                              double* ws, int32_t* status);
hipError_t launch_f64_to_f32(hipStream_t st, size_t n, const double* src, float* dst);

// ---- diagnostics (probe.hip) ----
// bytes must be a positive multiple of stream_probe_quantum(grid, depth);
// depth is 4 or 8 loads of 16 bytes in flight per thread; out holds grid words.
size_t stream_probe_quantum(int grid, int depth);
hipError_t launch_stream_probe(hipStream_t st, int grid, int depth, const void* buf, size_t bytes, unsigned* out);

}  // namespace dllm
