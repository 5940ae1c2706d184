/*
 * libdllm -- one denoising step of a bidirectional diffusion LLM under
 * approximate KV caching, on one MI355X (gfx950).
 *
 * The step has four parts, each an entry point below:
 *   1. a cheap per-token drift score      (dllm_drift_score, dllm_commit's entropy gate)
 *   2. a per-layer budgeted selection      (dllm_select)
 *   3. a sparse forward on the selection   (dllm_sparse_layer)
 *   4. LM-head statistics and the commit   (dllm_lm_head, dllm_commit)
 * and dllm_step runs all of them for every layer.
 *
 * Sources (four summary pages):
 *   SPA-Cache -- "Singular proxy for adaptive caching in diffusion language
 *     models": step 1 (value proxy from the truncated SVD of W_V, cosine
 *     against the cached proxy, lowest similarity refreshed), step 2 (per-layer
 *     update ratio rho(l), piecewise Gaussian), step 3 (sparse execution on I).
 *   EntropyCache summary, section 2: the maximum entropy of the tokens decoded
 *     in a step decides whether the next step runs a full pass; otherwise the
 *     current mask block and the k most recently decoded tokens are recomputed.
 *   Polestar, section 1 / TSPD-CE, problem statement: parallel decoding commits
 *     every masked token whose confidence clears a static threshold.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE memory unless the name ends in _h (host memory).
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the null stream).  Only dllm_step with a non-NULL result pointer, and
 *     dllm_step in DLLM_MODE_AUTO, wait on the stream.
 *   - Matrices are row-major; weight matrices are [in][out] (y = x W).
 *   - Activations, weights, the hidden-state cache and the K/V cache use the
 *     model dtype (DLLM_FP32 or DLLM_BF16); norm gains and the proxy basis are
 *     fp32; proxies and drift scores are fp64; token ids and indices int32.
 *   - Every function validates its arguments before enqueuing anything and
 *     returns a dllm_status; on failure dllm_last_error() describes it.  A HIP
 *     failure returns DLLM_E_HIP.  After a failure inside a step the state
 *     contents are unspecified.
 *   - One model serves one stream at a time (its workspace is shared).
 */
#ifndef LIBDLLM_H
#define LIBDLLM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dllm_model dllm_model; /* opaque; owned by the library */
typedef int32_t dllm_status;

enum {
  DLLM_OK = 0,
  DLLM_E_ARG = -1,         /* NULL or out-of-range argument */
  DLLM_E_SHAPE = -2,       /* dimensions the library cannot handle */
  DLLM_E_STATE = -3,       /* call order violated (e.g. layer weights missing) */
  DLLM_E_NOMEM = -4,       /* device allocation failed */
  DLLM_E_HIP = -5,         /* a HIP runtime call failed */
  DLLM_E_UNSUPPORTED = -6, /* feature not built */
  DLLM_E_NUMERIC = -7      /* a factorisation broke down (dllm_derive_proxy_basis) */
};
enum { DLLM_FP32 = 0, DLLM_BF16 = 1 };
enum { DLLM_MODE_AUTO = 0, DLLM_MODE_FULL = 1, DLLM_MODE_SPARSE = 2 };
enum { DLLM_FORCED_NONE = 0, DLLM_FORCED_BLOCK = 1, DLLM_FORCED_BLOCK_RECENT = 2 };

/* Model and sequence dimensions.  Limits checked by dllm_create:
 * head_dim a multiple of 32 and <= 256; d_model <= 8192 and a multiple of 32;
 * d_ffn a multiple of 32; n_q_heads a multiple of n_kv_heads;
 * seq_len <= 8192 and a multiple of 4; block_len <= 64; proxy_rank <= 128 and
 * <= d_model; for DLLM_BF16 also d_model, d_ffn and n_q_heads*head_dim
 * multiples of 64, n_kv_heads*head_dim and vocab multiples of 32. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
  int32_t max_batch, seq_len, block_len, proxy_rank, dtype;
  float rms_eps;    /* RMSNorm epsilon (1e-5) */
  float rope_theta; /* rotary base (1e4) */
} dllm_dims;

/* One layer's weights (device pointers, model dtype unless noted).  The layer
 * is h' = x + Attn(RMSNorm(x) * attn_norm) W_o,
 *       out = h' + (SiLU(n W_gate) * (n W_up)) W_down,  n = RMSNorm(h') * ffn_norm,
 * attention bidirectional (no mask) with rotate-half RoPE on q and k. */
typedef struct {
  const float *attn_norm; /* [d_model] fp32 */
  const void *w_q;        /* [d_model][n_q_heads*head_dim] */
  const void *w_k;        /* [d_model][n_kv_heads*head_dim] */
  const void *w_v;        /* [d_model][n_kv_heads*head_dim] */
  const void *w_o;        /* [n_q_heads*head_dim][d_model] */
  const float *ffn_norm;  /* [d_model] fp32 */
  const void *w_gate;     /* [d_model][d_ffn] */
  const void *w_up;       /* [d_model][d_ffn] */
  const void *w_down;     /* [d_ffn][d_model] */
  /* SPA-Cache step 1: W_r = U_r S_r, the top-r left singular vectors of W_v
   * scaled by their singular values, [d_model][proxy_rank] fp32.  NULL: the
   * library derives it from w_v (dllm_derive_proxy_basis, DLLM_PROXY_ITERS). */
  const float *w_proxy;
} dllm_layer_weights;

/* Caller-owned decode state (e.g. torch tensors); B = batch <= max_batch,
 * L = seq_len, N = n_layers, r = proxy_rank.  Everything a step reads or
 * writes lives here, so a copy of these buffers is a checkpoint. */
typedef struct {
  void *hidden;         /* [N+1][B][L][d_model]: slot 0 = embeddings, slot l+1 = layer l output */
  void *k_cache;        /* [N][B][n_kv_heads][L32/32][head_dim/16][64][8] post-RoPE keys in
                         * matrix-core fragment order, L32 = L rounded up to 32: key j,
                         * dimension t at [j/32][t/16][j%32 + 32*((t/8)%2)][t%8] */
  void *v_cache;        /* [N][B][n_kv_heads][L32][head_dim] values, row-major: key j,
                         * dimension t at [j][t] */
  double *proxy_cur;    /* [N][B][L][r]  current proxy C of each row's layer input */
  double *proxy_ref;    /* [N][B][L][r]  proxy P at the row's last refresh */
  double *score;        /* [N][B][L]     drift of C against P (0 for refreshed rows) */
  int32_t *tokens;      /* [B][L]  token ids (masked rows hold the mask id) */
  uint8_t *committed;   /* [B][L]  1 = prompt or committed token */
  int32_t *history;     /* [B][L]  decode history: committed positions in commit order */
  int32_t *n_history;   /* [B] */
  int32_t *n_new;       /* [B]  commits made by the last commit (the tail of history) */
  int32_t *block_start; /* [B]  first row of the current block (>= L when done) */
  uint8_t *full_next;   /* [B]  entropy gate: 1 = the next step runs a full pass */
  double *max_entropy;  /* [B]  max entropy (nats) over the last commit's tokens */
  int32_t batch;
} dllm_state;

/* Drift score used by dllm_step's sparse refresh. */
enum { DLLM_SCORE_SPA_COS = 0,       /* SPA-Cache value-proxy cosine + top-k (SPA-Cache, method steps 1-2) */
       DLLM_SCORE_POLESTAR_KL = 1 }; /* Polestar-Cache cluster KL (Polestar, section 2A) */

/* Polestar-Cache drift path parameters.  Window W = window_blocks * block_len
 * rows (<= 120 and <= seq_len); n_clusters <= 16 and <= W; d_model % 128 == 0;
 * head_dim <= 128.  Other shapes return DLLM_E_SHAPE or DLLM_E_UNSUPPORTED. */
typedef struct {
  int32_t n_clusters;    /* spherical k-means clusters (16) */
  int32_t kmeans_iters;  /* assign/update iterations before the final assignment (10) */
  int32_t top_clusters;  /* clusters refreshed per layer and step (4), <= n_clusters */
  int32_t window_blocks; /* prefix, current and suffix block: 3 */
  int32_t drift_commit;  /* 1: dllm_step commits with Polestar-Commit (dllm_polestar_commit);
                            0: the static threshold commit */
  double commit_alpha;   /* Polestar-Commit alpha (>= 0; +inf disables the drift rule) */
  int32_t tau_upd;       /* schedule: a layer's drift refresh runs on a window's first step or once
                            this many tokens were decoded since its last one (0: every step);
                            otherwise the step refreshes only the current block */
  int32_t full_period;   /* schedule: dllm_step in AUTO mode runs a full pass every this many steps
                            (0: never) */
} dllm_polestar_params;

/* Caller-owned Polestar state (K = n_clusters, Hq = n_q_heads, W as above).
 * log_attn/win_start persist across steps; the rest describes the last layer
 * processed (for inspection; codes/scales are the compressed proxy that the
 * Polestar page keeps in host memory, not consumed by the step). */
typedef struct {
  double *log_attn;      /* [N][B][K][Hq][W] proxy log-attention of the previous step, per layer */
  int32_t *win_start;    /* [N][B] window that log_attn belongs to; -1 = none (initialise to -1) */
  double *centroids;     /* [B][K][d_model] unit centroids (fp64) */
  double *norms;         /* [B][W] Euclidean norm of each window row's layer input */
  int32_t *assign;       /* [B][W] cluster of each window row */
  uint8_t *codes;        /* [B][W][d_model/2] E2M1 residual codes, element 2i in the low nibble */
  uint8_t *scales;       /* [B][W][d_model/16] E4M3 (FN) scale per 16 elements */
  void *queries;         /* [B][K][n_q_heads*head_dim] centroid queries (storage dtype) */
  double *kl;            /* [B][K] cluster drift (mean over heads of KL(A_t || A_t-1)) */
  int32_t *top;          /* [B][top_clusters] refreshed clusters, ascending */
  /* Polestar-Commit (initialise to zero): */
  double *drift_sum;     /* [B][block_len] sum of the current block rows' drifts at earlier steps */
  int32_t *drift_cnt;    /* [B][block_len] number of drifts in drift_sum */
  int32_t *drift_valid;  /* [B] 1 when the last dllm_polestar_select found the cluster drift
                            defined (window unchanged); the Polestar commit clears it */
  int32_t *upd_hist;     /* [N][B] state.n_history at the layer's last drift refresh (initialise to 0) */
  int32_t steps_since_full; /* host value: steps since the last full pass (dllm_step keeps it) */
} dllm_polestar_state;

/* Confidence Extrapolation (TSPD + CE page, method section 2) on top of the
 * threshold commit: a constant-velocity Kalman filter (fp64) on each masked
 * current-block row's top-1 confidence, state (level, velocity), transition
 * [[1,1],[0,1]] per step, process noise q [[1/4,1/2],[1/2,1]], observation
 * noise r; first observation: state (c, 0), covariance diag(r, p_v0).  A
 * masked row commits early when its left-context coverage (share of the
 * block rows to its left committed before this step; 1 for the block's first
 * row) is >= gamma and, for some h in 1..horizon, the forecast level minus
 * kappa standard deviations is >= the commit threshold. */
typedef struct {
  int32_t horizon;       /* look-ahead steps H, 1..64 */
  double q;              /* process noise scale (>= 0) */
  double r;              /* observation noise variance (> 0) */
  double p_v0;           /* initial velocity variance (>= 0) */
  double kappa;          /* lower bound = mean - kappa * sd (>= 0, +inf: no early commit) */
  double gamma;          /* minimum left-context coverage */
} dllm_ce_params;

/* Caller-owned filter state of the current block's rows (initialise to zero;
 * a block's states are dropped when it advances). */
typedef struct {
  double *kf;            /* [B][block_len][5] level, velocity, P00, P01, P11 */
  int32_t *has;          /* [B][block_len] 1 when kf holds a state */
} dllm_ce_state;

typedef struct {
  int32_t mode;          /* DLLM_MODE_*; AUTO reads state.full_next (one host wait) */
  int32_t forced_rule;   /* DLLM_FORCED_* */
  int32_t recent_k;      /* EntropyCache k: recent decoded tokens always refreshed */
  double tau;            /* entropy gate threshold in nats (+inf: never full) */
  double conf_threshold; /* commit threshold on the top-1 probability */
  const double *rho_h;   /* [n_layers] host: per-layer update ratio rho(l) (SPA score) */
  int32_t score;         /* DLLM_SCORE_* */
  const dllm_polestar_params *polestar;   /* host; DLLM_SCORE_POLESTAR_KL only */
  dllm_polestar_state *polestar_state;    /* DLLM_SCORE_POLESTAR_KL only */
  const dllm_ce_params *ce;               /* host; non-NULL: commit with Confidence Extrapolation
                                             (dllm_commit_ce); not with Polestar-Commit */
  dllm_ce_state *ce_state;                /* with ce */
  /* Optional inspection output (both NULL or both set): every layer's index
   * set of this step, sets_out[l][b][0..n_sets_out[l][b]) ascending
   * ([N][B][L] and [N][B], device). */
  int32_t *sets_out;
  int32_t *n_sets_out;
} dllm_step_params;

typedef struct {
  int32_t n_full;        /* sequences that ran a full pass in this step */
  int32_t n_committed;   /* tokens committed in this step (all sequences) */
  int32_t n_active;      /* sequences that still hold masked rows */
  double max_entropy;    /* max over sequences of state.max_entropy */
} dllm_step_result;

/* Text of the last error on the calling thread ("" if none). */
const char *dllm_last_error(void);

/* Allocate a model for `dims` on the current HIP device, with workspace for
 * max_batch sequences of seq_len rows.  *out is set on success. */
dllm_status dllm_create(const dllm_dims *dims, dllm_model **out);

/* Free a model and its workspace (waits for the device). NULL is a no-op. */
dllm_status dllm_destroy(dllm_model *m);

/* Copy layer `layer`'s weights into library-owned, repacked buffers (the
 * caller may free its copies once the stream has passed this call).  With
 * w->w_proxy == NULL the proxy basis is derived from w->w_v on the device
 * (waits for the stream). */
dllm_status dllm_init_layer(dllm_model *m, int32_t layer, const dllm_layer_weights *w,
                            void *stream);

/* Power steps of the in-library proxy basis when dllm_init_layer derives it. */
#define DLLM_PROXY_ITERS 200

/* SPA-Cache step 1 in the library (init-time): W_r = U_r S_r, the top-r
 * (r = proxy_rank) left singular vectors of the value projection
 * w_v [d_model][n_kv_heads*head_dim] (device, storage dtype) times their
 * singular values, written to w_r_out [d_model][proxy_rank] (device, fp64;
 * dllm_init_layer stores it in fp32 like a supplied basis).
 * Randomised subspace iteration in fp64: p = min(r + 8, d_model, n_v, 136)
 * (rounded down to even) columns started from a fixed pseudo-random matrix,
 * `iters` steps Q <- orth(W (W^T Q)) with CholeskyQR2, then Rayleigh-Ritz
 * (Jacobi eigen-decomposition of Z^T Z, Z = W^T Q).  The columns come out in
 * descending singular value order with an arbitrary sign each, which leaves
 * every proxy cosine unchanged.  Convergence needs a gap between the r-th and
 * (p+1)-th singular values: the subspace error shrinks by (s_{p+1}/s_r)^2
 * per step.  Allocates and frees its fp64 workspace and waits for `stream`.
 * Errors: DLLM_E_ARG (NULL pointer, iters < 0), DLLM_E_UNSUPPORTED
 * (proxy_rank > 128 or p < proxy_rank), DLLM_E_NUMERIC (a non-positive
 * Cholesky pivot: the iterated subspace lost rank). */
dllm_status dllm_derive_proxy_basis(dllm_model *m, const void *w_v, int32_t iters, double *w_r_out, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dllm_derive_proxy_basis with its fp64 workspace and status word in a fixed
 * library-owned device array instead of memory allocated and freed per call;
 * the same kernels, so the same W_r bit for bit.  The array holds
 * DLLM_BASIS_NOALLOC_DOUBLES doubles (32 MiB) per device, from the first
 * dllm_create on that device until the process ends.  The workspace a shape
 * needs, (2 d_model + n_kv_heads*head_dim) p + 4 p^2 + p + p*proxy_rank + 16
 * doubles with p as in dllm_derive_proxy_basis, must fit (every shape with
 * d_model and n_kv_heads*head_dim <= 8192 does); otherwise DLLM_E_SHAPE.
 * Every call on a device shares that device's array, so calls that overlap
 * on one device (any stream, any model) race: the caller serialises them.
 * Waits for `stream`.  Other errors as dllm_derive_proxy_basis. */
#define DLLM_BASIS_NOALLOC_DOUBLES (4u << 20)
dllm_status dllm_derive_proxy_basis_noalloc(dllm_model *m, const void *w_v, int32_t iters, double *w_r_out,
                                            void *stream);

/* Copy the embedding table [vocab][d_model], the final norm gain [d_model]
 * (fp32) and the LM head [d_model][vocab]. */
dllm_status dllm_init_head(dllm_model *m, const void *embed, const float *final_norm,
                           const void *lm_head, void *stream);

/* Layer-0 input for listed rows: hidden[0][b][i] = embed[tokens[b][i]].
 * Rows: rows[b][0..n_rows[b]) (layout [B][L]); rows == NULL means every row.
 * A token id outside [0, vocab) yields a zero row. */
dllm_status dllm_embed(dllm_model *m, const dllm_state *s, const int32_t *rows,
                       const int32_t *n_rows, void *stream);

/* SPA-Cache step 1 at `layer` for the rows whose layer input changed (rows as
 * in dllm_embed; NULL = every row): C = (x * attn_norm) W_r in fp64 from
 * x = hidden[layer][b][i], stored to proxy_cur, and
 * score = 1 - cos(C, P) = 0.5 |C/|C| - P/|P||^2 (both zero: 0; one zero: 1)
 * with P = proxy_ref.  Rows not listed keep their stored score.
 * max_rows (host) bounds sum(n_rows); 0 means batch*seq_len. */
dllm_status dllm_drift_score(dllm_model *m, int32_t layer, dllm_state *s, const int32_t *rows,
                             const int32_t *n_rows, int32_t max_rows, void *stream);

/* SPA-Cache step 2 / EntropyCache step 3: index set I of `layer` per sequence.
 * k = floor(rho * seq_len + 1/2); rows with forced[b][i] != 0 (forced may be
 * NULL) are always selected; the other max(k, |F|) - |F| rows are those with
 * the largest score[layer][b][i], ties to the lower index.  Sequences with
 * full[b] != 0 (full may be NULL) select every row.  Writes idx[b][0..n_sel[b])
 * in ascending order ([B][L] layout) and n_sel[b]. */
dllm_status dllm_select(dllm_model *m, int32_t layer, const dllm_state *s, const uint8_t *forced,
                        const uint8_t *full, double rho, int32_t *idx, int32_t *n_sel,
                        void *stream);

/* SPA-Cache step 3 at `layer` on rows I = idx/n_sel (as from dllm_select):
 * gather rows of hidden[layer], RMSNorm, QKV projection, RoPE, scatter the new
 * keys/values into k_cache/v_cache (before attention), bidirectional attention
 * of the selected queries over all seq_len cached rows, output projection and
 * residual, FFN on the selected rows only, then hidden[layer+1][b][i] <- output
 * for i in I (other rows keep their cached output), proxy_ref <- proxy_cur and
 * score <- 0 for i in I.  max_rows bounds sum(n_sel) (0: batch*seq_len). */
dllm_status dllm_sparse_layer(dllm_model *m, int32_t layer, dllm_state *s, const int32_t *idx,
                              const int32_t *n_sel, int32_t max_rows, void *stream);

/* LM-head statistics of the current block's rows (rows block_start[b] + j,
 * j < block_len): z = (RMSNorm(hidden[N][b][row]) * final_norm) W_lm with the
 * norm in fp64 and z accumulated in fp32.  stats_out[b][j][0..3] (fp64) =
 * max z, argmax (lowest id on ties), S = sum exp(z - max), T = sum exp(z - max)(z - max);
 * confidence = 1/S, entropy = ln S - T/S.  logits_out ([B][block_len][vocab]
 * fp32) is optional (NULL: not written).  Rows past the end are zero. */
dllm_status dllm_lm_head(dllm_model *m, const dllm_state *s, double *stats_out,
                         float *logits_out, void *stream);

/* Static-threshold commit over the current block plus the entropy gate:
 * computes the LM-head statistics, commits every masked block row with
 * confidence >= conf_threshold (if none, the single most confident masked row,
 * lowest position on ties), writes tokens/committed, appends the commits to
 * history in ascending position order, sets n_new, max_entropy (max entropy
 * of the committed rows, 0 if none) and full_next = (max_entropy > tau), and
 * advances block_start past fully committed blocks. */
dllm_status dllm_commit(dllm_model *m, dllm_state *s, double conf_threshold, double tau,
                        void *stream);

/* dllm_commit with Confidence Extrapolation (see dllm_ce_params): the LM-head
 * statistics of the current block, the filter update of its masked rows, then
 * a masked row commits at conf >= conf_threshold or early by extrapolation;
 * if none does, the most confident masked row (lowest position on ties).
 * History, entropy gate and block advance as in dllm_commit.  Errors:
 * DLLM_E_ARG for NULL pointers, NaN thresholds, horizon outside 1..64, r <= 0,
 * or a negative q, p_v0 or kappa. */
dllm_status dllm_commit_ce(dllm_model *m, dllm_state *s, const dllm_ce_params *ce, dllm_ce_state *ce_state,
                           double conf_threshold, double tau, void *stream);

/* Polestar-Cache drift path at `layer` (Polestar, section 2A), per sequence:
 * window rows [ws, ws + W), ws = clamp(block_start - block_len, 0, L - W);
 * spherical k-means (fp64) of the rows' layer inputs hidden[layer] scaled to
 * unit length, seeds at window rows (W / K) * j, kmeans_iters iterations of
 * (assign to the largest dot product, lowest cluster on ties; each cluster
 * with members and a non-zero member sum becomes the normalised member sum)
 * and a final assignment; NVFP4 codes of the residuals (E4M3 scale of amax/6
 * per 16 elements, E2M1 codes of r/scale, both round-to-nearest-even,
 * saturating); centroid queries bf16(RMSNorm(c) * attn_norm) W_q with RoPE at
 * the seed row's position; per query head the fp64 log-softmax over the window
 * keys of k_cache[layer] (scale 1/sqrt(head_dim)), and the per-head KL against
 * log_attn, which it then replaces.  Everything runs on `stream`. */
dllm_status dllm_polestar_drift(dllm_model *m, int32_t layer, const dllm_state *s, dllm_polestar_state *ps,
                                const dllm_polestar_params *p, void *stream);

/* Polestar selection at `layer`: cluster drift = mean over heads of the KL
 * from dllm_polestar_drift, or 0 when win_start[layer][b] != ws (the window's
 * first step); the top_clusters of largest drift (lowest index on ties); index
 * set I = current block rows + the window rows assigned to those clusters,
 * ascending, into idx[b][0..n_sel[b]) ([B][L]); records win_start.  Follow
 * with dllm_sparse_layer(max_rows = batch * W). */
dllm_status dllm_polestar_select(dllm_model *m, int32_t layer, const dllm_state *s, dllm_polestar_state *ps,
                                 const dllm_polestar_params *p, int32_t *idx, int32_t *n_sel, void *stream);

/* Polestar-Commit (Polestar, section 2B) of one step, in place of dllm_commit
 * for callers of the Polestar drift path.  The LM-head statistics are taken
 * for the current block and the next one (rows past seq_len are skipped).
 * Uses the cluster drift, assignment and top clusters that the last
 * dllm_polestar_drift / dllm_polestar_select left in ps (the last layer's),
 * when ps->drift_valid says they are defined.  For each still-masked row j of
 * the current block with confidence c_j: commit if c_j >= conf_threshold (tau_s),
 * or if its drift D_j (its cluster's drift) exceeds the mean of its earlier
 * drifts in this block by more than alpha (tau_s - c_j)^2 (strictly; no
 * earlier drift: no drift commit).  If none commits, the most confident
 * masked row does (lowest position on ties).  If a top cluster has a member
 * among the window rows after the current block, the next block's masked
 * rows with c >= tau_s commit too.  Commits are appended to the history in
 * ascending position order; the entropy gate and block advance are those of
 * dllm_commit.  Then D_j is added to drift_sum/drift_cnt (both cleared when
 * the block advances) and drift_valid is cleared. */
dllm_status dllm_polestar_commit(dllm_model *m, dllm_state *s, dllm_polestar_state *ps,
                                 const dllm_polestar_params *p, double conf_threshold, double tau,
                                 void *stream);

/* Forced rows for the next step, forced[b][i] in {0,1} ([B][L]):
 * DLLM_FORCED_BLOCK marks the current block, DLLM_FORCED_BLOCK_RECENT also the
 * last recent_k entries of history, DLLM_FORCED_NONE marks nothing. */
dllm_status dllm_forced_set(dllm_model *m, const dllm_state *s, int32_t rule, int32_t recent_k,
                            uint8_t *forced, void *stream);

/* One denoising step for every sequence: embed the rows whose token changed
 * (every row in a full pass), then per layer drift score, selection (every
 * row in a full pass) and sparse layer, then commit.  With
 * score = DLLM_SCORE_POLESTAR_KL a sparse step uses dllm_polestar_drift and
 * dllm_polestar_select instead of the value-proxy drift and top-k, and leaves
 * proxy_ref and score untouched.  Mode FULL or SPARSE applies to every
 * sequence; AUTO runs a full pass for the sequences whose full_next is set
 * (the caller sets it before the first step, whose caches are empty).  With
 * DLLM_SCORE_POLESTAR_KL, AUTO returns DLLM_E_UNSUPPORTED (nothing enqueued
 * after the read of full_next) when full_next is set for some sequences but
 * not all, and no periodic full pass is due.  If res_h is non-NULL the call
 * waits for the stream and fills it. */
dllm_status dllm_step(dllm_model *m, dllm_state *s, const dllm_step_params *p,
                      dllm_step_result *res_h, void *stream);

/* Diagnostics: live timing of kernel classes.  While enabled, the library
 * records a HIP event pair on the launch stream around every launch of the
 * class's kernels, together with the launch's algorithmic bytes and flops
 * (weights + activations read, outputs written; split-K partials are not
 * counted).  dllm_profile_read waits for the recorded events, writes
 * DLLM_PROF_N entries to stats_h and clears them. */
enum { DLLM_PROF_GEMM = 0,      /* layer GEMMs (QKV, O, gate|up, down; Polestar centroid queries) */
       DLLM_PROF_LMHEAD = 1,    /* LM-head GEMM */
       DLLM_PROF_ATTN = 2,      /* attention */
       DLLM_PROF_PROXY = 3,     /* value proxy + drift */
       DLLM_PROF_SELECT = 4,    /* index-set selection (top-k, or Polestar cluster selection) */
       DLLM_PROF_ROWS = 5,      /* row kernels: gather + RMSNorm, QKV / O / down epilogues, SwiGLU
                                   (these count the split-K partials they read) */
       DLLM_PROF_POLESTAR = 6,  /* Polestar drift path except its query GEMM */
       DLLM_PROF_DECIDE = 7,    /* prep, embedding, LM-head gather and statistics, commit */
       DLLM_PROF_N = 8 };
typedef struct {
  int64_t launches;
  double ms;      /* sum of event-pair durations */
  double bytes;   /* sum of algorithmic bytes */
  double flops;   /* sum of algorithmic flops */
} dllm_kernel_stats;
#define DLLM_PROF_ALL ((1 << DLLM_PROF_N) - 1)
/* class_mask: bit c (1 << DLLM_PROF_c) records class c; 0 stops recording.
 * Every recorded launch adds two stream markers, so time the step with only
 * the classes needed. */
dllm_status dllm_profile(dllm_model *m, int32_t class_mask);
dllm_status dllm_profile_read(dllm_model *m, dllm_kernel_stats *stats_h);

/* Diagnostics: achievable streaming-read bandwidth, the measured ceiling the
 * kernels' algorithmic GB/s is also compared with (besides the published HBM
 * peak).  Streams dev_buf (device memory, bytes >= 256 MiB; only the leading
 * multiple of 64 MiB is read) with 16-byte nontemporal loads under four launch
 * shapes (1024 or 2048 workgroups of 256 threads, 4 or 8 loads in flight per
 * thread), each once untimed and then `reps` times between HIP events on
 * `stream`, and stores the best shape's mean rate in *gbps_h (1e9 bytes/s).
 * dev_scratch: device memory of at least 8 KiB (checksum words).  Waits for
 * the stream.  Errors: DLLM_E_ARG (NULL pointer, reps < 1, bytes < 256 MiB). */
dllm_status dllm_stream_probe(const void *dev_buf, size_t bytes, void *dev_scratch, int32_t reps, double *gbps_h,
                              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBDLLM_H */
