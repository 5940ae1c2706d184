// libdllm C-ABI: argument validation, weight repacking, workspace and the
// per-step orchestration of the kernels (see include/libdllm.h).
#include "../../include/libdllm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

using namespace dllm;

namespace {

thread_local std::string g_err;

dllm_status fail(dllm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIPCHK(expr)                                                                  \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess) return fail(DLLM_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define CHK(expr)                   \
  do {                              \
    dllm_status s_ = (expr);        \
    if (s_ != DLLM_OK) return s_;   \
  } while (0)

struct LayerW {
  float* attn_norm = nullptr;
  float* ffn_norm = nullptr;
  void* w_qkv = nullptr;   // packed [d][nq + 2 nv]
  void* w_o = nullptr;     // packed [nq][d]
  void* w_gu = nullptr;    // packed [d][2F]: bf16 gate/up 16 + 16 columns per 32-column tile; fp32 by 32 columns
  void* w_down = nullptr;  // packed [F][d]
  float* w_proxy = nullptr;  // W_r, fp32 [d][proxy_rpad(r)] (zero columns past r)
  bool ready = false;
};

}  // namespace

struct dllm_model {
  dllm_dims d{};
  int device = 0;
  bool bf16 = false;
  int n_cu = 256;
  size_t esize = 4;
  std::vector<LayerW> layers;
  void* embed = nullptr;
  float* final_norm = nullptr;
  void* lm_head = nullptr;
  bool head_ready = false;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  // workspace
  int M_cap = 0;   // max_batch * seq_len
  int M_pad = 0;   // rows allocated in activation buffers
  int MTt = 0;     // 32-row tiles of the packed GEMM inputs (M_pad / 32)
  int lm_MTt = 0;  // same for the LM-head input
  void* A1 = nullptr;
  void* q = nullptr;
  void* attn_o = nullptr;
  void* A2 = nullptr;
  void* act = nullptr;
  float* hprime = nullptr;
  float* part = nullptr;
  size_t part_floats = 0;
  double* ppart = nullptr;
  size_t ppart_doubles = 0;
  int32_t* idx[2] = {nullptr, nullptr};
  int32_t* nsel[2] = {nullptr, nullptr};
  int32_t* idx0 = nullptr;
  int32_t* n0 = nullptr;
  uint8_t* forced = nullptr;
  uint8_t* step_full = nullptr;
  void* A_lm = nullptr;
  float* logits = nullptr;
  double* lm_part = nullptr;
  double* lm_stats = nullptr;
  double* lm_wpart = nullptr;  // per-slab statistics of the fused LM head [rows][vocab/128][4]
  int32_t* lm_rows = nullptr;
  int lm_slabs = 0;
  // Polestar drift path workspace
  double* ps_R = nullptr;      // Gram split partials [max_batch][ps_gram_splits()][W][W]
  double* ps_coef = nullptr;   // centroid coefficients [max_batch][16][W]
  double* ps_klp = nullptr;    // per-head KL [max_batch][Hq][16]
  int32_t* ps_nsel = nullptr;  // centroid rows per sequence
  void* ps_A = nullptr;        // packed centroid rows for the query GEMM
  int ps_MTt = 0;
  void* res_dev = nullptr;
  void* res_host = nullptr;   // pinned, 32 bytes
  uint8_t* full_host = nullptr;  // pinned, max_batch
  std::vector<void*> allocs;
  // diagnostics
  struct ProfRec {
    hipEvent_t a, b;
    int cls;
    double bytes, flops;
  };
  bool prof_on = false;
  int32_t prof_mask = 0;  // bit c: class c records events
  std::vector<ProfRec> prof_pending;
  std::vector<hipEvent_t> ev_pool;
  std::vector<hipEvent_t> ev_all;

  dllm_status alloc(void** p, size_t bytes) {
    if (bytes == 0) bytes = 16;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
      *p = nullptr;
      return fail(DLLM_E_NOMEM, "hipMalloc(%zu bytes): %s", bytes, hipGetErrorString(e));
    }
    allocs.push_back(*p);
    e = hipMemset(*p, 0, bytes);
    if (e != hipSuccess) return fail(DLLM_E_HIP, "hipMemset: %s", hipGetErrorString(e));
    return DLLM_OK;
  }
  template <typename T>
  dllm_status alloc_t(T** p, size_t count) {
    void* v = nullptr;
    dllm_status s = alloc(&v, count * sizeof(T));
    *p = (T*)v;
    return s;
  }
};

namespace {

inline hipStream_t S(void* stream) { return (hipStream_t)stream; }

// Event pair around a group of launches of one kernel class (diagnostics).
struct Prof {
  dllm_model* m;
  hipStream_t st;
  int cls;
  double bytes, flops;
  hipEvent_t a = nullptr;
  static hipEvent_t get(dllm_model* m) {
    if (!m->ev_pool.empty()) {
      hipEvent_t e = m->ev_pool.back();
      m->ev_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    m->ev_all.push_back(e);
    return e;
  }
  Prof(dllm_model* m_, hipStream_t st_, int cls_, double bytes_, double flops_)
      : m(m_), st(st_), cls(cls_), bytes(bytes_), flops(flops_) {
    if (m->prof_on && ((m->prof_mask >> cls) & 1)) {
      a = get(m);
      if (a) (void)hipEventRecord(a, st);
    }
  }
  void done() {
    if (!a) return;
    hipEvent_t b = get(m);
    if (!b) return;
    (void)hipEventRecord(b, st);
    m->prof_pending.push_back({a, b, cls, bytes, flops});
    a = nullptr;
  }
};

// Event pair of one kernel launch of a class, stamped by the launch itself
// (hipExtLaunchKernel): the kernel's own begin and end, with no marker packets
// in the stream around it (diagnostics).
struct ProfLaunch {
  dllm_model* m;
  int cls;
  double bytes, flops;
  LaunchEvents ev;
  ProfLaunch(dllm_model* m_, int cls_, double bytes_, double flops_) : m(m_), cls(cls_), bytes(bytes_), flops(flops_) {
    if (m->prof_on && ((m->prof_mask >> cls) & 1)) {
      ev.start = Prof::get(m);
      ev.stop = ev.start ? Prof::get(m) : nullptr;
      if (!ev.stop) ev.start = nullptr;
    }
  }
  // after a successful launch
  void done() {
    if (ev.start) m->prof_pending.push_back({ev.start, ev.stop, cls, bytes, flops});
    ev = {};
  }
};

int nq_of(const dllm_dims& d) { return d.n_q_heads * d.head_dim; }
int nv_of(const dllm_dims& d) { return d.n_kv_heads * d.head_dim; }

dllm_status check_model(const dllm_model* m) {
  if (!m) return fail(DLLM_E_ARG, "model is NULL");
  return DLLM_OK;
}

dllm_status check_state(const dllm_model* m, const dllm_state* s, bool need_proxy = true) {
  if (!s) return fail(DLLM_E_ARG, "state is NULL");
  if (s->batch < 1 || s->batch > m->d.max_batch)
    return fail(DLLM_E_ARG, "state.batch=%d outside [1, %d]", s->batch, m->d.max_batch);
  if (!s->hidden || !s->k_cache || !s->v_cache || !s->tokens || !s->committed || !s->history || !s->n_history ||
      !s->n_new || !s->block_start || !s->full_next || !s->max_entropy || !s->score)
    return fail(DLLM_E_ARG, "state has a NULL buffer");
  if (need_proxy && (!s->proxy_cur || !s->proxy_ref)) return fail(DLLM_E_ARG, "state has a NULL proxy buffer");
  return DLLM_OK;
}

dllm_status check_layer(const dllm_model* m, int layer) {
  if (layer < 0 || layer >= m->d.n_layers)
    return fail(DLLM_E_ARG, "layer %d outside [0, %d)", layer, m->d.n_layers);
  if (!m->layers[layer].ready) return fail(DLLM_E_STATE, "layer %d weights not initialised", layer);
  return DLLM_OK;
}

// state slices
void* hid(const dllm_model* m, const dllm_state* s, int slot) {
  return (char*)s->hidden + (size_t)slot * s->batch * m->d.seq_len * m->d.d_model * m->esize;
}
size_t l32(const dllm_dims& d) { return (size_t)((d.seq_len + 31) / 32) * 32; }
void* kcache(const dllm_model* m, const dllm_state* s, int l) {
  return (char*)s->k_cache + (size_t)l * s->batch * nv_of(m->d) * l32(m->d) * m->esize;
}
void* vcache(const dllm_model* m, const dllm_state* s, int l) {
  return (char*)s->v_cache + (size_t)l * s->batch * nv_of(m->d) * l32(m->d) * m->esize;
}
double* pcur(const dllm_model* m, const dllm_state* s, int l) {
  return s->proxy_cur + (size_t)l * s->batch * m->d.seq_len * m->d.proxy_rank;
}
double* pref(const dllm_model* m, const dllm_state* s, int l) {
  return s->proxy_ref + (size_t)l * s->batch * m->d.seq_len * m->d.proxy_rank;
}
double* score(const dllm_model* m, const dllm_state* s, int l) {
  return s->score + (size_t)l * s->batch * m->d.seq_len;
}

int clamp_rows(const dllm_model* m, const dllm_state* s, int max_rows) {
  const int cap = s->batch * m->d.seq_len;
  return (max_rows <= 0 || max_rows > cap) ? cap : max_rows;
}

// out = A W (partials into `out`, split count returned)
dllm_status gemm(dllm_model* m, hipStream_t st, int max_rows, int B, int K, int N, const void* A, const void* W,
                 const int32_t* n_sel, float* out, size_t out_floats, int* splits, int cls = DLLM_PROF_GEMM,
                 int MTt = -1, void* act = nullptr) {
  if (MTt < 0) MTt = m->MTt;
  // algorithmic bytes: the weight, the input rows and the output rows in the
  // storage type (SwiGLU halves the output width); split-K partials are the
  // kernel's own traffic, not the method's
  const double n_out = act ? N / 2.0 : (double)N;
  ProfLaunch prof(m, cls, (double)K * N * m->esize + (double)max_rows * K * m->esize + (double)max_rows * n_out * m->esize,
                  2.0 * max_rows * (double)K * N);
  if (m->bf16) {
    // up to 288 rows: the weight-streaming kernel, when the shape suits it, on
    // 96-column slabs where those fill more of the chip
    int s3 = gemm_stream3_pick_splits(max_rows, K, N, m->n_cu, act != nullptr, MTt);
    if (s3 > 0 && !act && (size_t)s3 * max_rows * N > out_floats) s3 = 0;
    if (s3 > 0) {
      HIPCHK(launch_gemm_stream3(st, max_rows, B, K, N, (const uint16_t*)A, MTt, (const uint16_t*)W, n_sel, out, s3,
                                 (uint16_t*)act, m->MTt, prof.ev));
      *splits = s3;
      prof.done();
      return DLLM_OK;
    }
    int ss = gemm_stream_pick_splits(max_rows, K, N, m->n_cu, act != nullptr, MTt);
    if (ss > 0 && !act && (size_t)ss * max_rows * N > out_floats) ss = 0;
    if (ss > 0) {
      HIPCHK(launch_gemm_stream(st, max_rows, B, K, N, (const uint16_t*)A, MTt, (const uint16_t*)W, n_sel, out, ss,
                                (uint16_t*)act, m->MTt, prof.ev));
      *splits = ss;
      prof.done();
      return DLLM_OK;
    }
    int sp = act ? 1 : gemm_bf16_pick_splits(max_rows, K, N, m->n_cu);
    while (sp > 1 && (size_t)sp * max_rows * N > out_floats) sp /= 2;
    if (!act && (size_t)sp * max_rows * N > out_floats) return fail(DLLM_E_SHAPE, "GEMM partial buffer too small");
    HIPCHK(launch_gemm_bf16(st, max_rows, B, K, N, (const uint16_t*)A, MTt, (const uint16_t*)W, n_sel, out, sp,
                            (uint16_t*)act, m->MTt, gemm_bf16_pick_cols(max_rows, K, N, m->n_cu, sp), prof.ev));
    *splits = sp;
  } else {
    if ((size_t)max_rows * N > out_floats) return fail(DLLM_E_SHAPE, "GEMM partial buffer too small");
    HIPCHK(launch_gemm_f32(st, max_rows, B, K, N, (const float*)A, (const float*)W, n_sel, out, prof.ev));
    *splits = 1;
  }
  prof.done();
  return DLLM_OK;
}

dllm_status pack(dllm_model* m, hipStream_t st, int K, int Nsrc, const void* src, void* dst, int Ndst, int col0,
                 int tile_stride, int gw = 32) {
  if (m->bf16)
    HIPCHK(launch_pack_bf16(st, K, Nsrc, (const uint16_t*)src, Nsrc, (uint16_t*)dst, col0, tile_stride, gw));
  else
    HIPCHK(launch_pack_f32(st, K, Nsrc, (const float*)src, Nsrc, (float*)dst, Ndst, col0, tile_stride));
  return DLLM_OK;
}

dllm_status do_drift(dllm_model* m, int layer, dllm_state* s, const int32_t* rows, const int32_t* n, int max_rows,
                     hipStream_t st) {
  const dllm_dims& d = m->d;
  Prof prof(m, st, DLLM_PROF_PROXY,
            (double)max_rows * d.d_model * m->esize + (double)d.d_model * d.proxy_rank * 4.0 +
                (double)max_rows * d.proxy_rank * 8.0 * 3.0,
            2.0 * max_rows * (double)d.d_model * d.proxy_rank);
  HIPCHK(launch_proxy_drift(st, m->bf16, max_rows, s->batch, d.seq_len, d.d_model, d.proxy_rank, rows, n,
                            hid(m, s, layer), m->layers[layer].attn_norm, m->layers[layer].w_proxy, m->ppart,
                            pcur(m, s, layer),
                            pref(m, s, layer), score(m, s, layer)));
  prof.done();
  return DLLM_OK;
}

// refresh_proxy: P <- C and score <- 0 on I (the value-proxy path; the
// Polestar drift path keeps no value proxy and leaves both untouched)
dllm_status do_sparse(dllm_model* m, int layer, dllm_state* s, const int32_t* idx, const int32_t* n, int max_rows,
                      hipStream_t st, bool refresh_proxy = true, bool gathered = false) {
  const dllm_dims& d = m->d;
  const int B = s->batch, L = d.seq_len, D = d.d_model, F = d.d_ffn;
  const int nq = nq_of(d), nv = nv_of(d);
  const LayerW& w = m->layers[layer];
  const void* Hin = hid(m, s, layer);
  int sp = 1;
  const double Mr = max_rows, es = m->esize, nqkv = nq + 2 * nv;
  if (!gathered) {
    Prof prof(m, st, DLLM_PROF_ROWS, 2.0 * Mr * D * es + D * 4.0, 4.0 * Mr * D);
    HIPCHK(launch_gather_norm(st, m->bf16, max_rows, B, L, D, d.rms_eps, m->MTt, idx, n, Hin, w.attn_norm, m->A1));
    prof.done();
  }
  CHK(gemm(m, st, max_rows, B, D, nq + 2 * nv, m->A1, w.w_qkv, n, m->part, m->part_floats, &sp));
  {
    Prof prof(m, st, DLLM_PROF_ROWS, sp * Mr * nqkv * 4.0 + Mr * nqkv * es, Mr * nqkv * (sp + 3.0));
    HIPCHK(launch_qkv_epilogue(st, m->bf16, max_rows, B, L, d.n_q_heads, d.n_kv_heads, d.head_dim, sp, idx, n,
                               m->part, m->rope_cos, m->rope_sin, m->q, kcache(m, s, layer), vcache(m, s, layer)));
    prof.done();
  }
  {
    Prof prof(m, st, DLLM_PROF_ATTN,
              2.0 * B * L * nv * m->esize + 2.0 * max_rows * nq * m->esize,
              4.0 * max_rows * (double)L * nq);
    HIPCHK(launch_attention(st, m->bf16, max_rows, B, L, d.n_q_heads, d.n_kv_heads, d.head_dim, idx, n, m->q,
                            kcache(m, s, layer), vcache(m, s, layer), m->attn_o, m->MTt));
    prof.done();
  }
  CHK(gemm(m, st, max_rows, B, nq, D, m->attn_o, w.w_o, n, m->part, m->part_floats, &sp));
  {
    Prof prof(m, st, DLLM_PROF_ROWS, sp * Mr * D * 4.0 + Mr * D * (2.0 * es + 4.0), Mr * D * (sp + 5.0));
    HIPCHK(launch_o_epilogue(st, m->bf16, max_rows, B, L, D, sp, d.rms_eps, m->MTt, idx, n, m->part, Hin,
                             w.ffn_norm, m->hprime, m->A2));
    prof.done();
  }
  if (m->bf16) {
    // SwiGLU fused into the gate|up GEMM
    CHK(gemm(m, st, max_rows, B, D, 2 * F, m->A2, w.w_gu, n, m->part, m->part_floats, &sp, DLLM_PROF_GEMM, m->MTt,
             m->act));
  } else {
    CHK(gemm(m, st, max_rows, B, D, 2 * F, m->A2, w.w_gu, n, m->part, m->part_floats, &sp));
    Prof prof(m, st, DLLM_PROF_ROWS, sp * Mr * 2.0 * F * 4.0 + Mr * F * es, Mr * F * (2.0 * sp + 4.0));
    HIPCHK(launch_swiglu(st, m->bf16, max_rows, B, F, sp, n, m->part, m->act));
    prof.done();
  }
  CHK(gemm(m, st, max_rows, B, F, D, m->act, w.w_down, n, m->part, m->part_floats, &sp));
  {
    Prof prof(m, st, DLLM_PROF_ROWS,
              sp * Mr * D * 4.0 + Mr * D * (4.0 + es) + Mr * d.proxy_rank * 16.0 + Mr * 8.0, Mr * D * sp);
    HIPCHK(launch_down_epilogue(st, m->bf16, max_rows, B, L, D, d.proxy_rank, sp, idx, n, m->part, m->hprime,
                                hid(m, s, layer + 1), pcur(m, s, layer), refresh_proxy ? pref(m, s, layer) : nullptr,
                                score(m, s, layer)));
    prof.done();
  }
  return DLLM_OK;
}

// Rows the weight-streaming GEMM takes (9 row tiles): the LM head's fused
// statistics path and its streaming logits path.
constexpr int LM_FUSED_ROWS = 288;

// LM-head statistics of the first nblk blocks from each sequence's block
// start (nblk = 1: the current block; 2: also the next one).  Up to
// LM_FUSED_ROWS rows and no logits wanted: the statistics come out of the
// weight-streaming GEMM per 128-column slab and one merge (no logits buffer);
// otherwise the logits are materialised (m->logits) and reduced by slab and
// merge kernels.
dllm_status do_lm_head(dllm_model* m, const dllm_state* s, hipStream_t st, int nblk = 1, bool want_logits = false) {
  const dllm_dims& d = m->d;
  const int B = s->batch, blk = d.block_len * nblk;
  {
    Prof prof(m, st, DLLM_PROF_DECIDE, 2.0 * B * blk * d.d_model * m->esize, 4.0 * B * blk * d.d_model);
    HIPCHK(launch_lm_gather(st, m->bf16, B, d.seq_len, blk, d.d_model, d.rms_eps, m->lm_MTt, s->block_start,
                            hid(m, s, d.n_layers), m->final_norm, m->A_lm, m->lm_rows));
    prof.done();
  }
  if (m->bf16 && !want_logits && m->lm_wpart && B * blk <= LM_FUSED_ROWS &&
      gemm_stream_pick_splits(B * blk, d.d_model, d.vocab, m->n_cu, false, m->lm_MTt) > 0) {
    const int ns = d.vocab / 128;
    ProfLaunch prof(m, DLLM_PROF_LMHEAD,
                    (double)d.d_model * d.vocab * 2.0 + (double)B * blk * d.d_model * 2.0 + (double)B * blk * 32.0,
                    2.0 * B * blk * (double)d.d_model * d.vocab);
    HIPCHK(launch_gemm_stream_stats(st, B * blk, d.d_model, d.vocab, (const uint16_t*)m->A_lm, m->lm_MTt,
                                    (const uint16_t*)m->lm_head, m->lm_rows, m->lm_wpart, prof.ev));
    prof.done();
    Prof prof2(m, st, DLLM_PROF_DECIDE, (double)B * blk * ns * 32.0, 0.0);
    HIPCHK(launch_lm_merge_wide(st, B * blk, ns, m->lm_wpart, m->lm_stats));
    prof2.done();
    return DLLM_OK;
  }
  int sp = 1;
  const size_t cap = (size_t)d.max_batch * 2 * d.block_len * d.vocab;
  if (m->bf16) {
    ProfLaunch prof(m, DLLM_PROF_LMHEAD,
                    (double)d.d_model * d.vocab * 2.0 + (double)B * blk * d.d_model * 2.0 +
                        (double)B * blk * d.vocab * 4.0,
                    2.0 * B * blk * (double)d.d_model * d.vocab);
    // the weight-streaming kernel (one split: the logits are written once, in
    // the same [M][V] layout), as in the fused path, where the rows fit it
    const int ss =
        B * blk <= LM_FUSED_ROWS ? gemm_stream_pick_splits(B * blk, d.d_model, d.vocab, m->n_cu, false, m->lm_MTt) : 0;
    if (ss == 1)
      HIPCHK(launch_gemm_stream(st, B * blk, 1, d.d_model, d.vocab, (const uint16_t*)m->A_lm, m->lm_MTt,
                                (const uint16_t*)m->lm_head, m->lm_rows, m->logits, 1, nullptr, 0, prof.ev));
    else
      HIPCHK(launch_gemm_bf16(st, B * blk, 1, d.d_model, d.vocab, (const uint16_t*)m->A_lm, m->lm_MTt,
                              (const uint16_t*)m->lm_head, m->lm_rows, m->logits, 1, nullptr, 0,
                              gemm_bf16_pick_cols(B * blk, d.d_model, d.vocab, m->n_cu, 1), prof.ev));
    prof.done();
  } else {
    CHK(gemm(m, st, B * blk, 1, d.d_model, d.vocab, m->A_lm, m->lm_head, m->lm_rows, m->logits, cap, &sp,
             DLLM_PROF_LMHEAD));
  }
  Prof prof(m, st, DLLM_PROF_DECIDE, 4.0 * B * blk * d.vocab, 4.0 * B * blk * d.vocab);
  HIPCHK(launch_lm_stats(st, B * blk, d.vocab, m->logits, m->lm_part, m->lm_stats, m->lm_slabs));
  prof.done();
  return DLLM_OK;
}

dllm_status do_commit(dllm_model* m, dllm_state* s, double thr, double tau, hipStream_t st) {
  CHK(do_lm_head(m, s, st));
  const dllm_dims& d = m->d;
  Prof prof(m, st, DLLM_PROF_DECIDE, (double)s->batch * d.block_len * (32.0 + 4.0 + 1.0), 0.0);
  HIPCHK(launch_commit(st, s->batch, d.seq_len, d.block_len, thr, tau, m->lm_stats, s->tokens, s->committed,
                       s->history, s->n_history, s->n_new, s->block_start, s->full_next, s->max_entropy));
  prof.done();
  return DLLM_OK;
}

dllm_status check_ce(const dllm_model* m, const dllm_ce_params* ce, const dllm_ce_state* cs) {
  if (!ce || !cs || !cs->kf || !cs->has) return fail(DLLM_E_ARG, "CE params/state is NULL");
  if (ce->horizon < 1 || ce->horizon > 64) return fail(DLLM_E_ARG, "CE horizon must be in [1, 64]");
  if (!(ce->r > 0.0) || !(ce->q >= 0.0) || !(ce->p_v0 >= 0.0) || !(ce->kappa >= 0.0) || std::isnan(ce->gamma))
    return fail(DLLM_E_ARG, "CE needs r > 0, q, p_v0, kappa >= 0 and a gamma");
  if (m->d.block_len > 64) return fail(DLLM_E_UNSUPPORTED, "CE needs block_len <= 64");
  return DLLM_OK;
}

dllm_status do_commit_ce(dllm_model* m, dllm_state* s, const dllm_ce_params* ce, dllm_ce_state* cs, double thr,
                         double tau, hipStream_t st) {
  CHK(do_lm_head(m, s, st));
  const dllm_dims& d = m->d;
  Prof prof(m, st, DLLM_PROF_DECIDE, (double)s->batch * d.block_len * (32.0 + 4.0 + 1.0 + 44.0), 0.0);
  HIPCHK(launch_ce_commit(st, s->batch, d.seq_len, d.block_len, thr, tau, ce->horizon, ce->q, ce->r, ce->p_v0,
                          ce->kappa, ce->gamma, m->lm_stats, cs->kf, cs->has, s->tokens, s->committed, s->history,
                          s->n_history, s->n_new, s->block_start, s->full_next, s->max_entropy));
  prof.done();
  return DLLM_OK;
}

dllm_status do_polestar_commit(dllm_model* m, dllm_state* s, dllm_polestar_state* ps, const dllm_polestar_params* p,
                               double thr, double tau, hipStream_t st) {
  CHK(do_lm_head(m, s, st, 2));
  const dllm_dims& d = m->d;
  const int W = p->window_blocks * d.block_len;
  Prof prof(m, st, DLLM_PROF_DECIDE, (double)s->batch * d.block_len * 2.0 * (32.0 + 4.0 + 1.0 + 12.0), 0.0);
  HIPCHK(launch_ps_commit(st, s->batch, d.seq_len, d.block_len, W, p->n_clusters, p->top_clusters, thr,
                          p->commit_alpha, tau, m->lm_stats, ps->kl, ps->assign, ps->top, ps->drift_valid,
                          ps->drift_sum, ps->drift_cnt, s->tokens, s->committed, s->history, s->n_history, s->n_new,
                          s->block_start, s->full_next, s->max_entropy));
  prof.done();
  return DLLM_OK;
}

// copy of layer l's index set into the caller's inspection buffers
dllm_status save_sets(dllm_model* m, const dllm_state* s, const dllm_step_params* p, int l, const int32_t* idx,
                      const int32_t* n, hipStream_t st) {
  if (!p->sets_out) return DLLM_OK;
  const size_t BL = (size_t)s->batch * m->d.seq_len;
  HIPCHK(hipMemcpyAsync(p->sets_out + (size_t)l * BL, idx, BL * 4, hipMemcpyDeviceToDevice, st));
  HIPCHK(hipMemcpyAsync(p->n_sets_out + (size_t)l * s->batch, n, (size_t)s->batch * 4, hipMemcpyDeviceToDevice, st));
  return DLLM_OK;
}

dllm_status finish_step(dllm_model* m, dllm_state* s, dllm_step_result* res_h, hipStream_t st) {
  if (!res_h) return DLLM_OK;
  const int B = s->batch, L = m->d.seq_len;
  HIPCHK(launch_step_result(st, B, m->step_full, s->n_new, s->block_start, s->max_entropy, L, m->res_dev));
  HIPCHK(hipMemcpyAsync(m->res_host, m->res_dev, 32, hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  const int32_t* r = (const int32_t*)m->res_host;
  res_h->n_full = r[0];
  res_h->n_committed = r[1];
  res_h->n_active = r[2];
  std::memcpy(&res_h->max_entropy, r + 4, 8);
  return DLLM_OK;
}

dllm_status check_polestar(const dllm_model* m, const dllm_state* s, const dllm_polestar_state* ps,
                           const dllm_polestar_params* p) {
  const dllm_dims& d = m->d;
  if (!ps || !p) return fail(DLLM_E_ARG, "polestar state/params is NULL");
  if (!ps->log_attn || !ps->win_start || !ps->centroids || !ps->norms || !ps->assign || !ps->codes || !ps->scales ||
      !ps->queries || !ps->kl || !ps->top || !ps->drift_sum || !ps->drift_cnt || !ps->drift_valid || !ps->upd_hist)
    return fail(DLLM_E_ARG, "polestar state has a NULL buffer");
  if (p->drift_commit && !(p->commit_alpha >= 0.0)) return fail(DLLM_E_ARG, "commit_alpha must be >= 0");
  if (p->tau_upd < 0 || p->full_period < 0) return fail(DLLM_E_ARG, "tau_upd and full_period must be >= 0");
  if (d.block_len > 64) return fail(DLLM_E_UNSUPPORTED, "the Polestar path needs block_len <= 64");
  if (!m->ps_R) return fail(DLLM_E_UNSUPPORTED, "the Polestar path needs d_model %% 128 == 0");
  const int W = p->window_blocks * d.block_len;
  if (p->n_clusters < 1 || p->n_clusters > 16) return fail(DLLM_E_ARG, "n_clusters must be in [1, 16]");
  if (p->kmeans_iters < 0) return fail(DLLM_E_ARG, "kmeans_iters < 0");
  if (p->top_clusters < 1 || p->top_clusters > p->n_clusters) return fail(DLLM_E_ARG, "top_clusters out of range");
  if (p->window_blocks < 1 || W > 120 || W > d.seq_len || W < p->n_clusters)
    return fail(DLLM_E_SHAPE, "window of %d rows: need n_clusters <= W <= min(120, seq_len)", W);
  if (d.head_dim % 32 || d.head_dim > 128)
    return fail(DLLM_E_UNSUPPORTED, "the Polestar proxy attention needs head_dim %% 32 == 0 and <= 128");
  (void)s;
  return DLLM_OK;
}

dllm_status do_polestar_drift(dllm_model* m, int layer, const dllm_state* s, dllm_polestar_state* ps,
                              const dllm_polestar_params* p, hipStream_t st) {
  const dllm_dims& d = m->d;
  const int B = s->batch, L = d.seq_len, D = d.d_model, blk = d.block_len;
  const int W = p->window_blocks * blk, K = p->n_clusters, Hq = d.n_q_heads, dh = d.head_dim;
  const LayerW& w = m->layers[layer];
  void* H = hid(m, const_cast<dllm_state*>(s), layer);
  const double es = m->esize, Bw = (double)B * W;
  // window rows read by the Gram and the centroids; centroids (fp64 and
  // packed) written
  Prof prof(m, st, DLLM_PROF_POLESTAR, 2.0 * Bw * D * es + (double)B * K * D * (8.0 + es),
            2.0 * Bw * W * D + 2.0 * Bw * D);
  HIPCHK(launch_ps_gram(st, m->bf16, B, L, D, blk, W, s->block_start, H, m->ps_R));
  HIPCHK(launch_ps_kmeans(st, B, W, K, p->kmeans_iters, m->ps_R, ps->assign, ps->norms, m->ps_coef, m->ps_nsel));
  HIPCHK(launch_ps_centroids(st, m->bf16, B, L, D, blk, W, K, d.rms_eps, m->ps_MTt, s->block_start, H, m->ps_coef,
                             ps->norms, w.attn_norm, ps->centroids, m->ps_A));
  prof.done();
  // The NVFP4 codes of the residuals (the compressed proxy; nothing in the
  // step reads them) on the same stream.  Run beside the step's kernels on a
  // second stream they cost more than they hide (measured at batch 4, L=4096:
  // 13.39 vs 13.25 ms per step): their workgroups take CUs the one-workgroup-
  // per-CU GEMMs wait for.
  HIPCHK(launch_ps_codes(st, m->bf16, B, L, D, blk, W, K, s->block_start, H, ps->norms, ps->assign,
                         ps->centroids, ps->codes, ps->scales));
  // centroid queries through the layer's query projection (the first
  // n_q_heads*head_dim columns of the packed QKV weight; fp32 models use the
  // whole row-major QKV weight and read the query columns)
  const int N = m->bf16 ? nq_of(d) : nq_of(d) + 2 * nv_of(d);
  int sp = 1;
  CHK(gemm(m, st, B * K, B, D, N, m->ps_A, w.w_qkv, m->ps_nsel, m->part, m->part_floats, &sp, DLLM_PROF_GEMM,
           m->ps_MTt));
  // query partials read, queries written, window keys per head, log-attention
  // read and written
  Prof prof2(m, st, DLLM_PROF_POLESTAR,
             (double)sp * B * K * Hq * dh * 4.0 + (double)B * K * Hq * dh * es + Bw * Hq * dh * es +
                 (double)B * K * Hq * W * 16.0,
             2.0 * B * K * (double)Hq * W * dh);
  HIPCHK(launch_ps_queries(st, m->bf16, B, L, blk, W, K, Hq, dh, sp, N, s->block_start, m->part, m->rope_cos,
                           m->rope_sin, ps->queries));
  double* la = ps->log_attn + (size_t)layer * B * K * Hq * W;
  HIPCHK(launch_ps_attn_kl(st, m->bf16, B, L, blk, W, K, Hq, d.n_kv_heads, dh, s->block_start, ps->queries,
                           kcache(m, const_cast<dllm_state*>(s), layer), la, m->ps_klp, p->tau_upd,
                           ps->win_start + (size_t)layer * B, s->n_history, ps->upd_hist + (size_t)layer * B));
  prof2.done();
  return DLLM_OK;
}

dllm_status do_polestar_select(dllm_model* m, int layer, const dllm_state* s, dllm_polestar_state* ps,
                               const dllm_polestar_params* p, int32_t* idx, int32_t* n, hipStream_t st) {
  const dllm_dims& d = m->d;
  const int B = s->batch, W = p->window_blocks * d.block_len;
  Prof prof(m, st, DLLM_PROF_SELECT, (double)B * d.n_q_heads * p->n_clusters * 8.0 + (double)B * W * 8.0, 0.0);
  HIPCHK(launch_ps_select(st, B, d.seq_len, d.block_len, W, p->n_clusters, d.n_q_heads, p->top_clusters,
                          s->block_start, ps->assign, m->ps_klp, ps->win_start + (size_t)layer * B, ps->kl, ps->top,
                          idx, n, ps->drift_valid, p->tau_upd, s->n_history, ps->upd_hist + (size_t)layer * B));
  prof.done();
  return DLLM_OK;
}

}  // namespace

extern "C" {

const char* dllm_last_error(void) { return g_err.c_str(); }

dllm_status dllm_create(const dllm_dims* dims, dllm_model** out) {
  if (!dims || !out) return fail(DLLM_E_ARG, "dims/out is NULL");
  *out = nullptr;
  const dllm_dims& d = *dims;
  if (d.n_layers < 1 || d.d_model < 1 || d.n_q_heads < 1 || d.n_kv_heads < 1 || d.head_dim < 2 || d.d_ffn < 1 ||
      d.vocab < 2 || d.max_batch < 1 || d.seq_len < 1 || d.block_len < 1 || d.proxy_rank < 1)
    return fail(DLLM_E_ARG, "non-positive dimension");
  if (d.dtype != DLLM_FP32 && d.dtype != DLLM_BF16) return fail(DLLM_E_ARG, "unknown dtype %d", d.dtype);
  if (d.head_dim % 32 || d.head_dim > 256) return fail(DLLM_E_SHAPE, "head_dim must be a multiple of 32 and <= 256");
  if (d.d_model > 8192) return fail(DLLM_E_SHAPE, "d_model %d > 8192", d.d_model);
  if (d.n_q_heads % d.n_kv_heads) return fail(DLLM_E_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (d.seq_len > 8192) return fail(DLLM_E_SHAPE, "seq_len %d > 8192", d.seq_len);
  if (d.seq_len % 4) return fail(DLLM_E_SHAPE, "seq_len must be a multiple of 4");
  if (d.block_len > 64) return fail(DLLM_E_SHAPE, "block_len %d > 64", d.block_len);
  if (d.proxy_rank > 128 || d.proxy_rank > d.d_model) return fail(DLLM_E_SHAPE, "proxy_rank must be <= 128 and <= d_model");
  if (d.d_model % 32 || d.d_ffn % 32) return fail(DLLM_E_SHAPE, "d_model and d_ffn must be multiples of 32");
  if (!(d.rms_eps >= 0.f) || !(d.rope_theta > 0.f)) return fail(DLLM_E_ARG, "bad rms_eps/rope_theta");
  const int nq = nq_of(d), nv = nv_of(d);
  if (d.dtype == DLLM_BF16) {
    if (d.d_model % 64 || d.d_ffn % 64 || nq % 64 || nv % 32 || d.vocab % 32)
      return fail(DLLM_E_SHAPE, "bf16 widths: d_model, d_ffn, n_q*head_dim multiples of 64; n_kv*head_dim, vocab multiples of 32");
  }
  dllm_model* m = new dllm_model();
  m->d = d;
  m->bf16 = d.dtype == DLLM_BF16;
  m->esize = m->bf16 ? 2 : 4;
  m->layers.resize(d.n_layers);
  auto cleanup = [&](dllm_status st) {
    std::string keep = g_err;
    dllm_destroy(m);
    g_err = keep;
    return st;
  };
  {
    hipError_t e = hipGetDevice(&m->device);
    if (e != hipSuccess) return cleanup(fail(DLLM_E_HIP, "hipGetDevice: %s", hipGetErrorString(e)));
    // the device address of the allocation-free basis workspace, once per device
    e = proxy_basis_static_setup(m->device);
    if (e != hipSuccess)
      return cleanup(fail(DLLM_E_HIP, "fixed proxy-basis workspace (hipGetSymbolAddress): %s", hipGetErrorString(e)));
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, m->device) == hipSuccess && prop.multiProcessorCount > 0)
    m->n_cu = prop.multiProcessorCount;
  const int L = d.seq_len, D = d.d_model, F = d.d_ffn;
  m->M_cap = d.max_batch * L;
  m->M_pad = (m->M_cap + 31) / 32 * 32 + 32;
  m->MTt = m->M_pad / 32;
  const size_t es = m->esize;
  dllm_status st;
#define ALLOC(ptr, bytes)                         \
  do {                                            \
    st = m->alloc((void**)&(ptr), (bytes));       \
    if (st != DLLM_OK) return cleanup(st);        \
  } while (0)
  const size_t apad = gemm_pad_elems(m->MTt) * es;  // packed activations are read past their end
  ALLOC(m->A1, (size_t)m->M_pad * D * es + apad);
  ALLOC(m->q, (size_t)m->M_pad * nq * es);
  ALLOC(m->attn_o, (size_t)m->M_pad * nq * es + apad);
  ALLOC(m->A2, (size_t)m->M_pad * D * es + apad);
  ALLOC(m->act, (size_t)m->M_pad * F * es + apad);
  ALLOC(m->hprime, (size_t)m->M_pad * D * 4);
  {
    const int nmax = std::max(std::max(nq + 2 * nv, 2 * F), D);
    // split-K partials: the sparse GEMMs split up to 16x; full passes use few splits
    m->part_floats = (size_t)std::max(m->M_cap, 16 * 320) * nmax;
    ALLOC(m->part, m->part_floats * 4);
  }
  m->ppart_doubles = proxy_partial_doubles(m->M_cap, D, d.proxy_rank);
  ALLOC(m->ppart, m->ppart_doubles * 8);
  for (int i = 0; i < 2; ++i) {
    ALLOC(m->idx[i], (size_t)m->M_cap * 4);
    ALLOC(m->nsel[i], (size_t)d.max_batch * 4);
  }
  ALLOC(m->idx0, (size_t)m->M_cap * 4);
  ALLOC(m->n0, (size_t)d.max_batch * 4);
  ALLOC(m->forced, (size_t)m->M_cap);
  ALLOC(m->step_full, (size_t)d.max_batch);
  const int lm_rows_cap = d.max_batch * 2 * d.block_len;  // current and next block (Polestar-Commit)
  m->lm_MTt = (lm_rows_cap + 31) / 32 + 1;
  ALLOC(m->A_lm, (size_t)m->lm_MTt * 32 * D * es + gemm_pad_elems(m->lm_MTt) * es);
  ALLOC(m->logits, (size_t)lm_rows_cap * d.vocab * 4);
  m->lm_slabs = lm_stats_slabs(d.vocab);
  ALLOC(m->lm_part, (size_t)lm_rows_cap * m->lm_slabs * 4 * 8);
  ALLOC(m->lm_stats, (size_t)lm_rows_cap * 4 * 8);
  if (m->bf16 && d.vocab % 128 == 0)
    ALLOC(m->lm_wpart, (size_t)std::min(lm_rows_cap, LM_FUSED_ROWS) * (d.vocab / 128) * 4 * 8);
  ALLOC(m->lm_rows, 16);
  if (D % 128 == 0) {
    const size_t wmax = 120;
    ALLOC(m->ps_R, (size_t)d.max_batch * ps_gram_splits() * wmax * wmax * 8);
    ALLOC(m->ps_coef, (size_t)d.max_batch * 16 * wmax * 8);
    ALLOC(m->ps_klp, (size_t)d.max_batch * d.n_q_heads * 16 * 8);
    ALLOC(m->ps_nsel, (size_t)d.max_batch * 4);
    m->ps_MTt = (d.max_batch * 16 + 31) / 32 + 1;
    ALLOC(m->ps_A, (size_t)m->ps_MTt * 32 * D * es + gemm_pad_elems(m->ps_MTt) * es);
  }
  ALLOC(m->res_dev, 64);
  if (hipHostMalloc(&m->res_host, 64, hipHostMallocDefault) != hipSuccess)
    return cleanup(fail(DLLM_E_NOMEM, "hipHostMalloc failed"));
  if (hipHostMalloc((void**)&m->full_host, (size_t)d.max_batch + 16, hipHostMallocDefault) != hipSuccess)
    return cleanup(fail(DLLM_E_NOMEM, "hipHostMalloc failed"));
  // RoPE tables: angle = pos * theta^(-2j/dh), computed in fp64 on the host
  {
    const int half = d.head_dim / 2;
    std::vector<float> c((size_t)L * half), sn((size_t)L * half);
    for (int p = 0; p < L; ++p)
      for (int j = 0; j < half; ++j) {
        const double inv = std::pow((double)d.rope_theta, -(2.0 * j) / d.head_dim);
        const double a = (double)p * inv;
        c[(size_t)p * half + j] = (float)std::cos(a);
        sn[(size_t)p * half + j] = (float)std::sin(a);
      }
    ALLOC(m->rope_cos, c.size() * 4);
    ALLOC(m->rope_sin, sn.size() * 4);
    if (hipMemcpy(m->rope_cos, c.data(), c.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(m->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
      return cleanup(fail(DLLM_E_HIP, "RoPE table upload failed"));
  }
#undef ALLOC
  *out = m;
  g_err.clear();
  return DLLM_OK;
}

dllm_status dllm_destroy(dllm_model* m) {
  if (!m) return DLLM_OK;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : m->ev_all) (void)hipEventDestroy(e);
  for (void* p : m->allocs) (void)hipFree(p);
  if (m->res_host) (void)hipHostFree(m->res_host);
  if (m->full_host) (void)hipHostFree(m->full_host);
  delete m;
  return DLLM_OK;
}

dllm_status basis_supported(const dllm_model* m) {
  const dllm_dims& d = m->d;
  if (d.proxy_rank > 128 || proxy_basis_width(d.d_model, nv_of(d), d.proxy_rank) < d.proxy_rank)
    return fail(DLLM_E_UNSUPPORTED, "proxy basis: need proxy_rank <= 128 and a subspace of at least r columns");
  return DLLM_OK;
}

// The derivation on a given workspace and status word; waits for the stream.
dllm_status run_derive(dllm_model* m, const void* w_v, int iters, double* wr, double* ws, int32_t* status,
                       hipStream_t st) {
  const dllm_dims& d = m->d;
  int32_t st_h = 0;
  hipError_t e = launch_proxy_basis(st, m->bf16, d.d_model, nv_of(d), d.proxy_rank, iters, w_v, wr, ws, status);
  if (e == hipSuccess) e = hipMemcpyAsync(&st_h, status, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(DLLM_E_HIP, "proxy basis: %s", hipGetErrorString(e));
  if (st_h != 0) return fail(DLLM_E_NUMERIC, "proxy basis: a Cholesky pivot was not positive");
  return DLLM_OK;
}

// W_r [d][r] fp64 from the value projection (device, storage dtype); waits
// for the stream and frees its workspace.
dllm_status derive_basis(dllm_model* m, const void* w_v, int iters, double* wr, hipStream_t st) {
  const dllm_dims& d = m->d;
  CHK(basis_supported(m));
  double* ws = nullptr;
  int32_t* status = nullptr;
  if (hipMalloc((void**)&ws, proxy_basis_workspace_doubles(d.d_model, nv_of(d), d.proxy_rank) * 8) != hipSuccess)
    return fail(DLLM_E_NOMEM, "proxy basis workspace");
  if (hipMalloc((void**)&status, 16) != hipSuccess) {
    (void)hipFree(ws);
    return fail(DLLM_E_NOMEM, "proxy basis workspace");
  }
  const dllm_status r = run_derive(m, w_v, iters, wr, ws, status, st);
  (void)hipFree(ws);
  (void)hipFree(status);
  return r;
}

dllm_status dllm_init_layer(dllm_model* m, int32_t layer, const dllm_layer_weights* w, void* stream) {
  CHK(check_model(m));
  if (!w) return fail(DLLM_E_ARG, "weights is NULL");
  if (layer < 0 || layer >= m->d.n_layers) return fail(DLLM_E_ARG, "layer %d outside [0, %d)", layer, m->d.n_layers);
  if (!w->attn_norm || !w->w_q || !w->w_k || !w->w_v || !w->w_o || !w->ffn_norm || !w->w_gate || !w->w_up ||
      !w->w_down)
    return fail(DLLM_E_ARG, "layer %d: a weight pointer is NULL", layer);
  const dllm_dims& d = m->d;
  const int D = d.d_model, F = d.d_ffn, nq = nq_of(d), nv = nv_of(d), r = d.proxy_rank;
  const size_t es = m->esize;
  LayerW& L = m->layers[layer];
  hipStream_t st = S(stream);
  if (!L.w_qkv) {
    CHK(m->alloc((void**)&L.attn_norm, (size_t)D * 4));
    CHK(m->alloc((void**)&L.ffn_norm, (size_t)D * 4));
    const size_t wpad = gemm_pad_elems(1) * es;  // the GEMM pipeline reads past the last chunk
    CHK(m->alloc(&L.w_qkv, (size_t)D * (nq + 2 * nv) * es + wpad));
    CHK(m->alloc(&L.w_o, (size_t)nq * D * es + wpad));
    CHK(m->alloc(&L.w_gu, (size_t)D * 2 * F * es + wpad));
    CHK(m->alloc(&L.w_down, (size_t)F * D * es + wpad));
    CHK(m->alloc((void**)&L.w_proxy, (size_t)D * proxy_rpad(r) * 4));
  }
  HIPCHK(hipMemcpyAsync(L.attn_norm, w->attn_norm, (size_t)D * 4, hipMemcpyDeviceToDevice, st));
  HIPCHK(hipMemcpyAsync(L.ffn_norm, w->ffn_norm, (size_t)D * 4, hipMemcpyDeviceToDevice, st));
  const int nqkv = nq + 2 * nv;
  CHK(pack(m, st, D, nq, w->w_q, L.w_qkv, nqkv, 0, 32));
  CHK(pack(m, st, D, nv, w->w_k, L.w_qkv, nqkv, nq, 32));
  CHK(pack(m, st, D, nv, w->w_v, L.w_qkv, nqkv, nq + nv, 32));
  CHK(pack(m, st, nq, D, w->w_o, L.w_o, D, 0, 32));
  if (m->bf16) {
    // gate and up columns 16 at a time inside each 32-column tile (gate in the
    // tile's first 16 columns, up in its last 16), so that every tile holds
    // complete SwiGLU pairs
    CHK(pack(m, st, D, F, w->w_gate, L.w_gu, 2 * F, 0, 32, 16));
    CHK(pack(m, st, D, F, w->w_up, L.w_gu, 2 * F, 16, 32, 16));
  } else {
    CHK(pack(m, st, D, F, w->w_gate, L.w_gu, 2 * F, 0, 64));
    CHK(pack(m, st, D, F, w->w_up, L.w_gu, 2 * F, 32, 64));
  }
  CHK(pack(m, st, F, D, w->w_down, L.w_down, D, 0, 32));
  if (w->w_proxy) {
    HIPCHK(launch_pad_proxy(st, D, r, w->w_proxy, L.w_proxy));
  } else {
    // derived in fp64, stored in fp32 like a supplied basis
    double* w64 = nullptr;
    float* w32 = nullptr;
    if (hipMalloc((void**)&w64, (size_t)D * r * 8) != hipSuccess) return fail(DLLM_E_NOMEM, "proxy basis buffer");
    if (hipMalloc((void**)&w32, (size_t)D * r * 4) != hipSuccess) {
      (void)hipFree(w64);
      return fail(DLLM_E_NOMEM, "proxy basis buffer");
    }
    dllm_status e = derive_basis(m, w->w_v, DLLM_PROXY_ITERS, w64, st);
    if (e == DLLM_OK && (launch_f64_to_f32(st, (size_t)D * r, w64, w32) != hipSuccess ||
                         launch_pad_proxy(st, D, r, w32, L.w_proxy) != hipSuccess))
      e = fail(DLLM_E_HIP, "proxy basis packing failed");
    if (e == DLLM_OK && hipStreamSynchronize(st) != hipSuccess) e = fail(DLLM_E_HIP, "hipStreamSynchronize failed");
    (void)hipFree(w64);
    (void)hipFree(w32);
    if (e != DLLM_OK) return e;
  }
  L.ready = true;
  return DLLM_OK;
}

dllm_status dllm_derive_proxy_basis(dllm_model* m, const void* w_v, int32_t iters, double* w_r_out, void* stream) {
  CHK(check_model(m));
  if (!w_v || !w_r_out) return fail(DLLM_E_ARG, "w_v/w_r_out is NULL");
  if (iters < 0) return fail(DLLM_E_ARG, "iters < 0");
  return derive_basis(m, w_v, iters, w_r_out, S(stream));
}

dllm_status dllm_derive_proxy_basis_noalloc(dllm_model* m, const void* w_v, int32_t iters, double* w_r_out,
                                            void* stream) {
  CHK(check_model(m));
  if (!w_v || !w_r_out) return fail(DLLM_E_ARG, "w_v/w_r_out is NULL");
  if (iters < 0) return fail(DLLM_E_ARG, "iters < 0");
  CHK(basis_supported(m));
  const dllm_dims& d = m->d;
  const size_t need = proxy_basis_workspace_doubles(d.d_model, nv_of(d), d.proxy_rank);
  if (need > PROXY_BASIS_STATIC_DOUBLES)
    return fail(DLLM_E_SHAPE, "proxy basis without allocation: the workspace needs %zu doubles, the fixed array "
                "holds %zu", need, (size_t)PROXY_BASIS_STATIC_DOUBLES);
  // set up at dllm_create on the model's device
  double* ws = proxy_basis_static_ws(m->device);
  if (!ws) return fail(DLLM_E_STATE, "the fixed workspace of device %d is not set up", m->device);
  return run_derive(m, w_v, iters, w_r_out, ws, (int32_t*)(ws + PROXY_BASIS_STATIC_DOUBLES), S(stream));
}

dllm_status dllm_init_head(dllm_model* m, const void* embed, const float* final_norm, const void* lm_head,
                           void* stream) {
  CHK(check_model(m));
  if (!embed || !final_norm || !lm_head) return fail(DLLM_E_ARG, "head pointer is NULL");
  const dllm_dims& d = m->d;
  hipStream_t st = S(stream);
  if (!m->embed) {
    CHK(m->alloc(&m->embed, (size_t)d.vocab * d.d_model * m->esize));
    CHK(m->alloc((void**)&m->final_norm, (size_t)d.d_model * 4));
    CHK(m->alloc(&m->lm_head, (size_t)d.d_model * d.vocab * m->esize + gemm_pad_elems(1) * m->esize));
  }
  HIPCHK(hipMemcpyAsync(m->embed, embed, (size_t)d.vocab * d.d_model * m->esize, hipMemcpyDeviceToDevice, st));
  HIPCHK(hipMemcpyAsync(m->final_norm, final_norm, (size_t)d.d_model * 4, hipMemcpyDeviceToDevice, st));
  CHK(pack(m, st, d.d_model, d.vocab, lm_head, m->lm_head, d.vocab, 0, 32));
  m->head_ready = true;
  return DLLM_OK;
}

dllm_status dllm_embed(dllm_model* m, const dllm_state* s, const int32_t* rows, const int32_t* n_rows, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s, false));
  if (!m->head_ready) return fail(DLLM_E_STATE, "head weights not initialised");
  if ((rows == nullptr) != (n_rows == nullptr)) return fail(DLLM_E_ARG, "rows and n_rows must both be set or NULL");
  hipStream_t st = S(stream);
  const int B = s->batch, L = m->d.seq_len;
  if (!rows) {
    HIPCHK(launch_all_rows(st, B, L, m->idx0, m->n0));
    rows = m->idx0;
    n_rows = m->n0;
  }
  HIPCHK(launch_embed(st, m->bf16, B * L, B, L, m->d.d_model, m->d.vocab, rows, n_rows, s->tokens, m->embed,
                      hid(m, s, 0)));
  return DLLM_OK;
}

dllm_status dllm_drift_score(dllm_model* m, int32_t layer, dllm_state* s, const int32_t* rows,
                             const int32_t* n_rows, int32_t max_rows, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s));
  CHK(check_layer(m, layer));
  if ((rows == nullptr) != (n_rows == nullptr)) return fail(DLLM_E_ARG, "rows and n_rows must both be set or NULL");
  hipStream_t st = S(stream);
  if (!rows) {
    HIPCHK(launch_all_rows(st, s->batch, m->d.seq_len, m->idx0, m->n0));
    rows = m->idx0;
    n_rows = m->n0;
    max_rows = s->batch * m->d.seq_len;
  }
  return do_drift(m, layer, s, rows, n_rows, clamp_rows(m, s, max_rows), st);
}

dllm_status dllm_select(dllm_model* m, int32_t layer, const dllm_state* s, const uint8_t* forced, const uint8_t* full,
                        double rho, int32_t* idx, int32_t* n_sel, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s));
  if (layer < 0 || layer >= m->d.n_layers) return fail(DLLM_E_ARG, "layer %d outside [0, %d)", layer, m->d.n_layers);
  if (!idx || !n_sel) return fail(DLLM_E_ARG, "idx/n_sel is NULL");
  if (!(rho >= 0.0)) return fail(DLLM_E_ARG, "rho must be >= 0");
  const int L = m->d.seq_len;
  const double kf = std::floor(rho * L + 0.5);
  const int k = kf > (double)L ? L : (int)kf;
  HIPCHK(launch_select(S(stream), s->batch, L, k, score(m, s, layer), forced, full, idx, n_sel));
  return DLLM_OK;
}

dllm_status dllm_sparse_layer(dllm_model* m, int32_t layer, dllm_state* s, const int32_t* idx, const int32_t* n_sel,
                              int32_t max_rows, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s));
  CHK(check_layer(m, layer));
  if (!idx || !n_sel) return fail(DLLM_E_ARG, "idx/n_sel is NULL");
  return do_sparse(m, layer, s, idx, n_sel, clamp_rows(m, s, max_rows), S(stream));
}

dllm_status dllm_lm_head(dllm_model* m, const dllm_state* s, double* stats_out, float* logits_out, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s, false));
  if (!m->head_ready) return fail(DLLM_E_STATE, "head weights not initialised");
  hipStream_t st = S(stream);
  const size_t rows = (size_t)s->batch * m->d.block_len;
  CHK(do_lm_head(m, s, st, 1, logits_out != nullptr));
  if (stats_out) HIPCHK(hipMemcpyAsync(stats_out, m->lm_stats, rows * 4 * 8, hipMemcpyDeviceToDevice, st));
  if (logits_out)
    HIPCHK(hipMemcpyAsync(logits_out, m->logits, rows * m->d.vocab * 4, hipMemcpyDeviceToDevice, st));
  return DLLM_OK;
}

dllm_status dllm_commit(dllm_model* m, dllm_state* s, double conf_threshold, double tau, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s, false));
  if (!m->head_ready) return fail(DLLM_E_STATE, "head weights not initialised");
  if (std::isnan(conf_threshold) || std::isnan(tau)) return fail(DLLM_E_ARG, "threshold is NaN");
  return do_commit(m, s, conf_threshold, tau, S(stream));
}

dllm_status dllm_commit_ce(dllm_model* m, dllm_state* s, const dllm_ce_params* ce, dllm_ce_state* ce_state,
                           double conf_threshold, double tau, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s, false));
  CHK(check_ce(m, ce, ce_state));
  if (!m->head_ready) return fail(DLLM_E_STATE, "head weights not initialised");
  if (std::isnan(conf_threshold) || std::isnan(tau)) return fail(DLLM_E_ARG, "threshold is NaN");
  return do_commit_ce(m, s, ce, ce_state, conf_threshold, tau, S(stream));
}

dllm_status dllm_polestar_commit(dllm_model* m, dllm_state* s, dllm_polestar_state* ps,
                                 const dllm_polestar_params* p, double conf_threshold, double tau, void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s, false));
  CHK(check_polestar(m, s, ps, p));
  if (!m->head_ready) return fail(DLLM_E_STATE, "head weights not initialised");
  if (std::isnan(conf_threshold) || std::isnan(tau)) return fail(DLLM_E_ARG, "threshold is NaN");
  if (!(p->commit_alpha >= 0.0)) return fail(DLLM_E_ARG, "commit_alpha must be >= 0");
  return do_polestar_commit(m, s, ps, p, conf_threshold, tau, S(stream));
}

dllm_status dllm_polestar_drift(dllm_model* m, int32_t layer, const dllm_state* s, dllm_polestar_state* ps,
                                const dllm_polestar_params* p, void* stream) {
  CHK(check_model(m));
  CHK(check_layer(m, layer));
  CHK(check_state(m, s, false));
  CHK(check_polestar(m, s, ps, p));
  return do_polestar_drift(m, layer, s, ps, p, S(stream));
}

dllm_status dllm_polestar_select(dllm_model* m, int32_t layer, const dllm_state* s, dllm_polestar_state* ps,
                                 const dllm_polestar_params* p, int32_t* idx, int32_t* n_sel, void* stream) {
  CHK(check_model(m));
  CHK(check_layer(m, layer));
  CHK(check_state(m, s, false));
  CHK(check_polestar(m, s, ps, p));
  if (!idx || !n_sel) return fail(DLLM_E_ARG, "idx/n_sel is NULL");
  return do_polestar_select(m, layer, s, ps, p, idx, n_sel, S(stream));
}

dllm_status dllm_forced_set(dllm_model* m, const dllm_state* s, int32_t rule, int32_t recent_k, uint8_t* forced,
                            void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s, false));
  if (!forced) return fail(DLLM_E_ARG, "forced is NULL");
  if (rule < DLLM_FORCED_NONE || rule > DLLM_FORCED_BLOCK_RECENT) return fail(DLLM_E_ARG, "unknown forced rule %d", rule);
  if (recent_k < 0) return fail(DLLM_E_ARG, "recent_k < 0");
  HIPCHK(launch_forced(S(stream), s->batch, m->d.seq_len, m->d.block_len, rule, recent_k, s->history, s->n_history,
                       s->block_start, forced));
  return DLLM_OK;
}

dllm_status dllm_step(dllm_model* m, dllm_state* s, const dllm_step_params* p, dllm_step_result* res_h,
                      void* stream) {
  CHK(check_model(m));
  CHK(check_state(m, s));
  if (!p || !p->rho_h) return fail(DLLM_E_ARG, "params/rho_h is NULL");
  if (p->mode < DLLM_MODE_AUTO || p->mode > DLLM_MODE_SPARSE) return fail(DLLM_E_ARG, "unknown mode %d", p->mode);
  if (p->forced_rule < DLLM_FORCED_NONE || p->forced_rule > DLLM_FORCED_BLOCK_RECENT)
    return fail(DLLM_E_ARG, "unknown forced rule %d", p->forced_rule);
  if (p->recent_k < 0) return fail(DLLM_E_ARG, "recent_k < 0");
  if (std::isnan(p->tau) || std::isnan(p->conf_threshold)) return fail(DLLM_E_ARG, "threshold is NaN");
  if ((p->sets_out == nullptr) != (p->n_sets_out == nullptr))
    return fail(DLLM_E_ARG, "sets_out and n_sets_out must both be set or NULL");
  if (p->score != DLLM_SCORE_SPA_COS && p->score != DLLM_SCORE_POLESTAR_KL)
    return fail(DLLM_E_ARG, "unknown score %d", p->score);
  const bool polestar = p->score == DLLM_SCORE_POLESTAR_KL;
  if (polestar) CHK(check_polestar(m, s, p->polestar_state, p->polestar));
  if (p->ce) {
    CHK(check_ce(m, p->ce, p->ce_state));
    if (polestar && p->polestar->drift_commit)
      return fail(DLLM_E_ARG, "Confidence Extrapolation and Polestar-Commit are exclusive");
  }
  const dllm_dims& d = m->d;
  for (int l = 0; l < d.n_layers; ++l) {
    CHK(check_layer(m, l));
    if (!(p->rho_h[l] >= 0.0)) return fail(DLLM_E_ARG, "rho[%d] must be >= 0", l);
  }
  if (!m->head_ready) return fail(DLLM_E_STATE, "head weights not initialised");
  hipStream_t st = S(stream);
  const int B = s->batch, L = d.seq_len;
  bool any_full = p->mode == DLLM_MODE_FULL;
  int mode = p->mode;
  if (p->mode == DLLM_MODE_AUTO) {
    HIPCHK(hipMemcpyAsync(m->full_host, s->full_next, (size_t)B, hipMemcpyDeviceToHost, st));
    HIPCHK(hipStreamSynchronize(st));
    for (int b = 0; b < B; ++b) any_full = any_full || m->full_host[b] != 0;
    // Polestar schedule: a periodic full pass of every sequence
    const int fp = polestar ? p->polestar->full_period : 0;
    if (fp > 0 && p->polestar_state->steps_since_full + 1 >= fp) {
      any_full = true;
      mode = DLLM_MODE_FULL;
    }
  }
  if (polestar && any_full && mode != DLLM_MODE_FULL) {
    // the entropy gate fired for some sequences only: the Polestar drift path
    // runs for every sequence of a step or for none
    int nf = 0;
    for (int b = 0; b < B; ++b) nf += m->full_host[b] != 0;
    if (nf != B)
      return fail(DLLM_E_UNSUPPORTED,
                  "Polestar drift path: the entropy gate fired for %d of %d sequences; a step is full or "
                  "sparse for every sequence (run the step in FULL or SPARSE mode)", nf, B);
  }
  if (polestar) {
    // the step is a full pass for every sequence exactly when mode is FULL
    p->polestar_state->steps_since_full = mode == DLLM_MODE_FULL ? 0 : p->polestar_state->steps_since_full + 1;
  }
  const int fmax = p->forced_rule == DLLM_FORCED_NONE ? 0
                   : (p->forced_rule == DLLM_FORCED_BLOCK ? d.block_len : d.block_len + p->recent_k);
  // rows whose token changed: the last commit's, at most one block (two with
  // Polestar-Commit's suffix-block commit)
  const int new_max = (polestar && p->polestar->drift_commit) ? 2 * d.block_len : d.block_len;
  int prev_max = any_full ? B * L : B * std::min(L, new_max);
  {
    Prof prof(m, st, DLLM_PROF_DECIDE, (double)B * L * 6.0 + 2.0 * prev_max * d.d_model * m->esize, 0.0);
    HIPCHK(launch_prep(st, B, L, d.block_len, p->forced_rule, p->recent_k, mode, s->history, s->n_history,
                       s->n_new, s->block_start, s->full_next, m->forced, m->step_full, m->idx0, m->n0));
    HIPCHK(launch_embed(st, m->bf16, prev_max, B, L, d.d_model, d.vocab, m->idx0, m->n0, s->tokens, m->embed,
                        hid(m, s, 0)));
    prof.done();
  }
  const int32_t* prev_idx = m->idx0;
  const int32_t* prev_n = m->n0;
  if (polestar && !any_full) {
    // Polestar-Cache: the cluster drift path picks the rows of every layer
    const int W = p->polestar->window_blocks * d.block_len;
    for (int l = 0; l < d.n_layers; ++l) {
      int32_t* idx = m->idx[l & 1];
      int32_t* n = m->nsel[l & 1];
      CHK(do_polestar_drift(m, l, s, p->polestar_state, p->polestar, st));
      CHK(do_polestar_select(m, l, s, p->polestar_state, p->polestar, idx, n, st));
      CHK(do_sparse(m, l, s, idx, n, B * W, st, false));
      CHK(save_sets(m, s, p, l, idx, n, st));
    }
    if (p->polestar->drift_commit)
      CHK(do_polestar_commit(m, s, p->polestar_state, p->polestar, p->conf_threshold, p->tau, st));
    else if (p->ce)
      CHK(do_commit_ce(m, s, p->ce, p->ce_state, p->conf_threshold, p->tau, st));
    else
      CHK(do_commit(m, s, p->conf_threshold, p->tau, st));
    return finish_step(m, s, res_h, st);
  }
  for (int l = 0; l < d.n_layers; ++l) {
    CHK(do_drift(m, l, s, prev_idx, prev_n, prev_max, st));
    const double kf = std::floor(p->rho_h[l] * L + 0.5);
    const int k = kf > (double)L ? L : (int)kf;
    int32_t* idx = m->idx[l & 1];
    int32_t* n = m->nsel[l & 1];
    const int rows = any_full ? B * L : B * std::min(L, std::max(k, fmax));
    // one sequence and a small row bound: every gather workgroup selects for
    // itself (no selection launch); otherwise the selection, then the gather
    const bool fused = B == 1 && rows <= SG_MAX_ROWS;
    if (fused) {
      Prof prof(m, st, DLLM_PROF_SELECT, (double)L * 13.0 + 2.0 * rows * d.d_model * m->esize + d.d_model * 4.0,
                4.0 * rows * (double)d.d_model);
      HIPCHK(launch_select_gather(st, m->bf16, rows, L, d.d_model, d.rms_eps, m->MTt, k, score(m, s, l), m->forced,
                                  m->step_full, hid(m, s, l), m->layers[l].attn_norm, idx, n, m->A1));
      prof.done();
    } else {
      Prof prof(m, st, DLLM_PROF_SELECT, (double)B * L * 13.0, 0.0);
      HIPCHK(launch_select(st, B, L, k, score(m, s, l), m->forced, m->step_full, idx, n));
      prof.done();
    }
    CHK(do_sparse(m, l, s, idx, n, rows, st, true, fused));
    CHK(save_sets(m, s, p, l, idx, n, st));
    prev_idx = idx;
    prev_n = n;
    prev_max = rows;
  }
  if (polestar && p->polestar->drift_commit)
    CHK(do_polestar_commit(m, s, p->polestar_state, p->polestar, p->conf_threshold, p->tau, st));
  else if (p->ce)
    CHK(do_commit_ce(m, s, p->ce, p->ce_state, p->conf_threshold, p->tau, st));
  else
    CHK(do_commit(m, s, p->conf_threshold, p->tau, st));
  return finish_step(m, s, res_h, st);
}

dllm_status dllm_stream_probe(const void* dev_buf, size_t bytes, void* dev_scratch, int32_t reps, double* gbps_h,
                              void* stream) {
  if (!dev_buf || !dev_scratch || !gbps_h) return fail(DLLM_E_ARG, "stream probe: NULL pointer");
  if (reps < 1) return fail(DLLM_E_ARG, "stream probe: reps < 1");
  if (bytes < ((size_t)256 << 20)) return fail(DLLM_E_ARG, "stream probe: need at least 256 MiB");
  const size_t use = bytes / ((size_t)64 << 20) * ((size_t)64 << 20);
  hipStream_t st = S(stream);
  hipEvent_t a = nullptr, b = nullptr;
  HIPCHK(hipEventCreate(&a));
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return fail(DLLM_E_HIP, "hipEventCreate failed");
  }
  double best = 0.0;
  hipError_t e = hipSuccess;
  const int grids[2] = {1024, 2048}, depths[2] = {4, 8};
  for (int gi = 0; gi < 2 && e == hipSuccess; ++gi)
    for (int di = 0; di < 2 && e == hipSuccess; ++di) {
      e = launch_stream_probe(st, grids[gi], depths[di], dev_buf, use, (unsigned*)dev_scratch);
      if (e == hipSuccess) e = hipEventRecord(a, st);
      for (int r = 0; r < reps && e == hipSuccess; ++r)
        e = launch_stream_probe(st, grids[gi], depths[di], dev_buf, use, (unsigned*)dev_scratch);
      if (e == hipSuccess) e = hipEventRecord(b, st);
      if (e == hipSuccess) e = hipEventSynchronize(b);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      if (e == hipSuccess && ms > 0.f) best = std::max(best, (double)use * reps / (ms * 1e-3) / 1e9);
    }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (e != hipSuccess) return fail(DLLM_E_HIP, "stream probe: %s", hipGetErrorString(e));
  *gbps_h = best;
  return DLLM_OK;
}

dllm_status dllm_profile(dllm_model* m, int32_t class_mask) {
  CHK(check_model(m));
  m->prof_mask = class_mask & ((1 << DLLM_PROF_N) - 1);
  m->prof_on = m->prof_mask != 0;
  return DLLM_OK;
}

dllm_status dllm_profile_read(dllm_model* m, dllm_kernel_stats* stats_h) {
  CHK(check_model(m));
  if (!stats_h) return fail(DLLM_E_ARG, "stats_h is NULL");
  for (int c = 0; c < DLLM_PROF_N; ++c) stats_h[c] = dllm_kernel_stats{0, 0.0, 0.0, 0.0};
  for (auto& r : m->prof_pending) {
    HIPCHK(hipEventSynchronize(r.b));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, r.a, r.b));
    dllm_kernel_stats& k = stats_h[r.cls];
    k.launches += 1;
    k.ms += ms;
    k.bytes += r.bytes;
    k.flops += r.flops;
    m->ev_pool.push_back(r.a);
    m->ev_pool.push_back(r.b);
  }
  m->prof_pending.clear();
  return DLLM_OK;
}

}  // extern "C"
