// Bidirectional attention of the selected (sparse) queries over every cached
// row (SPA-Cache method step 3: the sparse queries attend over the partially
// updated KV cache; dLLM attention is non-causal, so there is no mask).
// Query head h reads KV head floor(h * Hkv / Hq).
//
// Cache layouts: K is stored in matrix-core fragment order (kc_off), so every
// key fragment a wave needs is one contiguous 1 KB load (16 bytes per lane)
// straight into registers.  V is stored row-major ([key][dh] per sequence and
// KV head), so the QKV epilogue writes a refreshed key's values as whole
// contiguous pieces; the attention moves each 32-key value tile into LDS by
// DMA (1 KB per request, contiguous in memory) and builds the value operand
// with transposed LDS reads (ds_read_b64_tr_b16).
//
// bf16, dh in {64, 128}, L % 32 == 0: MFMA flash attention.  A workgroup owns
// 32 query rows of one sequence and one head; its 8 waves split the keys and
// each keeps an online softmax (fp32) over 32-key tiles, computing S^T = K Q^T
// (so a query's scores sit in one lane pair and the row max/sum need one
// cross-lane exchange) and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16.  The
// next tile's key fragments are in flight during the current tile; its value
// tile is requested as soon as the current one has been read.  The eight
// partial results are merged in one LDS round (over the value buffers), each
// wave combining and storing an eighth of the output in a fixed wave order.
// Otherwise a reference kernel (one wave per query row and head).
#include "common.h"
#include "kernels.h"

namespace dllm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

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
  const T* K = Kc + ((size_t)b * Hkv + g) * (size_t)l32_of(L) * dh;
  const T* V = Vc + ((size_t)b * Hkv + g) * (size_t)l32_of(L) * dh;
  float mx = -INFINITY;
  for (int j = lane; j < L; j += 64) {
    float s = 0.f;
    for (int t = 0; t < dh; ++t) s = fmaf(qs[t], io<T>::ld(K + kc_off(j, t, dh)), s);
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
    for (int j = 0; j < L; ++j) acc = fmaf(ps[j], io<T>::ld(V + (size_t)j * dh + t), acc);
    store_a1(out, m, h * dh + t, MTt, Hq * dh, acc * inv);
  }
}

constexpr int ATT_NW = 8;
constexpr int ATT_ONE_ROUND = 256;  // (query tile, head) workgroups of 8 waves that fit one round (one per CU)
constexpr int ATT_HALF_MAX_KEYS = 1024;  // longest cache the 4-wave variant takes
// The running maximum of a query's scores (log2 units) moves only when a key
// tile's maximum passes it by more than this.  Softmax is shift-invariant, so
// any value at or below the true maximum gives the same result; a stale one
// only lets the probabilities grow up to 2^ATT_M_SLACK (far inside bf16 and
// fp32 range), and a tile that moves no lane's maximum skips the rescale of
// the output accumulators, which is most of a tile's vector work.
constexpr float ATT_M_SLACK = 8.0f;

typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <int DH, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_mfma_kernel(int B, int L, int Hq, int Hkv, int ntq, float sl2e, int cap,
                                                                const int32_t* __restrict__ n,
                                                                const bf16* __restrict__ q,
                                                                const bf16* __restrict__ Kc,
                                                                const bf16* __restrict__ Vc,
                                                                bf16* __restrict__ out, int MTt) {
  constexpr int KS = DH / 16;   // k-steps of S^T
  constexpr int DT = DH / 32;   // d-tiles of O^T
  constexpr int RB = DH * 2;    // bytes of one key's values
  constexpr int VT = 32 * RB;   // bytes of a 32-key value tile
  constexpr int NV = VT / 1024; // 1 KB DMA requests per value tile
  constexpr int RPI = 1024 / RB;  // key rows per request
  constexpr int CPR = DH / 8;     // 16-byte chunks per key row
  constexpr int VBUF = 2 * NW * VT;              // two value tiles per wave
  constexpr int OXB = NW * DT * 16 * 64 * 4;     // the merge's partial outputs
  // the value tiles during the key loop, the merge's partial outputs after it
  __shared__ __attribute__((aligned(16))) unsigned char smem[VBUF > OXB ? VBUF : OXB];
  __shared__ float ms[NW][32], ls[NW][32];
  // Workgroups are dealt round-robin to the 8 XCDs; remap so that the query
  // tiles of one head run on one XCD and share its K/V through that L2.
  const int G = gridDim.x;  // ntq * Hq rounded up to a multiple of 8
  const int wl = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int h = wl / ntq;
  if (h >= Hq) return;
  // query tile -> (sequence, first compact row)
  int T = wl - h * ntq, b = -1, off = 0, nb = 0;
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
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, hlf = lane >> 5,
            ln = lane & 31;

  // Q^T fragments (B operand): lane holds q[r0 + ln][h*DH + ks*16 + 8*hlf + 0..7]
  u32x4 qf[KS];
  const bool qv = ln < nqv;
  const bf16* qrow = q + (size_t)(r0 + ln) * Hq * DH + (size_t)h * DH + 8 * hlf;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = qv ? *reinterpret_cast<const u32x4*>(qrow + ks * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  const bf16* Kb = Kc + ((size_t)b * Hkv + g) * (size_t)l32_of(L) * DH;
  const bf16* Vb = Vc + ((size_t)b * Hkv + g) * (size_t)l32_of(L) * DH;
  const int ntiles = L >> 5;
  const int t_beg = (wv * ntiles) / NW, t_end = ((wv + 1) * ntiles) / NW;

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // K fragment (A operand of S^T) of key tile kt and dims ks*16 ..: 1 KB at
  // ((kt*KS + ks)*64 + lane)*8, straight into registers.
  auto load_k = [&](int kt, u32x4 (&k)[KS]) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(Kb) + (size_t)kt * KS * 64 + lane;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k[ks] = kp[ks * 64];
  };
  // Value tile kt (32 key rows of DH values, row-major in the cache) into
  // this wave's LDS buffer by DMA (1 KB, RPI rows, per request).  Chunk c of
  // key row r is stored in slot c ^ vswz(r), so that the transposed reads
  // below touch every bank once per half-wave.  The requests are issued from
  // inline asm (the compiler would otherwise make every LDS read wait for
  // them); each tile starts with a wait for every load in flight, which were
  // all issued one tile earlier, so the value tile read in a tile has landed.
  auto vswz = [](int r) { return DH == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  lds_u8* vbuf = (lds_u8*)smem + wv * 2 * VT;
  // lane byte offset inside a request; vswz(r) depends on r % 4 only, and
  // every request starts at a multiple of 4 rows
  const unsigned voff = (unsigned)((lane / CPR) * RB + 16 * ((lane % CPR) ^ vswz(lane / CPR)));
  auto load_v = [&](int kt, int buf) {
    const void* src = uniform_ptr(Vb + (size_t)kt * 32 * DH);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is only ever set here
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const unsigned l = (unsigned)(uintptr_t)(vbuf + buf * VT + i * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(l)),
                   "v"(voff + i * 1024u), "s"(src)
                   : "memory", "m0");
    }
#pragma clang diagnostic pop
  };
  // V^T fragment (A operand of O^T) of 16-key half kk and dims dt*32 ..:
  // lane l needs value [key 16 kk + 4 (l/32) + e%4 + 8 (e/4)][dim dt*32 + l%32]
  // for e = 0..7 (the key order of the score accumulator's rows).  Two
  // transposed 64-bit LDS reads give e = 0..3 and e = 4..7: in each group of
  // 16 lanes, lane j reads the 4 dims 4 (j%4) .. of key j/4, and lane i of
  // the group receives dim i of those 4 keys.
  const int jq = lane & 15, Gq = lane >> 4;
  const int mf = DH == 128 ? (jq >> 2) : (jq >> 3);  // vswz of the lane's key, over 4
  int vrd[DT];  // byte offset in a value tile for kk = 0 and keys +0..3
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    vrd[dt] = (4 * (Gq >> 1) + (jq >> 2)) * RB + (4 * (dt ^ mf) + 2 * (Gq & 1) + ((jq & 3) >> 1)) * 16 + 8 * (jq & 1);
  auto read_v = [&](int buf, int kk, u32x4 (&vf)[DT]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
      const lds_u8* a = vbuf + buf * VT + kk * 16 * RB + vrd[dt];
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)a);
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a + 8 * RB));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      vf[dt] = u32x4{l2.x, l2.y, h2.x, h2.y};
    }
  };
  // one key tile: S^T, online softmax, then the value tile's reads, the next
  // value tile's request (into the other buffer, read two tiles ago), O^T
  // kf holds this tile's key fragments; the next tile's (index kn) go into
  // kn_f, its value tile (index vnext, none if negative) into the other buffer
  auto tile = [&](const u32x4 (&kf)[KS], u32x4 (&kn_f)[KS], int kn, int buf, bool rescale, int vnext) {
    // this tile's key fragments and value tile (both requested one tile ago)
    // have landed; the other value buffer was read by the previous tile
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
    __builtin_amdgcn_sched_barrier(0);
    if (vnext >= 0) load_v(vnext, buf ^ 1);
    load_k(kn, kn_f);
    __builtin_amdgcn_sched_barrier(0);
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
    const float m_new = mt > m_run + ATT_M_SLACK ? mt : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 where m_run stays
    // probabilities packed to bf16 as they are made (P^T operands of the two
    // 16-key halves); the row sum in element order
    u32x4 pf[2];
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * e], sl2e, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * e + 1], sl2e, -m_new));
        rs += p0;
        rs += p1;
        pf[kk][e] = pack2bf(p0, p1);
      }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    // o is still zero on a wave's first tile; a multiply by 1 is skipped
    if (rescale && __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
    // the value reads stay after the softmax: the wait for this tile's value
    // request comes as late as possible
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 vf[DT];
      read_v(buf, kk, vf);
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pf[kk]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[dt]), pb, o[dt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // one half's value fragments live at a time
    }
  };

  // the next key tile's fragments and value tile are in flight during the
  // current tile
  if (t_beg < t_end) {
    u32x4 ka[KS], kb[KS];
    load_k(t_beg, ka);
    load_v(t_beg, 0);
    // (the key prefetch index is clamped, so every load is unconditional and
    // in range; the value request is skipped past the last tile)
    for (int kt = t_beg; kt < t_end; kt += 2) {
      tile(ka, kb, min(kt + 1, t_end - 1), 0, kt != t_beg, kt + 1 < t_end ? kt + 1 : -1);
      if (kt + 1 >= t_end) break;
      tile(kb, ka, min(kt + 2, t_end - 1), 1, true, kt + 2 < t_end ? kt + 2 : -1);
    }
  }

  // merge the waves' partial softmax states in one LDS round: every wave
  // writes (m, l, O), then wave w combines the output groups (dt, q4) it owns
  // from all NW waves in a fixed order and stores them.  The partial
  // outputs reuse the value buffers: every wave's reads (and requests) are
  // done first.
  static_assert((DT * 4) % NW == 0, "output groups per wave");
  constexpr int GPW = DT * 4 / NW;
  float (*ox)[DT][16][64] = reinterpret_cast<float (*)[DT][16][64]>(smem);  // element i of lane l at [i][l]
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no request still writing LDS
  __syncthreads();
  if (lane < 32) {
    ms[wv][ln] = m_run;
    ls[wv][ln] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) ox[wv][dt][i][lane] = o[dt][i];
  __syncthreads();
  float mg = ms[0][ln];
#pragma unroll
  for (int w2 = 1; w2 < NW; ++w2) mg = fmaxf(mg, ms[w2][ln]);
  float fw[NW], lg = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) {
    fw[w2] = exp2f(ms[w2][ln] - mg);  // 0 for a wave without keys
    lg += ls[w2][ln] * fw[w2];
  }
  const float inv = 1.0f / lg;
  const int m = r0 + ln;
#pragma unroll
  for (int gg = 0; gg < GPW; ++gg) {
    const int gr = wv * GPW + gg, dt = gr >> 2, q4 = gr & 3;
    float mine[4], part[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) acc += ox[w2][dt][q4 * 4 + e][lane] * fw[w2];
      mine[e] = acc * inv;
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

// ---------------------------------------------------------------------------
// Grouped-query attention (4 <= Hq/Hkv <= 8, bf16, dh in {64, 128}): a
// workgroup owns 32 query rows of one sequence and every query head of one KV
// head.  Wave w < Hq/Hkv owns query head g*(Hq/Hkv) + w over all the keys, so
// the waves' results need no merge.  Each 32-key tile of keys (fragment order)
// and values (row-major, chunks XOR-swizzled as above) is moved into LDS once
// per workgroup by DMA, 1 KB requests spread over the 8 waves, in a ring of
// GQ_NB slots, and read by all the group's waves: the L2 reads of a KV head's
// cache shrink by the group size against one workgroup per query head.  Every
// GQ_TPB tiles: a wait for this wave's requests of those tiles, a workgroup
// barrier (every wave's requests visible, every wave done with the slots about
// to be refilled), the requests of the tiles GQ_NB - GQ_TPB ahead; then each
// tile's arithmetic as in attn_mfma_kernel.
// ---------------------------------------------------------------------------
constexpr int GQ_TPB = 1;           // key tiles per barrier (2 measured no faster)
constexpr int GQ_NB = 4 * GQ_TPB;  // ring slots (key tiles)

// Four waves per SIMD (at most 128 VGPRs; 10 spill, 28 bytes of scratch): two
// workgroups share a CU, so more (query tile, KV head) pairs than CUs run in
// one round instead of two.
template <int DH>
__global__ __launch_bounds__(ATT_NW * 64, 4) void attn_gqa_kernel(int B, int L, int Hq, int Hkv, int ntq, float sl2e, int cap,
                                                               const int32_t* __restrict__ n,
                                                               const bf16* __restrict__ q,
                                                               const bf16* __restrict__ Kc,
                                                               const bf16* __restrict__ Vc,
                                                               bf16* __restrict__ out, int MTt) {
  constexpr int KS = DH / 16;     // k-steps of S^T (1 KB key fragments per tile)
  constexpr int DT = DH / 32;     // d-tiles of O^T
  constexpr int RB = DH * 2;      // bytes of one key's values
  constexpr int KTB = 32 * RB;    // bytes of a key tile
  constexpr int SLOT = 2 * KTB;   // key tile, then value tile
  constexpr int NREQ = SLOT / 1024;
  static_assert(NREQ % ATT_NW == 0, "requests per wave");
  constexpr int RPW = NREQ / ATT_NW;  // 1 KB requests per wave per tile
  constexpr int RPI = 1024 / RB;      // value rows per request
  constexpr int CPR = DH / 8;         // 16-byte chunks per value row
  constexpr int P = GQ_NB - GQ_TPB;   // tiles requested ahead
  __shared__ __attribute__((aligned(16))) unsigned char smem[GQ_NB * SLOT];
  const int G = gridDim.x;  // ntq * Hkv rounded up to a multiple of 8
  // a KV head's query tiles side by side on one XCD (its K/V shared in L2)
  const int wl = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int grp = wl / ntq;
  if (grp >= Hkv) return;
  // query tile -> (sequence, first compact row)
  int T = wl - grp * ntq, b = -1, off = 0, nb = 0;
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
  const int GQ = Hq / Hkv;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, hlf = lane >> 5,
            ln = lane & 31;
  const bool comp = wv < GQ;  // waves past the group only move tiles
  const int h = grp * GQ + (comp ? wv : 0);

  // Q^T fragments (B operand): lane holds q[r0 + ln][h*DH + ks*16 + 8*hlf + 0..7]
  u32x4 qf[KS];
  const bool qv = ln < nqv;
  const bf16* qrow = q + (size_t)(r0 + ln) * Hq * DH + (size_t)h * DH + 8 * hlf;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = (qv && comp) ? *reinterpret_cast<const u32x4*>(qrow + ks * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  const bf16* Kb = Kc + ((size_t)b * Hkv + grp) * (size_t)l32_of(L) * DH;
  const bf16* Vb = Vc + ((size_t)b * Hkv + grp) * (size_t)l32_of(L) * DH;
  const int ntiles = L >> 5;

  // this wave's RPW requests of tile kt into ring slot `slot`: request r < KS
  // copies key fragment r (1 KB, lane l at 16 l); the others copy value rows,
  // chunk c of row r into slot c ^ vswz(r)
  auto vswz = [](int r) { return DH == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
  const unsigned voff = (unsigned)((lane / CPR) * RB + 16 * ((lane % CPR) ^ vswz(lane / CPR)));
  auto request = [&](int kt, int slot) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is only ever set here
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = wv * RPW + j;  // wave-uniform
      const unsigned l = (unsigned)(uintptr_t)((lds_u8*)smem + slot * SLOT + r * 1024);
      const void* src;
      unsigned vo;
      if (r < KS) {
        src = uniform_ptr(Kb + ((size_t)kt * KS + r) * 512);
        vo = (unsigned)lane * 16u;
      } else {
        src = uniform_ptr(Vb + (size_t)kt * 32 * DH + (size_t)(r - KS) * 512);
        vo = voff;
      }
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(__builtin_amdgcn_readfirstlane(l)),
                   "v"(vo), "s"(src)
                   : "memory", "m0");
    }
#pragma clang diagnostic pop
  };
  // transposed value reads (see attn_mfma_kernel): lane byte offsets in a
  // value tile for kk = 0 and keys +0..3
  const int jq = lane & 15, Gq = lane >> 4;
  const int mf = DH == 128 ? (jq >> 2) : (jq >> 3);
  int vrd[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    vrd[dt] = (4 * (Gq >> 1) + (jq >> 2)) * RB + (4 * (dt ^ mf) + 2 * (Gq & 1) + ((jq & 3) >> 1)) * 16 + 8 * (jq & 1);

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // the query fragments have landed before any request goes out, so the only
  // memory operations in flight in the key loop are this wave's requests
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
#pragma unroll
  for (int t = 0; t < P; ++t) request(min(t, ntiles - 1), t);
  for (int kt = 0; kt < ntiles; ++kt) {
    if (kt % GQ_TPB == 0) {
      // this wave's requests of tiles kt .. kt + GQ_TPB - 1 have landed
      // (those of the P - GQ_TPB newer tiles may not have); after the barrier
      // every wave's have, and every wave is done with the GQ_TPB previous
      // tiles, whose slots the next requests refill (past the last tile the
      // requests repeat it, into slots nobody reads again)
      constexpr int WAITN = (P - GQ_TPB) * RPW;
      __builtin_amdgcn_s_waitcnt((WAITN & 15) | ((WAITN >> 4) << 14) | (7 << 4) | (15 << 8));
      __syncthreads();
#pragma unroll
      for (int t = 0; t < GQ_TPB; ++t) request(min(kt + P + t, ntiles - 1), (kt + P + t) % GQ_NB);
    }
    if (!comp) continue;
    const lds_u8* sb = (lds_u8*)smem + (kt % GQ_NB) * SLOT;
    u32x4 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(sb + ks * 1024 + lane * 16);
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
    const float m_new = mt > m_run + ATT_M_SLACK ? mt : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 1 where m_run stays
    u32x4 pf[2];
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * e], sl2e, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * kk + 2 * e + 1], sl2e, -m_new));
        rs += p0;
        rs += p1;
        pf[kk][e] = pack2bf(p0, p1);
      }
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (kt > 0 && __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
        const lds_u8* a = sb + KTB + kk * 16 * RB + vrd[dt];
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)a);
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a + 8 * RB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        vf[dt] = u32x4{l2.x, l2.y, h2.x, h2.y};
      }
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pf[kk]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[dt]), pb, o[dt], 0, 0, 0);
    }
  }
  // no request may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
  if (!comp) return;
  // O / l, this wave's head only: lanes pair up (shuffle across the halves)
  // into 8 consecutive dimensions, as in attn_mfma_kernel's merge
  const float inv = 1.0f / l_run;
  const int m = r0 + ln;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
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

hipError_t launch_attention(hipStream_t st, bool bf16m, int max_rows, int B, int L, int Hq, int Hkv, int dh,
                            const int32_t* idx, const int32_t* n, const void* q, const void* Kc, const void* Vc,
                            void* out, int MTt) {
  if (max_rows <= 0) return hipSuccess;
  const float scale = 1.0f / sqrtf((float)dh);
  if (bf16m && (dh == 128 || dh == 64) && L % 32 == 0) {
    const float sl2e = scale * 1.4426950408889634f;
    const int ntq = (max_rows + 31) / 32 + B;  // query tiles per head, an upper bound
    if (Hq % Hkv == 0 && Hq / Hkv >= 4 && Hq / Hkv <= ATT_NW) {
      // grouped-query heads: one workgroup per (query tile, KV head)
      const int grid = (ntq * Hkv + 7) / 8 * 8;
      if (dh == 128)
        hipLaunchKernelGGL(attn_gqa_kernel<128>, dim3(grid), dim3(ATT_NW * 64), 0, st, B, L, Hq, Hkv, ntq, sl2e,
                           max_rows, n, (const bf16*)q, (const bf16*)Kc, (const bf16*)Vc, (bf16*)out, MTt);
      else
        hipLaunchKernelGGL(attn_gqa_kernel<64>, dim3(grid), dim3(ATT_NW * 64), 0, st, B, L, Hq, Hkv, ntq, sl2e,
                           max_rows, n, (const bf16*)q, (const bf16*)Kc, (const bf16*)Vc, (bf16*)out, MTt);
      return hipGetLastError();
    }
    const int grid = (ntq * Hq + 7) / 8 * 8;
    // more (query tile, head) pairs than CUs and at most 1024 keys: 4 waves
    // per workgroup (64 KB of LDS, two workgroups per CU, each wave twice the
    // keys) instead of a second round of 8-wave ones.  Measured: C3's largest
    // layers (L = 1024, 288 pairs) 0.529 -> 0.506 ms of attention per step;
    // at L = 4096 (384 pairs) the doubled key chain per wave costs more than
    // the second round (1.93 -> 2.69 ms), so longer caches keep 8 waves.
    const bool half = ntq * Hq > ATT_ONE_ROUND && L <= ATT_HALF_MAX_KEYS;
#define AM(D, W)                                                                                              \
  hipLaunchKernelGGL((attn_mfma_kernel<D, W>), dim3(grid), dim3(W * 64), 0, st, B, L, Hq, Hkv, ntq, sl2e, max_rows, \
                     n, (const bf16*)q, (const bf16*)Kc, (const bf16*)Vc, (bf16*)out, MTt)
    if (dh == 128) {
      if (half) AM(128, 4); else AM(128, 8);
    } else {
      if (half) AM(64, 4); else AM(64, 8);
    }
#undef AM
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
