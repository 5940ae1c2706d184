"""Numerical core of the oracle (one sequence at a time).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Precision: activations are fp32 (``Spec.gemm64`` switches every array to fp64
for comparisons against the pure-Python brute force); norms, RoPE angles,
softmax, attention, the value proxy, drift, LM-head logits and their
statistics are fp64.  ``Spec.bf16`` additionally rounds (RNE) every GEMM input
and every stored K/V/hidden row to the bfloat16 grid, mirroring how a bf16
model stores its activations.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Spec", "round_bf16", "rmsnorm", "rope", "attention", "layer_dense",
    "sparse_layer", "proxy", "drift", "budget_k", "select", "lm_stats",
    "commit", "proxy_basis",
]


@dataclasses.dataclass(frozen=True)
class Spec:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    seq_len: int
    block_len: int
    proxy_rank: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    bf16: bool = False
    gemm64: bool = False

    @property
    def wd(self):
        return np.float64 if self.gemm64 else np.float32


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _act(x, spec: Spec):
    """A GEMM input or a stored row, in the model's activation precision."""
    if spec.gemm64:
        return np.asarray(x, dtype=np.float64)
    return round_bf16(x) if spec.bf16 else np.asarray(x, dtype=np.float32)


def _mm(a, w, spec: Spec):
    if spec.gemm64:
        return np.asarray(a, np.float64) @ np.asarray(w, np.float64)
    return np.asarray(a, np.float32) @ np.asarray(w, np.float32)


# --------------------------------------------------------------------------
# transformer pieces (the pages name a bidirectional transformer; the block
# layout is the reading: pre-RMSNorm, RoPE, no biases, SwiGLU FFN)
# --------------------------------------------------------------------------

def rmsnorm(x, g, eps: float, wd=np.float32):
    """x / sqrt(mean(x^2) + eps) * g over the last axis, computed in fp64."""
    x64 = np.asarray(x, np.float64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    return (x64 / np.sqrt(ms + eps) * np.asarray(g, np.float64)).astype(wd)


def rope(x, pos, theta: float, wd=np.float32):
    """Rotate-half rotary embedding of x [n, H, dh] at integer positions pos [n].

    Reading: the pages never name a position encoding, but without one a
    bidirectional layer is permutation-equivariant and every [MASK] row would be
    identical, so RoPE with theta = 10^4 is assumed.  Pair (j, j + dh/2) is
    rotated by angle pos * theta^(-2j/dh).
    """
    x = np.asarray(x, np.float64)
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / dh)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(wd)


def attention(q, K, V, wd=np.float32):
    """Bidirectional (unmasked) attention of queries q [n, Hq, dh] over every
    cached row K, V [L, Hkv, dh].

    Bidirectional attention over the whole sequence is what makes dLLM caching
    hard (SPA-Cache, problem statement; EntropyCache section 1).  Query head h
    reads KV head floor(h * Hkv / Hq) (grouped-query attention for the Dream
    shape).  Softmax and both products in fp64 with an explicit [n, L] matrix.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n, hq, dh = q.shape
    hkv = K.shape[1]
    out = np.empty((n, hq, dh), np.float64)
    for h in range(hq):
        g = (h * hkv) // hq
        s = q[:, h, :] @ K[:, g, :].T / math.sqrt(dh)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, g, :]
    return out.astype(wd)


def _silu(x):
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def _qkv(a, W, pos, spec: Spec):
    n = a.shape[0]
    H, G, dh = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    q = _mm(a, W["w_q"], spec).reshape(n, H, dh)
    k = _mm(a, W["w_k"], spec).reshape(n, G, dh)
    v = _mm(a, W["w_v"], spec).reshape(n, G, dh)
    q = _act(rope(q, pos, spec.rope_theta, spec.wd), spec)
    k = _act(rope(k, pos, spec.rope_theta, spec.wd), spec)
    v = _act(v, spec)
    return q, k, v


def _attn_out_ffn(x_rows, q, K, V, W, spec: Spec):
    n = x_rows.shape[0]
    o = _act(attention(q, K, V, spec.wd).reshape(n, -1), spec)
    h1 = (np.asarray(x_rows, spec.wd) + _mm(o, W["w_o"], spec)).astype(spec.wd)
    nrm = _act(rmsnorm(h1, W["ffn_norm"], spec.rms_eps, spec.wd), spec)
    g = _mm(nrm, W["w_gate"], spec)
    u = _mm(nrm, W["w_up"], spec)
    act = _act((_silu(g) * np.asarray(u, np.float64)).astype(spec.wd), spec)
    out = (h1 + _mm(act, W["w_down"], spec)).astype(spec.wd)
    return _act(out, spec)


def layer_dense(x, W, spec: Spec, pos=None):
    """Full recompute of one layer over all L rows (the baseline every step of
    a cache-free dLLM pays: EntropyCache section 1, TSPD/CE problem statement).

    Row i sits at position pos[i] (default: i).
    Returns (out [L, d], K [L, Hkv, dh], V [L, Hkv, dh]).
    """
    x = np.asarray(x, spec.wd)
    L = x.shape[0]
    pos = np.arange(L) if pos is None else np.asarray(pos)
    a = _act(rmsnorm(x, W["attn_norm"], spec.rms_eps, spec.wd), spec)
    q, k, v = _qkv(a, W, pos, spec)
    return _attn_out_ffn(x, q, k, v, W, spec), k, v


def sparse_layer(x, K, V, H_out, idx, W, spec: Spec):
    """Sparse execution on index set I (SPA-Cache, method step 3).

    The selected rows of the layer input produce sparse queries, keys and
    values; the new keys/values are written into the cache first, then the
    sparse queries attend over the whole, partially updated cache; the FFN runs
    on the sparse rows only and the layer output is updated only at I, every
    other row keeping its cached output.  K, V and H_out ([L, ...]) are updated
    in place.  idx must be sorted and unique.
    """
    idx = np.asarray(idx, np.int64)
    if idx.size == 0:
        return
    x = np.asarray(x, spec.wd)
    xr = x[idx]
    a = _act(rmsnorm(xr, W["attn_norm"], spec.rms_eps, spec.wd), spec)
    q, k, v = _qkv(a, W, idx, spec)
    K[idx] = k
    V[idx] = v
    H_out[idx] = _attn_out_ffn(xr, q, K, V, W, spec)


# --------------------------------------------------------------------------
# SPA-Cache: singular value proxy and drift (method step 1)
# --------------------------------------------------------------------------

def proxy_basis(w_v, r: int):
    """Truncated SVD factor of the value projection (SPA-Cache, step 1).

    W_V = U S V^T (fp64); the top-r singular vectors and values are kept as
    W_r = U_r S_r, so that x W_r are the coordinates of the rank-r value
    approximation x U_r S_r V_r^T in the orthonormal basis V_r (the cosine of two
    proxies equals the cosine of their rank-r value states).
    """
    u, s, _ = np.linalg.svd(np.asarray(w_v, np.float64), full_matrices=False)
    return u[:, :r] * s[None, :r], s


def proxy(x, g1, w_r):
    """Singular proxy of layer inputs x [n, d]: (x * g1) W_r in fp64.

    SPA-Cache step 1 projects the input state onto the rank-r manifold.  Reading:
    the input state is the attention-norm input, whose 1/rms row scale is
    dropped because the cosine is invariant to it; the gain g1 is kept.
    """
    return (np.asarray(x, np.float64) * np.asarray(g1, np.float64)[None, :]) @ np.asarray(w_r, np.float64)


def drift(C, P):
    """Drift of current proxies C [n, r] against cached proxies P [n, r].

    SPA-Cache step 1 ranks tokens by the cosine similarity of the current and
    cached proxy, lowest first.  The score is s = 1 - cos computed as
    0.5 * ||C/|C| - P/|P| ||^2 (no cancellation; identical rows give exactly 0).
    Both zero: 0; exactly one zero: 1 (cos taken as 0).
    """
    C = np.asarray(C, np.float64)
    P = np.asarray(P, np.float64)
    nc = np.sqrt(np.sum(C * C, axis=-1))
    npp = np.sqrt(np.sum(P * P, axis=-1))
    out = np.empty(C.shape[0], np.float64)
    for i in range(C.shape[0]):
        if nc[i] == 0.0 and npp[i] == 0.0:
            out[i] = 0.0
        elif nc[i] == 0.0 or npp[i] == 0.0:
            out[i] = 1.0
        else:
            dlt = C[i] / nc[i] - P[i] / npp[i]
            out[i] = 0.5 * np.sum(dlt * dlt)
    return out


def budget_k(rho: float, L: int) -> int:
    """Rows refreshed at a layer with update ratio rho (SPA-Cache step 2):
    k = floor(rho * L + 1/2), in fp64."""
    return int(math.floor(float(rho) * L + 0.5))


def select(s, forced, k: int):
    """Index set I of one layer (SPA-Cache steps 1-2, EntropyCache step 3).

    Forced rows F (EntropyCache: current mask block plus the k most recently
    decoded tokens) are always in I; the remaining max(k, |F|) - |F| rows are
    the non-forced ones with the largest drift, ties broken by lower index.
    Returned in ascending order.
    """
    s = np.asarray(s, np.float64)
    L = s.shape[0]
    forced = np.zeros(L, bool) if forced is None else np.asarray(forced, bool)
    F = [i for i in range(L) if forced[i]]
    keff = min(max(k, len(F)), L)
    rest = sorted((i for i in range(L) if not forced[i]), key=lambda i: (-s[i], i))
    return np.array(sorted(F + rest[: keff - len(F)]), np.int64)


# --------------------------------------------------------------------------
# LM head statistics and commit (EntropyCache section 2; static threshold)
# --------------------------------------------------------------------------

def lm_stats(h, g_f, w_lm, spec: Spec):
    """Per-row logits statistics of hidden rows h [n, d].

    z = (RMSNorm(h) * g_f) W_lm, the normed rows in the activation precision
    (bf16 for bf16 models) and the product in fp64.  Returns a dict of fp64
    arrays: m = max z, argmax (lowest id on ties), S = sum exp(z - m),
    T = sum exp(z - m)(z - m), conf = 1/S (top-1 softmax probability) and
    entropy = ln S - T/S (nats), the quantity EntropyCache thresholds.
    """
    nrm = _act(rmsnorm(h, g_f, spec.rms_eps, spec.wd), spec)
    z = np.asarray(nrm, np.float64) @ np.asarray(w_lm, np.float64)
    m = z.max(axis=1)
    am = np.argmax(z, axis=1)  # numpy returns the first maximal index
    e = np.exp(z - m[:, None])
    S = e.sum(axis=1)
    T = (e * (z - m[:, None])).sum(axis=1)
    return {"m": m, "argmax": am.astype(np.int64), "S": S, "T": T,
            "conf": 1.0 / S, "entropy": np.log(S) - T / S, "logits": z}


def commit(rows, conf, argmax, entropy, committed, threshold: float):
    """Static-threshold parallel commit over the current block.

    Parallel decoding commits every still-masked token whose confidence clears
    a fixed threshold (Polestar section 1; TSPD/CE problem statement).  Reading:
    if none clears it, the single most confident masked row is committed
    (lowest position on ties) so that every step makes progress.

    rows: block positions [n]; conf/argmax/entropy: their statistics [n];
    committed: bool [L] (not modified).  Returns (positions committed in
    ascending order, their token ids, max entropy over them or 0.0 if none).
    """
    cand = [j for j in range(len(rows)) if not committed[rows[j]]]
    pick = [j for j in cand if conf[j] >= threshold]
    if not pick and cand:
        best = cand[0]
        for j in cand[1:]:
            if conf[j] > conf[best] or (conf[j] == conf[best] and rows[j] < rows[best]):
                best = j
        pick = [best]
    pick.sort(key=lambda j: rows[j])
    pos = [int(rows[j]) for j in pick]
    tok = [int(argmax[j]) for j in pick]
    emax = max((float(entropy[j]) for j in pick), default=0.0)
    return pos, tok, emax
