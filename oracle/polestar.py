"""Polestar-Cache drift path (Polestar page, section 2A "Polestar-Cache").

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the page states:
- A token's drift is the KL divergence between its attention distributions at
  two consecutive steps.
- A local window (prefix and suffix blocks around the current block) is kept.
- The window's hidden states are clustered with spherical k-means, and the
  residuals are quantised with NVFP4 into a compressed proxy.
- Every step, attention computed from the cluster centroids ("proxy
  attention") ranks the clusters by drift.
- The top-k drifting clusters get a sparse forward pass.

The page gives no sizes, seeds, precisions or formulas beyond the KL, so the
readings taken here are:

- **Window.** Three blocks: prefix, current and suffix. It starts at
  ``clamp(block_start - blk, 0, L - 3 blk)``.
- **Hidden state.** The layer input H_l of each window row, scaled to unit
  length in fp64. Spherical k-means clusters directions.
- **k-means.**
  - ``n_clusters`` seeds sit at window rows ``stride * j``, with
    ``stride = W // n_clusters``.
  - There are ``iters`` iterations. Each assigns every row to the centroid of
    largest dot product (lowest cluster index on ties). Each then replaces
    every centroid that has members by the normalised sum of those members.
    An empty cluster, or one whose member sum is the zero vector, keeps its
    centroid.
  - A final assignment against the final centroids gives the membership.
- **NVFP4 of the residual** ``x_hat - c_a``: one E4M3 scale per 16
  consecutive elements, ``s = E4M3_RNE(amax / 6)``, and E2M1 codes
  ``E2M1_RNE(r / s)`` saturated at 6. A zero scale gives zero codes.
  - These codes are the compressed proxy that the page keeps in host memory.
    Nothing on a single GPU consumes them.
- **Centroid queries.** ``q_c = bf16(RMSNorm(c) * g1) @ W_q``, rotated (RoPE)
  at the position of the cluster's seed row.
- **Proxy attention.** For each query head: a softmax in fp64, scale
  1/sqrt(dh), over the current keys of the window rows in that head's KV group.
- **Cluster drift.** The mean over query heads of KL(A_t || A_{t-1}), where
  A_{t-1} is the same cluster's proxy attention at the same layer in the
  previous step. It is 0 when no previous step exists for this window (the
  first step, or the window moved).
- **Selection.** The ``top`` clusters of largest drift (lowest index on ties).
  I = the current block's rows plus the members of those clusters, in
  ascending order.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from .model import Spec, _act, _mm, rmsnorm, rope


@dataclasses.dataclass(frozen=True)
class PolestarParams:
    n_clusters: int = 16
    iters: int = 10
    top: int = 4
    window_blocks: int = 3
    tau_upd: int = 0        # drift refresh once this many tokens were decoded since the last (0: every step)
    full_period: int = 0    # a full pass every this many steps (0: never)


def window_start(block_start: int, L: int, blk: int, wblocks: int = 3) -> int:
    """First row of the window: one block before the current block, clamped so
    that the whole window lies inside the sequence."""
    W = wblocks * blk
    return int(min(max(block_start - blk, 0), L - W))


def unit_rows(x) -> np.ndarray:
    """Rows scaled to unit Euclidean length in fp64 (zero rows stay zero)."""
    x = np.asarray(x, np.float64)
    n = np.sqrt(np.sum(x * x, axis=1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def _assign(X, C):
    D = X @ C.T  # [n, k] dot products
    return np.argmax(D, axis=1), D  # argmax returns the lowest index on ties


def spherical_kmeans(X, n_clusters: int, iters: int):
    """Spherical k-means of unit rows X [n, d] (fp64), following the readings
    above.  Returns (centroids [k, d], assignment [n], objective per
    iteration, dot products of the final assignment [n, k])."""
    X = np.asarray(X, np.float64)
    n = X.shape[0]
    stride = n // n_clusters
    C = X[stride * np.arange(n_clusters)].copy()
    obj = []
    for _ in range(iters):
        a, D = _assign(X, C)
        obj.append(float(np.sum(D[np.arange(n), a])))
        for j in range(n_clusters):
            m = a == j
            if not m.any():
                continue
            v = X[m].sum(axis=0)
            nv = math.sqrt(float(v @ v))
            if nv > 0:
                C[j] = v / nv
    a, D = _assign(X, C)
    obj.append(float(np.sum(D[np.arange(n), a])))
    return C, a, obj, D


# --------------------------------------------------------------------------
# NVFP4: E2M1 elements with one E4M3 (OCP FN) scale per 16 elements
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3FN byte: 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent 0 is subnormal; S.1111.111 is NaN; there is no infinity."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m1_value(code: int) -> float:
    """Value of an E2M1 nibble: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * 0.5 * m
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


_E4M3_POS = [e4m3_value(c) for c in range(0x7F)]  # codes 0x00..0x7E, increasing
_E2M1_POS = [e2m1_value(c) for c in range(8)]


def _rne_on_grid(v: float, grid) -> int:
    """Index of the grid value nearest to v >= 0 (grid increasing from 0),
    ties to the even index, saturating at the top."""
    if not v > 0.0:
        return 0
    if v >= grid[-1]:
        return len(grid) - 1
    hi = 1
    while grid[hi] < v:
        hi += 1
    lo = hi - 1
    dl, dh = v - grid[lo], grid[hi] - v
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if lo % 2 == 0 else hi


def e4m3_rne(v: float) -> int:
    """Non-negative value -> E4M3FN code, round to nearest even, saturating at 448."""
    return _rne_on_grid(v, _E4M3_POS)


def e2m1_rne(v: float) -> int:
    """Value -> E2M1 code (sign = 1 iff v < 0), magnitude rounded to nearest
    even and saturated at 6."""
    c = _rne_on_grid(abs(v), _E2M1_POS)
    return c | (0x8 if v < 0 else 0)


def nvfp4_encode(R):
    """Residual rows R [n, d] (d % 16 == 0, fp64) -> (codes uint8 [n, d/2]:
    element 2i in the low nibble of byte i; scales uint8 [n, d/16])."""
    R = np.asarray(R, np.float64)
    n, d = R.shape
    codes = np.zeros((n, d // 2), np.uint8)
    scales = np.zeros((n, d // 16), np.uint8)
    for i in range(n):
        nib = np.zeros(d, np.uint8)
        for g in range(d // 16):
            blk = R[i, 16 * g:16 * g + 16]
            sc = e4m3_rne(float(np.max(np.abs(blk))) / 6.0)
            scales[i, g] = sc
            s = _E4M3_POS[sc]
            if s == 0.0:
                continue
            for e in range(16):
                nib[16 * g + e] = e2m1_rne(float(blk[e]) / s)
        codes[i] = nib[0::2] | (nib[1::2] << 4)
    return codes, scales


# --------------------------------------------------------------------------
# centroid queries, proxy attention, cluster drift, selection
# --------------------------------------------------------------------------

def centroid_queries(C, pos, W, spec: Spec):
    """q_c = bf16(RMSNorm(c) * g1) @ W_q, RoPE at pos [k] -> [k, Hq, dh] in the
    activation precision (the model's query path applied to the centroids)."""
    a = _act(rmsnorm(C, W["attn_norm"], spec.rms_eps, spec.wd), spec)
    q = _mm(a, W["w_q"], spec).reshape(C.shape[0], spec.n_q_heads, spec.head_dim)
    return _act(rope(q, pos, spec.rope_theta, spec.wd), spec)


def proxy_log_attention(q, Kw):
    """log A [k, Hq, W]: per centroid query and query head, the log-softmax
    (fp64) of q . k / sqrt(dh) over the window keys Kw [W, Hkv, dh] of the
    head's KV group."""
    q = np.asarray(q, np.float64)
    Kw = np.asarray(Kw, np.float64)
    k, hq, dh = q.shape
    hkv = Kw.shape[1]
    out = np.empty((k, hq, Kw.shape[0]), np.float64)
    for h in range(hq):
        g = (h * hkv) // hq
        s = q[:, h, :] @ Kw[:, g, :].T / math.sqrt(dh)
        m = s.max(axis=1, keepdims=True)
        out[:, h, :] = (s - m) - np.log(np.sum(np.exp(s - m), axis=1, keepdims=True))
    return out


def cluster_kl(logA, logA_prev):
    """Drift of each cluster: mean over query heads of KL(A_t || A_{t-1}) =
    sum_w A_t (log A_t - log A_{t-1})."""
    logA = np.asarray(logA, np.float64)
    kl = np.sum(np.exp(logA) * (logA - np.asarray(logA_prev, np.float64)), axis=2)
    return np.mean(kl, axis=1)


def top_clusters(kl, top: int):
    """The ``top`` clusters of largest drift, lowest index on ties."""
    kl = np.asarray(kl, np.float64)
    order = sorted(range(kl.size), key=lambda j: (-kl[j], j))
    return np.array(sorted(order[:top]), np.int64)


def select_rows(block_rows, wstart: int, assign, clusters):
    """I = current block rows + window rows assigned to the chosen clusters."""
    members = wstart + np.nonzero(np.isin(assign, clusters))[0]
    return np.union1d(np.asarray(block_rows, np.int64), members).astype(np.int64)


@dataclasses.dataclass
class PolestarLayerState:
    """Per layer and sequence: the proxy log-attention of the last drift
    refresh, the window it belongs to, and the number of decoded tokens at
    that refresh."""
    logA: Optional[np.ndarray] = None
    wstart: int = -1
    hist_at_update: int = 0


def refresh_due(prev: PolestarLayerState, ws: int, n_decoded: int, pp: PolestarParams) -> bool:
    """Schedule of the drift refresh (Polestar section 2A, schedule).  The page
    triggers updates once the decoded context has moved enough, e.g. after
    tau_upd decoded tokens.  Reading: a layer's refresh runs when tau_upd <= 0
    (every step), on a window's first step (no stored attention, or the window
    moved), or once at least tau_upd tokens were decoded since its last
    refresh.  Full passes do not reset the count."""
    if pp.tau_upd <= 0 or prev.logA is None or prev.wstart != ws:
        return True
    return n_decoded - prev.hist_at_update >= pp.tau_upd


def drift_and_select(x, K, block_start: int, W, spec: Spec, pp: PolestarParams, prev: PolestarLayerState,
                     n_decoded: int = 0):
    """The whole drift path of one layer and one sequence: window, k-means,
    NVFP4 codes, centroid queries, proxy attention, cluster drift, top
    clusters and the index set I.  Updates ``prev``; returns a dict of every
    intermediate.  ``n_decoded``: tokens decoded before this step (for the
    refresh schedule).  Without a due refresh (``refresh_due``) the step
    refreshes only the current block, keeps ``prev`` and has no drift."""
    L, blk = spec.seq_len, spec.block_len
    Wn = pp.window_blocks * blk
    ws = window_start(block_start, L, blk, pp.window_blocks)
    Xh = unit_rows(np.asarray(x, np.float64)[ws:ws + Wn])
    C, a, obj, D = spherical_kmeans(Xh, pp.n_clusters, pp.iters)
    codes, scales = nvfp4_encode(Xh - C[a])
    stride = Wn // pp.n_clusters
    pos = ws + stride * np.arange(pp.n_clusters)
    q = centroid_queries(C, pos, W, spec)
    logA = proxy_log_attention(q, np.asarray(K)[ws:ws + Wn])
    rows = np.arange(block_start, min(block_start + blk, L))
    update = refresh_due(prev, ws, n_decoded, pp)
    valid = update and prev.logA is not None and prev.wstart == ws
    if valid:
        kl = cluster_kl(logA, prev.logA)
    else:
        kl = np.zeros(pp.n_clusters)
    top = top_clusters(kl, pp.top)
    if update:
        prev.logA, prev.wstart, prev.hist_at_update = logA, ws, n_decoded
        I = select_rows(rows, ws, a, top)
    else:
        I = rows.astype(np.int64)
    return {"wstart": ws, "Xh": Xh, "C": C, "assign": a, "obj": obj, "dots": D, "codes": codes,
            "scales": scales, "q": q, "logA": logA, "kl": kl, "valid": valid, "update": update, "top": top,
            "I": I}


# ---------------------------------------------------------------------------
# Polestar-Commit (Polestar page, section 2B).
#
# What the page states:
# - For the current block it tracks each token's drift delta: the token's
#   drift minus the historical mean of its drift.  A sharp positive delta
#   signals fast context integration.
# - A token commits when its delta exceeds a confidence-dependent threshold
#   alpha (tau_s - c)^2, so a low-confidence token with a strong convergence
#   signal can still commit.
# - The last layer's update packet is also inspected: when a centroid of the
#   suffix window is among the top drift clusters, suffix tokens commit, but
#   only at the high confidence threshold (>= tau_s).
#
# Readings (the page gives no values or definitions beyond these):
# - tau_s is the static confidence threshold of the threshold commit, and a
#   token that clears it commits as before; the drift rule adds commits.
# - A token's drift D_j is the cluster drift (mean over heads of the proxy
#   attention KL) of its cluster at the last layer.  It is defined only when
#   that layer's drift is (the window did not move since the previous step).
# - The historical mean is the mean of D_j over the earlier steps of the
#   current block at which it was defined; with no earlier value there is no
#   delta and no drift commit.  The history restarts when the block advances.
# - "A suffix centroid among the top clusters": a top cluster of the last
#   layer has a member among the window rows after the current block.  The
#   suffix tokens considered are the masked rows of the next block.
# - If nothing commits in the current block, the most confident masked row of
#   the block commits (lowest position on ties), as in the threshold commit.
# - Commits are appended to the decode history in ascending position order
#   (current block, then suffix); the entropy gate takes the maximum entropy
#   over all of them.
# ---------------------------------------------------------------------------
def token_drift(rows, wstart: int, assign, kl):
    """D_j of window rows ``rows``: the drift of the cluster each belongs to."""
    a = np.asarray(assign)
    return np.array([float(kl[a[int(r) - wstart]]) for r in rows], np.float64)


def suffix_hit(block_start: int, blk: int, wstart: int, assign, top) -> bool:
    """Whether a top cluster has a member among the window rows after the
    current block."""
    a = np.asarray(assign)
    first = block_start + blk - wstart  # first window index after the block
    return any(int(a[r]) in set(int(t) for t in top) for r in range(max(first, 0), a.size))


def drift_commit(cur_rows, cur, suf_rows, suf, committed, tau_s: float, alpha: float, D, hist_sum, hist_cnt,
                 hit: bool):
    """One Polestar-Commit decision.

    cur_rows / suf_rows: positions of the current and the next block; cur /
    suf: their LM statistics (dicts with conf, argmax, entropy); committed:
    bool [L] (not modified); D: drift of the current block rows, or None when
    undefined this step; hist_sum / hist_cnt: sum and count of their earlier
    drifts (read only here).  Returns (positions in ascending order, tokens,
    max entropy, pick flags of the current rows)."""
    n = len(cur_rows)
    cand = [j for j in range(n) if not committed[cur_rows[j]]]
    pick = []
    for j in cand:
        c = float(cur["conf"][j])
        if c >= tau_s:
            pick.append(j)
        elif D is not None and hist_cnt[j] > 0:
            delta = float(D[j]) - float(hist_sum[j]) / float(hist_cnt[j])
            t = tau_s - c
            if delta > alpha * (t * t):
                pick.append(j)
    if not pick and cand:
        best = cand[0]
        for j in cand[1:]:
            if cur["conf"][j] > cur["conf"][best]:
                best = j
        pick = [best]
    pick.sort()
    spick = []
    if hit:
        spick = [j for j in range(len(suf_rows))
                 if not committed[suf_rows[j]] and float(suf["conf"][j]) >= tau_s]
    pos = [int(cur_rows[j]) for j in pick] + [int(suf_rows[j]) for j in spick]
    tok = [int(cur["argmax"][j]) for j in pick] + [int(suf["argmax"][j]) for j in spick]
    ents = [float(cur["entropy"][j]) for j in pick] + [float(suf["entropy"][j]) for j in spick]
    flags = np.zeros(n, bool)
    flags[pick] = True
    return pos, tok, max(ents, default=0.0), flags
