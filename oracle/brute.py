"""Pure-Python brute force for tiny shapes (lists of floats, math.fsum).

TEST INFRASTRUCTURE ONLY.  An independent third formulation of every oracle
function, written with explicit loops so that the NumPy oracle can be checked
against it to ~1e-12 (d = 8, 2 heads of 4, L = 6, V = 11 and the like).
"""

from __future__ import annotations

import math


def matvec(x, W):
    """y_j = sum_k x_k W[k][j]."""
    return [math.fsum(x[k] * W[k][j] for k in range(len(x))) for j in range(len(W[0]))]


def rmsnorm(x, g, eps):
    ms = math.fsum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[i] * r * g[i] for i in range(len(x))]


def rope_head(v, pos, theta):
    dh = len(v)
    half = dh // 2
    out = [0.0] * dh
    for j in range(half):
        a = pos * theta ** (-(2.0 * j) / dh)
        out[j] = v[j] * math.cos(a) - v[j + half] * math.sin(a)
        out[j + half] = v[j + half] * math.cos(a) + v[j] * math.sin(a)
    return out


def softmax(xs):
    m = max(xs)
    e = [math.exp(v - m) for v in xs]
    s = math.fsum(e)
    return [v / s for v in e]


def layer_rows(x_all, Kc, Vc, rows, W, spec):
    """Recompute layer outputs for ``rows`` (sorted) given the full input
    x_all [L][d] and caches Kc, Vc [L][Hkv][dh] (updated in place).
    Returns {row: output list}."""
    H, G, dh = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
    eps, th = spec.rms_eps, spec.rope_theta
    L = len(x_all)
    qs = {}
    for i in rows:
        a = rmsnorm(x_all[i], W["attn_norm"], eps)
        q = matvec(a, W["w_q"])
        k = matvec(a, W["w_k"])
        v = matvec(a, W["w_v"])
        qs[i] = [rope_head(q[h * dh:(h + 1) * dh], i, th) for h in range(H)]
        Kc[i] = [rope_head(k[g * dh:(g + 1) * dh], i, th) for g in range(G)]
        Vc[i] = [v[g * dh:(g + 1) * dh] for g in range(G)]
    out = {}
    for i in rows:
        o = []
        for h in range(H):
            g = (h * G) // H
            sc = [math.fsum(qs[i][h][t] * Kc[j][g][t] for t in range(dh)) / math.sqrt(dh)
                  for j in range(L)]
            p = softmax(sc)
            o.extend(math.fsum(p[j] * Vc[j][g][t] for j in range(L)) for t in range(dh))
        ao = matvec(o, W["w_o"])
        h1 = [x_all[i][c] + ao[c] for c in range(len(ao))]
        n = rmsnorm(h1, W["ffn_norm"], eps)
        gt = matvec(n, W["w_gate"])
        up = matvec(n, W["w_up"])
        act = [gt[f] / (1.0 + math.exp(-gt[f])) * up[f] for f in range(len(gt))]
        dn = matvec(act, W["w_down"])
        out[i] = [h1[c] + dn[c] for c in range(len(h1))]
    return out


def proxy(x, g1, Wr):
    return matvec([x[i] * g1[i] for i in range(len(x))], Wr)


def drift(c, p):
    """1 - cos(c, p) with the zero-vector conventions (both 0 -> 0, one -> 1)."""
    nc = math.sqrt(math.fsum(v * v for v in c))
    npp = math.sqrt(math.fsum(v * v for v in p))
    if nc == 0.0 and npp == 0.0:
        return 0.0
    if nc == 0.0 or npp == 0.0:
        return 1.0
    return 1.0 - math.fsum(c[i] * p[i] for i in range(len(c))) / (nc * npp)


def select(s, forced, k):
    L = len(s)
    F = [i for i in range(L) if forced[i]]
    need = max(min(max(k, len(F)), L) - len(F), 0)
    order = sorted(range(L), key=lambda i: (-s[i], i))
    picked = [i for i in order if not forced[i]][:need]
    return sorted(F + picked)


def lm_stats(h, gf, Wlm, eps):
    n = rmsnorm(h, gf, eps)
    z = matvec(n, Wlm)
    m = max(z)
    am = z.index(m)
    e = [math.exp(v - m) for v in z]
    S = math.fsum(e)
    p = [v / S for v in e]
    ent = -math.fsum(pi * math.log(pi) for pi in p if pi > 0.0)
    return {"m": m, "argmax": am, "S": S, "conf": max(p), "entropy": ent}


def commit(rows, conf, argmax, entropy, committed, threshold):
    cand = [j for j in range(len(rows)) if not committed[rows[j]]]
    pick = [j for j in cand if conf[j] >= threshold]
    if not pick and cand:
        pick = [sorted(cand, key=lambda j: (-conf[j], rows[j]))[0]]
    pick = sorted(pick, key=lambda j: rows[j])
    return ([rows[j] for j in pick], [argmax[j] for j in pick],
            max([entropy[j] for j in pick], default=0.0))


# --------------------------------------------------------------------------
# Polestar drift path (pure Python)
# --------------------------------------------------------------------------

def unit(v):
    n = math.sqrt(math.fsum(a * a for a in v))
    return [a / n for a in v] if n > 0 else [0.0] * len(v)


def dot(a, b):
    return math.fsum(x * y for x, y in zip(a, b))


def kmeans(X, k, iters):
    """Spherical k-means on unit rows (lists), seeds at rows stride*j."""
    n = len(X)
    stride = n // k
    C = [list(X[stride * j]) for j in range(k)]

    def assign():
        out = []
        for x in X:
            best, bj = None, 0
            for j in range(k):
                v = dot(x, C[j])
                if best is None or v > best:
                    best, bj = v, j
            out.append(bj)
        return out

    for _ in range(iters):
        a = assign()
        for j in range(k):
            mem = [X[i] for i in range(n) if a[i] == j]
            if not mem:
                continue
            v = [math.fsum(col) for col in zip(*mem)]
            nv = math.sqrt(math.fsum(t * t for t in v))
            if nv > 0:
                C[j] = [t / nv for t in v]
    return C, assign()


def fp_encode_exhaustive(v, values):
    """Code of the value nearest to v >= 0 among `values` (non-negative,
    indexed by code, NaN entries skipped), ties to the even code."""
    best, bc = None, 0
    for c, val in enumerate(values):
        if val != val:
            continue
        d = abs(v - val)
        if best is None or d < best or (d == best and c % 2 == 0 and bc % 2 == 1):
            best, bc = d, c
    return bc


def log_softmax(s):
    m = max(s)
    lse = math.log(math.fsum(math.exp(t - m) for t in s))
    return [t - m - lse for t in s]


def kl(logp, logq):
    return math.fsum(math.exp(a) * (a - b) for a, b in zip(logp, logq))
