"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each of them.  This shows that the pins constrain the oracle
beyond restating its own formulas."""

import math

import numpy as np
import pytest

import oracle
import oracle.model as om
import pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(om, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _fails(checks):
    failed = []
    for c in checks:
        try:
            c()
        except AssertionError:
            failed.append(c.__name__)
    return failed


def m_rope_sign(monkeypatch):
    orig = om.rope

    def bad(x, pos, theta, wd=np.float32):
        return orig(x, -np.asarray(pos), theta, wd)
    _patch(monkeypatch, "rope", bad)


def m_drift_unnormalised(monkeypatch):
    def bad(C, P):
        d = np.asarray(C, np.float64) - np.asarray(P, np.float64)
        return 0.5 * np.sum(d * d, axis=-1)
    _patch(monkeypatch, "drift", bad)


def m_drift_abs_cos(monkeypatch):
    def bad(C, P):
        C = np.asarray(C, np.float64); P = np.asarray(P, np.float64)
        nc = np.linalg.norm(C, axis=-1); npp = np.linalg.norm(P, axis=-1)
        with np.errstate(invalid="ignore", divide="ignore"):
            c = np.abs(np.sum(C * P, -1)) / (nc * npp)
        return np.where((nc == 0) & (npp == 0), 0.0, np.where((nc == 0) | (npp == 0), 1.0, 1.0 - c))
    _patch(monkeypatch, "drift", bad)


def m_select_high_index_ties(monkeypatch):
    def bad(s, forced, k):
        s = np.asarray(s, np.float64); L = len(s)
        forced = np.zeros(L, bool) if forced is None else np.asarray(forced, bool)
        F = [i for i in range(L) if forced[i]]
        keff = min(max(k, len(F)), L)
        rest = sorted((i for i in range(L) if not forced[i]), key=lambda i: (-s[i], -i))
        return np.array(sorted(F + rest[: keff - len(F)]), np.int64)
    _patch(monkeypatch, "select", bad)


def m_scatter_after_attention(monkeypatch):
    def bad(x, K, V, H_out, idx, W, spec):
        idx = np.asarray(idx, np.int64)
        if idx.size == 0:
            return
        x = np.asarray(x, spec.wd)
        xr = x[idx]
        a = om._act(om.rmsnorm(xr, W["attn_norm"], spec.rms_eps, spec.wd), spec)
        q, k, v = om._qkv(a, W, idx, spec)
        H_out[idx] = om._attn_out_ffn(xr, q, K, V, W, spec)
        K[idx] = k
        V[idx] = v
    _patch(monkeypatch, "sparse_layer", bad)
    monkeypatch.setattr(oracle.decode, "sparse_layer", bad)


def m_entropy_sign(monkeypatch):
    orig = om.lm_stats

    def bad(h, g_f, w_lm, spec):
        st = orig(h, g_f, w_lm, spec)
        st["entropy"] = np.log(st["S"]) + st["T"] / st["S"]
        return st
    _patch(monkeypatch, "lm_stats", bad)


def m_drop_ffn_residual(monkeypatch):
    def bad(x_rows, q, K, V, W, spec):
        n = x_rows.shape[0]
        o = om._act(om.attention(q, K, V, spec.wd).reshape(n, -1), spec)
        h1 = (np.asarray(x_rows, spec.wd) + om._mm(o, W["w_o"], spec)).astype(spec.wd)
        nrm = om._act(om.rmsnorm(h1, W["ffn_norm"], spec.rms_eps, spec.wd), spec)
        act = om._silu(om._mm(nrm, W["w_gate"], spec)) * om._mm(nrm, W["w_up"], spec)
        return om._act(om._mm(act.astype(spec.wd), W["w_down"], spec), spec)
    _patch(monkeypatch, "_attn_out_ffn", bad)


def m_gqa_modulo(monkeypatch):
    def bad(q, K, V, wd=np.float32):
        q = np.asarray(q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
        n, hq, dh = q.shape
        hkv = K.shape[1]
        out = np.empty((n, hq, dh))
        for h in range(hq):
            g = h % hkv
            s = q[:, h] @ K[:, g].T / math.sqrt(dh)
            p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
            out[:, h] = p @ V[:, g]
        return out.astype(wd)
    _patch(monkeypatch, "attention", bad)


def m_proxy_drops_gain(monkeypatch):
    def bad(x, g1, w_r):
        return np.asarray(x, np.float64) @ np.asarray(w_r, np.float64)
    _patch(monkeypatch, "proxy", bad)
    monkeypatch.setattr(oracle.decode, "proxy", bad)


def m_commit_last_on_ties(monkeypatch):
    def bad(rows, conf, argmax, entropy, committed, threshold):
        cand = [j for j in range(len(rows)) if not committed[rows[j]]]
        pick = [j for j in cand if conf[j] >= threshold]
        if not pick and cand:
            pick = [sorted(cand, key=lambda j: (-conf[j], -rows[j]))[0]]
        pick.sort(key=lambda j: rows[j])
        return ([int(rows[j]) for j in pick], [int(argmax[j]) for j in pick],
                max((float(entropy[j]) for j in pick), default=0.0))
    _patch(monkeypatch, "commit", bad)


def m_budget_truncates(monkeypatch):
    _patch(monkeypatch, "budget_k", lambda rho, L: int(math.floor(rho * L)))


def m_key_uses_query_weights(monkeypatch):
    def bad(a, W, pos, spec):
        n = a.shape[0]
        H, G, dh = spec.n_q_heads, spec.n_kv_heads, spec.head_dim
        q = om._mm(a, W["w_q"], spec).reshape(n, H, dh)
        k = om._mm(a, W["w_q"], spec)[:, : G * dh].reshape(n, G, dh)
        v = om._mm(a, W["w_v"], spec).reshape(n, G, dh)
        q = om._act(om.rope(q, pos, spec.rope_theta, spec.wd), spec)
        k = om._act(om.rope(k, pos, spec.rope_theta, spec.wd), spec)
        return q, k, om._act(v, spec)
    _patch(monkeypatch, "_qkv", bad)


MUTATIONS = [m_rope_sign, m_drift_unnormalised, m_drift_abs_cos, m_select_high_index_ties,
             m_scatter_after_attention, m_entropy_sign, m_drop_ffn_residual, m_gqa_modulo,
             m_proxy_drops_gain, m_commit_last_on_ties, m_budget_truncates,
             m_key_uses_query_weights]


# ---- Polestar drift path ----
import oracle.polestar as ops  # noqa: E402


def m_fp_ties_up(monkeypatch):
    def bad(v, grid):
        if not v > 0.0:
            return 0
        if v >= grid[-1]:
            return len(grid) - 1
        hi = 1
        while grid[hi] < v:
            hi += 1
        lo = hi - 1
        return lo if v - grid[lo] < grid[hi] - v else hi
    monkeypatch.setattr(ops, "_rne_on_grid", bad)


def m_kmeans_mean_not_normalised(monkeypatch):
    def bad(X, n_clusters, iters):
        X = np.asarray(X, np.float64)
        n = X.shape[0]
        C = X[(n // n_clusters) * np.arange(n_clusters)].copy()
        for _ in range(iters):
            a = np.argmax(X @ C.T, axis=1)
            for j in range(n_clusters):
                if (a == j).any():
                    C[j] = X[a == j].mean(axis=0)
        D = X @ C.T
        a = np.argmax(D, axis=1)
        return C, a, [0.0], D
    monkeypatch.setattr(ops, "spherical_kmeans", bad)


def m_kl_reversed(monkeypatch):
    def bad(logA, logA_prev):
        logA = np.asarray(logA, np.float64); lp = np.asarray(logA_prev, np.float64)
        return np.mean(np.sum(np.exp(lp) * (lp - logA), axis=2), axis=1)
    monkeypatch.setattr(ops, "cluster_kl", bad)


def m_window_unclamped(monkeypatch):
    monkeypatch.setattr(ops, "window_start", lambda bs, L, blk, wb=3: int(max(bs - blk, 0)))


def m_proxy_attention_unscaled(monkeypatch):
    orig = ops.proxy_log_attention

    def bad(q, Kw):
        return orig(np.asarray(q, np.float64) * math.sqrt(np.asarray(q).shape[-1]), Kw)
    monkeypatch.setattr(ops, "proxy_log_attention", bad)


def m_top_clusters_high_ties(monkeypatch):
    def bad(kl, top):
        kl = np.asarray(kl, np.float64)
        order = sorted(range(kl.size), key=lambda j: (-kl[j], -j))
        return np.array(sorted(order[:top]), np.int64)
    monkeypatch.setattr(ops, "top_clusters", bad)


def _drift_commit_variant(monkeypatch, rule):
    """Replace the drift test of Polestar-Commit by ``rule(delta, c, tau_s,
    alpha)``; everything else as in the oracle."""
    orig = ops.drift_commit

    def bad(cur_rows, cur, suf_rows, suf, committed, tau_s, alpha, D, hist_sum, hist_cnt, hit):
        n = len(cur_rows)
        cand = [j for j in range(n) if not committed[cur_rows[j]]]
        pick = []
        for j in cand:
            c = float(cur["conf"][j])
            if c >= tau_s:
                pick.append(j)
            elif D is not None and hist_cnt[j] > 0:
                if rule(float(D[j]) - float(hist_sum[j]) / float(hist_cnt[j]), c, tau_s, alpha):
                    pick.append(j)
        if not pick:
            return orig(cur_rows, cur, suf_rows, suf, committed, tau_s, alpha, None, hist_sum, hist_cnt, hit)
        pick.sort()
        spick = [j for j in range(len(suf_rows)) if hit and not committed[suf_rows[j]] and suf["conf"][j] >= tau_s]
        pos = [int(cur_rows[j]) for j in pick] + [int(suf_rows[j]) for j in spick]
        tok = [int(cur["argmax"][j]) for j in pick] + [int(suf["argmax"][j]) for j in spick]
        ents = [float(cur["entropy"][j]) for j in pick] + [float(suf["entropy"][j]) for j in spick]
        fl = np.zeros(n, bool)
        fl[pick] = True
        return pos, tok, max(ents, default=0.0), fl
    monkeypatch.setattr(ops, "drift_commit", bad)


def m_commit_threshold_not_squared(monkeypatch):
    _drift_commit_variant(monkeypatch, lambda dl, c, ts, a: dl > a * (ts - c))


def m_commit_nonstrict(monkeypatch):
    _drift_commit_variant(monkeypatch, lambda dl, c, ts, a: dl >= a * (ts - c) ** 2)


def m_commit_raw_drift(monkeypatch):
    # the drift itself instead of its deviation from the historical mean
    orig = ops.drift_commit

    def bad(cur_rows, cur, suf_rows, suf, committed, tau_s, alpha, D, hist_sum, hist_cnt, hit):
        return orig(cur_rows, cur, suf_rows, suf, committed, tau_s, alpha, D, np.zeros_like(hist_sum),
                    hist_cnt, hit)
    monkeypatch.setattr(ops, "drift_commit", bad)


def m_suffix_any_conf(monkeypatch):
    orig = ops.drift_commit

    def bad(cur_rows, cur, suf_rows, suf, committed, tau_s, alpha, D, hist_sum, hist_cnt, hit):
        s2 = dict(suf)
        s2["conf"] = np.maximum(np.asarray(suf["conf"], np.float64), tau_s)
        return orig(cur_rows, cur, suf_rows, s2, committed, tau_s, alpha, D, hist_sum, hist_cnt, hit)
    monkeypatch.setattr(ops, "drift_commit", bad)


def m_suffix_hit_includes_block(monkeypatch):
    def bad(block_start, blk, wstart, assign, top):
        a = np.asarray(assign)
        first = block_start - wstart  # the current block counted as suffix
        return any(int(a[r]) in set(int(t) for t in top) for r in range(max(first, 0), a.size))
    monkeypatch.setattr(ops, "suffix_hit", bad)


MUTATIONS += [m_fp_ties_up, m_kmeans_mean_not_normalised, m_kl_reversed, m_window_unclamped,
              m_proxy_attention_unscaled, m_top_clusters_high_ties, m_commit_threshold_not_squared,
              m_commit_nonstrict, m_commit_raw_drift, m_suffix_any_conf, m_suffix_hit_includes_block]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    assert _fails(pins.ALL_CHECKS), f"no pin catches {mutation.__name__}"


# ---- Confidence Extrapolation ----
import oracle.extrapolation as oce  # noqa: E402


def m_ce_predict_drops_quarter_q(monkeypatch):
    def bad(s, p):
        x0, x1, a, b, d = s
        return [x0 + x1, x1, a + 2.0 * b + d, b + d + p.q / 2.0, d + p.q]
    monkeypatch.setattr(oce, "kf_predict", bad)


def m_ce_gain_swapped(monkeypatch):
    def bad(s, c, p):
        x0, x1, a, b, d = s
        S = a + p.r
        k0, k1 = b / S, a / S
        y = float(c) - x0
        return [x0 + k0 * y, x1 + k1 * y, a - k0 * a, b - k0 * b, d - k1 * b]
    monkeypatch.setattr(oce, "kf_update", bad)


def m_ce_forecast_not_propagated(monkeypatch):
    def bad(s, p):
        x0, x1, a, b, d = s
        return [x0 + h * x1 - p.kappa * math.sqrt(a) for h in range(1, p.horizon + 1)]
    monkeypatch.setattr(oce, "forecast_bounds", bad)


def m_ce_coverage_counts_self(monkeypatch):
    orig = oce.ce_commit

    def bad(rows, conf, argmax, entropy, committed, threshold, states, p):
        # coverage over the positions up to and including the token
        n = len(rows)
        cand = [j for j in range(n) if not committed[rows[j]]]
        for j in cand:
            states[j] = oce.kf_observe(states[j], conf[j], p)
        early = np.zeros(n, bool)
        pick = []
        for j in cand:
            if conf[j] >= threshold:
                pick.append(j)
                continue
            cov = sum(1 for i in range(j) if committed[rows[i]]) / (j + 1)
            if cov >= p.gamma and max(oce.forecast_bounds(states[j], p)) >= threshold:
                pick.append(j)
                early[j] = True
        if not pick and cand:
            best = max(cand, key=lambda j: (conf[j], -j))
            pick = [best]
        pick.sort()
        return ([int(rows[j]) for j in pick], [int(argmax[j]) for j in pick],
                max((float(entropy[j]) for j in pick), default=0.0), early)
    monkeypatch.setattr(oce, "ce_commit", bad)


CE_MUTATIONS = [m_ce_predict_drops_quarter_q, m_ce_gain_swapped, m_ce_forecast_not_propagated,
                m_ce_coverage_counts_self]


@pytest.mark.parametrize("mutation", CE_MUTATIONS, ids=lambda f: f.__name__)
def test_ce_mutation_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    assert _fails(pins.ALL_CHECKS), f"no pin catches {mutation.__name__}"


# ---- Polestar refresh schedule ----
def m_refresh_strict(monkeypatch):
    def bad(prev, ws, n_decoded, pp):
        if pp.tau_upd <= 0 or prev.logA is None or prev.wstart != ws:
            return True
        return n_decoded - prev.hist_at_update > pp.tau_upd
    monkeypatch.setattr(ops, "refresh_due", bad)


def m_refresh_ignores_window(monkeypatch):
    def bad(prev, ws, n_decoded, pp):
        if pp.tau_upd <= 0 or prev.logA is None:
            return True
        return n_decoded - prev.hist_at_update >= pp.tau_upd
    monkeypatch.setattr(ops, "refresh_due", bad)


@pytest.mark.parametrize("mutation", [m_refresh_strict, m_refresh_ignores_window], ids=lambda f: f.__name__)
def test_schedule_mutation_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    assert _fails(pins.ALL_CHECKS), f"no pin catches {mutation.__name__}"


# ---- EntropyCache gate, forced set, cached-proxy refresh (decode loop) ----
import oracle.decode as od


def _commit_variant(monkeypatch, emax_of):
    """Threshold commit whose reported entropy is ``emax_of(entropy, picks, cand)``."""
    orig = od.commit

    def bad(rows, conf, argmax, entropy, committed, threshold):
        pos, tok, _ = orig(rows, conf, argmax, entropy, committed, threshold)
        picks = [j for j in range(len(rows)) if int(rows[j]) in pos]
        cand = [j for j in range(len(rows)) if not committed[rows[j]]]
        return pos, tok, emax_of(entropy, picks, cand)
    monkeypatch.setattr(od, "commit", bad)


def m_gate_zero_entropy(monkeypatch):
    _commit_variant(monkeypatch, lambda e, p, c: 0.0)


def m_gate_first_commit(monkeypatch):
    _commit_variant(monkeypatch, lambda e, p, c: float(e[p[0]]) if p else 0.0)


def m_gate_block_max(monkeypatch):
    _commit_variant(monkeypatch, lambda e, p, c: max((float(e[j]) for j in c), default=0.0))


def m_gate_nonstrict(monkeypatch):
    orig = od.commit_block

    def bad(st, head, spec, pol):
        info = orig(st, head, spec, pol)
        st.full_next = info["emax"] >= pol.tau
        return info
    monkeypatch.setattr(od, "commit_block", bad)


def _forced_variant(monkeypatch, recent_of, with_block=True):
    def bad(self, pol):
        f = np.zeros(self.spec.seq_len, bool)
        if pol.forced in ("block", "block+recent") and (with_block or pol.forced == "block"):
            f[self.block_rows()] = True
        if pol.forced == "block+recent" and pol.recent_k > 0:
            f[recent_of(list(self.history), pol.recent_k)] = True
        return f
    monkeypatch.setattr(od.SeqState, "forced_set", bad)


def m_forced_oldest(monkeypatch):
    _forced_variant(monkeypatch, lambda h, k: h[:k])


def m_forced_by_position(monkeypatch):
    _forced_variant(monkeypatch, lambda h, k: sorted(h)[-k:])


def m_forced_drops_block(monkeypatch):
    _forced_variant(monkeypatch, lambda h, k: h[-k:], with_block=False)


def _refresh_variant(monkeypatch, update):
    def bad(x, K, V, H_out, P, W, spec, k, forced):
        C = om.proxy(x, W["attn_norm"], W["w_proxy"])
        s = om.drift(C, P)
        I = np.arange(spec.seq_len) if k is None else om.select(s, forced, k)
        om.sparse_layer(x, K, V, H_out, I, W, spec)
        update(P, C, I)
        return I, s, C
    monkeypatch.setattr(od, "layer_refresh", bad)


def m_refresh_every_row(monkeypatch):
    def upd(P, C, I):
        P[:] = C
    _refresh_variant(monkeypatch, upd)


def m_refresh_nothing(monkeypatch):
    _refresh_variant(monkeypatch, lambda P, C, I: None)


DECODE_MUTATIONS = [m_gate_zero_entropy, m_gate_first_commit, m_gate_block_max, m_gate_nonstrict,
                    m_forced_oldest, m_forced_by_position, m_forced_drops_block,
                    m_refresh_every_row, m_refresh_nothing]


@pytest.mark.parametrize("mutation", DECODE_MUTATIONS, ids=lambda f: f.__name__)
def test_decode_mutation_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    assert _fails(pins.ALL_CHECKS), f"no pin catches {mutation.__name__}"
