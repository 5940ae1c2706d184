"""Oracle decoding loop: full pass, sparse steps, forced sets and the entropy
gate, one sequence at a time.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Readings (where the pages leave the step open):
* Semi-autoregressive blocks of ``block_len`` left to right; the current block
  is the first one that still holds a masked row.  Tokens are the greedy
  argmax.  Step 0 is a full pass and also commits.
* Cached per layer: K, V, the layer output and the proxy P at the row's last
  refresh.  The current proxy C is recomputed for every row, so only rows
  whose layer input changed can show drift.
* EntropyCache gate (section 2, step 3): the maximum entropy over the tokens
  committed in this step decides the mode of the next step (full iff > tau).
* Forced sets: "block+recent" = every row of the current block plus the last
  ``recent_k`` entries of the decode history (EntropyCache); "block" = the
  current block (Polestar); "none" = drift alone (SPA-Cache).
* Confidence Extrapolation (TSPD + CE page, section 2) optionally adds early
  commits to the threshold commit (``extrapolation.ce_commit``).
* Commit rule: "threshold" (static confidence threshold) or "polestar"
  (Polestar section 2B, see ``polestar.drift_commit``; it needs the Polestar
  drift path and uses its last layer's cluster drift).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .model import (Spec, budget_k, commit, drift, lm_stats, proxy, select,
                    sparse_layer)
from . import extrapolation, polestar


@dataclasses.dataclass
class Policy:
    rho: tuple
    forced: str = "none"
    recent_k: int = 0
    tau: float = float("inf")
    conf_threshold: float = 0.9
    score: str = "spa_cos"          # or "polestar_kl" (Polestar section 2A drift path)
    polestar: polestar.PolestarParams = dataclasses.field(default_factory=polestar.PolestarParams)
    commit: str = "threshold"       # or "polestar" (Polestar section 2B)
    commit_alpha: float = 1.0       # Polestar-Commit alpha
    ce: Optional[extrapolation.CEParams] = None  # Confidence Extrapolation on the threshold commit


class SeqState:
    """Cache and decode state of one sequence."""

    def __init__(self, spec: Spec, tokens, committed):
        L, N = spec.seq_len, spec.n_layers
        self.spec = spec
        self.tokens = np.array(tokens, np.int64).reshape(L)
        self.committed = np.array(committed, bool).reshape(L)
        self.history: List[int] = []
        self.block_start = 0
        self.advance_block()
        self.H = np.zeros((N + 1, L, spec.d_model), spec.wd)
        self.K = np.zeros((N, L, spec.n_kv_heads, spec.head_dim), spec.wd)
        self.V = np.zeros_like(self.K)
        self.P = np.zeros((N, L, spec.proxy_rank), np.float64)
        self.full_next = True
        self.n_new = 0
        self.ps = [polestar.PolestarLayerState() for _ in range(N)]
        # Polestar-Commit: sum and count of the current block rows' past drifts
        self.drift_sum = np.zeros(spec.block_len, np.float64)
        self.drift_cnt = np.zeros(spec.block_len, np.int64)
        # Confidence Extrapolation: filter state per current block position
        self.ce_states = [None] * spec.block_len
        # Polestar schedule: steps since the last full pass
        self.steps_since_full = 0

    def advance_block(self):
        L, b = self.spec.seq_len, self.spec.block_len
        while self.block_start < L and self.committed[self.block_start:self.block_start + b].all():
            self.block_start += b

    def block_rows(self):
        L = self.spec.seq_len
        return np.arange(self.block_start, min(self.block_start + self.spec.block_len, L))

    def forced_set(self, pol: Policy):
        f = np.zeros(self.spec.seq_len, bool)
        if pol.forced in ("block", "block+recent"):
            f[self.block_rows()] = True
        if pol.forced == "block+recent" and pol.recent_k > 0:
            f[self.history[-pol.recent_k:]] = True
        return f

    def done(self):
        return self.block_start >= self.spec.seq_len


def layer_refresh(x, K, V, H_out, P, W, spec: Spec, k: Optional[int], forced):
    """One layer of a step: proxy of every row, drift against P, index set I,
    sparse execution on I, then P[I] <- C[I].  k=None means I = every row
    (full-pass mode).  Returns (I, s, C)."""
    C = proxy(x, W["attn_norm"], W["w_proxy"])
    s = drift(C, P)
    if k is None:
        I = np.arange(spec.seq_len)
    else:
        I = select(s, forced, k)
    sparse_layer(x, K, V, H_out, I, W, spec)
    P[I] = C[I]
    return I, s, C


def step(st: SeqState, layers, head, spec: Spec, pol: Policy, force_mode: Optional[str] = None):
    """One denoising step.  Mode is full when the previous step's gate fired
    (or at step 0), sparse otherwise; ``force_mode`` ("full"/"sparse")
    overrides.  Returns a dict with the per-layer index sets and scores, the
    block statistics and the commits."""
    full = st.full_next if force_mode is None else (force_mode == "full")
    # periodic full pass (Polestar section 2A, schedule): counted in steps
    # since the last periodic or explicitly requested full pass, apart from
    # the entropy gate
    fp = pol.polestar.full_period if pol.score == "polestar_kl" else 0
    periodic = force_mode is None and fp > 0 and st.steps_since_full + 1 >= fp
    full = full or periodic
    st.steps_since_full = 0 if (periodic or force_mode == "full") else st.steps_since_full + 1
    st.H[0] = np.asarray(head["embed"], spec.wd)[st.tokens]
    forced = st.forced_set(pol)
    sets, scores, ps_info = [], [], []
    for l in range(spec.n_layers):
        if pol.score == "polestar_kl" and not full:
            # Polestar: the drift path picks the rows; no value proxy involved
            r = polestar.drift_and_select(st.H[l], st.K[l], st.block_start, layers[l], spec, pol.polestar,
                                          st.ps[l], len(st.history))
            sparse_layer(st.H[l], st.K[l], st.V[l], st.H[l + 1], r["I"], layers[l], spec)
            sets.append(r["I"])
            scores.append(r["kl"])
            ps_info.append(r)
            continue
        k = None if full else budget_k(pol.rho[l], spec.seq_len)
        I, s, _ = layer_refresh(st.H[l], st.K[l], st.V[l], st.H[l + 1], st.P[l],
                                layers[l], spec, k, forced)
        sets.append(I)
        scores.append(s)
    info = {"full": full, "sets": sets, "scores": scores, "forced": forced, "polestar": ps_info}
    if pol.commit == "polestar":
        info.update(commit_block_polestar(st, head, spec, pol, ps_info[-1] if ps_info else None))
    else:
        info.update(commit_block(st, head, spec, pol))
    return info


def commit_block(st: SeqState, head, spec: Spec, pol: Policy):
    rows = st.block_rows()
    if rows.size == 0:
        st.n_new = 0
        st.full_next = False
        return {"rows": rows, "stats": None, "pos": [], "tok": [], "emax": 0.0}
    stats = lm_stats(st.H[spec.n_layers][rows], head["final_norm"], head["lm_head"], spec)
    early = None
    if pol.ce is not None:
        pos, tok, emax, early = extrapolation.ce_commit(rows, stats["conf"], stats["argmax"], stats["entropy"],
                                                        st.committed, pol.conf_threshold, st.ce_states, pol.ce)
    else:
        pos, tok, emax = commit(rows, stats["conf"], stats["argmax"], stats["entropy"],
                                st.committed, pol.conf_threshold)
    bs = st.block_start
    for p, t in zip(pos, tok):
        st.tokens[p] = t
        st.committed[p] = True
        st.history.append(p)
    st.n_new = len(pos)
    st.advance_block()
    if st.block_start != bs:
        st.ce_states = [None] * spec.block_len
    st.full_next = emax > pol.tau
    return {"rows": rows, "stats": stats, "pos": pos, "tok": tok, "emax": emax, "early": early}


def commit_block_polestar(st: SeqState, head, spec: Spec, pol: Policy, last):
    """Polestar-Commit of one step; ``last`` is the last layer's drift-path
    result of this step (None in a full step)."""
    L, blk = spec.seq_len, spec.block_len
    rows = st.block_rows()
    if rows.size == 0:
        st.n_new = 0
        st.full_next = False
        return {"rows": rows, "stats": None, "pos": [], "tok": [], "emax": 0.0}
    bs = st.block_start
    srows = np.arange(bs + blk, min(bs + 2 * blk, L))
    both = np.concatenate([rows, srows])
    stats = lm_stats(st.H[spec.n_layers][both], head["final_norm"], head["lm_head"], spec)
    n = rows.size
    cur = {k: stats[k][:n] for k in ("conf", "argmax", "entropy")}
    suf = {k: stats[k][n:] for k in ("conf", "argmax", "entropy")}
    valid = last is not None and last["valid"]
    D = polestar.token_drift(rows, last["wstart"], last["assign"], last["kl"]) if valid else None
    hit = valid and polestar.suffix_hit(bs, blk, last["wstart"], last["assign"], last["top"])
    pos, tok, emax, _ = polestar.drift_commit(rows, cur, srows, suf, st.committed, pol.conf_threshold,
                                              pol.commit_alpha, D, st.drift_sum[:n], st.drift_cnt[:n], hit)
    if D is not None:
        st.drift_sum[:n] += D
        st.drift_cnt[:n] += 1
    for p, t in zip(pos, tok):
        st.tokens[p] = t
        st.committed[p] = True
        st.history.append(p)
    st.n_new = len(pos)
    st.advance_block()
    if st.block_start != bs:
        st.drift_sum[:] = 0.0
        st.drift_cnt[:] = 0
    st.full_next = emax > pol.tau
    return {"rows": rows, "srows": srows, "stats": stats, "pos": pos, "tok": tok, "emax": emax, "D": D,
            "hit": hit}
