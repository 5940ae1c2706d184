"""Confidence Extrapolation (TSPD + CE page, method section 2 "Confidence
Extrapolation").

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the page states:
- The evolution of each token's confidence is modelled as a latent
  state-space process (Kalman-filter-like).  The observed confidence is a
  noisy observation of a latent confidence level and its velocity.
- From it, near-future confidence is forecast together with a quantified
  uncertainty.
- A risk-aware horizon rule sets the largest look-ahead from two factors:
  left-context coverage (enough earlier tokens are already fixed to give
  reliable context) and an uncertainty bound (a conservative lower bound of
  the forecast confidence).
- When the forecast lower bound clears the minimum threshold the token is
  committed early.  The module is training-free and sits on top of any
  decoding controller, here the static-threshold commit.

Readings (the page gives no model matrices, noise levels or constants):
- **Model.** A constant-velocity Kalman filter per masked position of the
  current block, fp64: state (level, velocity), transition
  F = [[1, 1], [0, 1]] per denoising step, observation H = [1, 0] of the
  top-1 confidence, process noise Q = q [[1/4, 1/2], [1/2, 1]] (white
  acceleration held over one step), observation noise r.
- **Start.** At a position's first observation in the block: state (c, 0),
  covariance diag(r, p_v0).  Every later step: predict, then update with the
  new confidence.  Only still-masked positions are filtered; the states of
  the block are dropped when the block advances.
- **Forecast and bound.** For h = 1 .. H: mean level + h velocity, variance
  from propagating the posterior covariance h steps (P <- F P F^T + Q), lower
  bound = mean - kappa sqrt(variance).
- **Horizon rule.** Left-context coverage of a position = the fraction of
  the current block's positions to its left that were committed before this
  step (1 for the block's first position).  A position may commit early only
  when its coverage is at least gamma; the horizon is then H.  It commits
  early when some h in 1 .. H has a lower bound >= the commit threshold.
- **Integration.** A masked position commits when its confidence clears the
  threshold (the base controller) or by extrapolation; if none commits, the
  most confident masked position does (lowest position on ties), as in the
  threshold commit.
- **Arithmetic order.** Predict: P00 + 2 P01 + P11 + q/4, P01 + P11 + q/2,
  P11 + q.  Update: S = P00 + r, K = (P00/S, P01/S), y = c - level;
  level + K0 y, velocity + K1 y; P00 - K0 P00, P01 - K0 P01, P11 - K1 P01.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class CEParams:
    horizon: int = 2        # H
    q: float = 1e-4         # process noise scale
    r: float = 1e-3         # observation noise variance
    p_v0: float = 1e-2      # initial velocity variance
    kappa: float = 2.0      # lower bound = mean - kappa * std
    gamma: float = 0.5      # minimum left-context coverage


def kf_init(c: float, p: CEParams):
    """State (level, velocity, P00, P01, P11) at the first observation."""
    return [float(c), 0.0, p.r, 0.0, p.p_v0]


def kf_predict(s, p: CEParams):
    x0, x1, a, b, d = s
    return [x0 + x1, x1, a + 2.0 * b + d + p.q / 4.0, b + d + p.q / 2.0, d + p.q]


def kf_update(s, c: float, p: CEParams):
    x0, x1, a, b, d = s
    S = a + p.r
    k0, k1 = a / S, b / S
    y = float(c) - x0
    return [x0 + k0 * y, x1 + k1 * y, a - k0 * a, b - k0 * b, d - k1 * b]


def kf_observe(s: Optional[list], c: float, p: CEParams):
    """One step of the filter for a new confidence observation."""
    if s is None:
        return kf_init(c, p)
    return kf_update(kf_predict(s, p), c, p)


def forecast_bounds(s, p: CEParams) -> List[float]:
    """Lower bounds of the forecast confidence at h = 1 .. H."""
    x0, x1, a, b, d = s
    out = []
    for h in range(1, p.horizon + 1):
        a, b, d = a + 2.0 * b + d + p.q / 4.0, b + d + p.q / 2.0, d + p.q
        out.append(x0 + h * x1 - p.kappa * math.sqrt(a))
    return out


def ce_commit(rows, conf, argmax, entropy, committed, threshold: float, states: list, p: CEParams):
    """One step of the threshold commit with Confidence Extrapolation.

    rows: current block positions [n]; conf/argmax/entropy: their
    statistics; committed: bool [L] (not modified); states: per block
    position, None or the filter state before this step -- updated in place
    for the masked positions.  Returns (positions committed in ascending
    order, tokens, max entropy over them, early-commit flags)."""
    n = len(rows)
    cand = [j for j in range(n) if not committed[rows[j]]]
    for j in cand:
        states[j] = kf_observe(states[j], conf[j], p)
    early = np.zeros(n, bool)
    pick = []
    for j in cand:
        if conf[j] >= threshold:
            pick.append(j)
            continue
        left = sum(1 for i in range(j) if committed[rows[i]])
        coverage = 1.0 if j == 0 else left / j
        if coverage >= p.gamma and max(forecast_bounds(states[j], p)) >= threshold:
            pick.append(j)
            early[j] = True
    if not pick and cand:
        best = cand[0]
        for j in cand[1:]:
            if conf[j] > conf[best]:
                best = j
        pick = [best]
    pick.sort()
    pos = [int(rows[j]) for j in pick]
    tok = [int(argmax[j]) for j in pick]
    emax = max((float(entropy[j]) for j in pick), default=0.0)
    return pos, tok, emax, early
