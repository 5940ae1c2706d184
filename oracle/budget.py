"""Per-layer update ratio rho(l) (SPA-Cache, method step 2).

TEST INFRASTRUCTURE ONLY.

The page parameterises rho(l) as a piecewise Gaussian that is low for the
early layers, peaks in the middle layers and falls again for the late ones; it
gives no constants.  Reading: a split Gaussian on a floor of 0.04,
rho(l) = 0.04 + (rho_pk - 0.04) exp(-(l - mu)^2 / (2 sigma^2)), mu = (N-1)/2,
sigma = N/4 on the rising side and N/6 on the falling side, rho_pk chosen by
bisection so that the mean over layers is the target ratio (16%, the mean the
page's ablation reports).
"""

import math


def split_gaussian(n_layers: int, mean: float = 0.16, floor: float = 0.04):
    mu = (n_layers - 1) / 2.0

    def table(pk):
        out = []
        for l in range(n_layers):
            sig = n_layers / 4.0 if l <= mu else n_layers / 6.0
            out.append(floor + (pk - floor) * math.exp(-((l - mu) ** 2) / (2.0 * sig * sig)))
        return out

    lo, hi = floor, 1.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if sum(table(mid)) / n_layers < mean:
            lo = mid
        else:
            hi = mid
    return table(0.5 * (lo + hi))
