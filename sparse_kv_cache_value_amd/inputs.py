"""Seeded synthetic inputs: random-init weights, prompts and stale caches.

This module only draws random numbers and arranges them into tensors; it holds
none of the caching method's arithmetic.  Both the HIP library and the CPU
oracle consume the bytes it produces (the oracle gets host copies).

Recipe (every tensor is drawn from its own stream, keyed by
``(config seed, layer, tensor id)``):

* matrices ~ N(0, std^2), std = 0.02, drawn in fp32 and rounded (RNE) to the
  config's storage dtype; row-major ``[in, out]`` so that ``y = x @ W``;
* norm gains = 1 (``gain_std > 0`` draws ``1 + gain_std * N(0,1)`` instead,
  which tests use to exercise the gain paths);
* the value projection carries a planted rank-r spectrum so that its
  truncated SVD factor ``W_r = U_r diag(sigma)`` is known by construction:
  ``W_V = U_r diag(sigma) V_r^T + (I - U_r U_r^T) G (I - V_r V_r^T)`` with
  ``U_r, V_r`` orthonormal (QR of Gaussian matrices, fp64 on the host),
  ``G ~ N(0, std^2)`` and ``sigma_j = e (1.35 - 0.25 j/(r-1))`` where
  ``e = std (sqrt(d) + sqrt(n_v))`` is the edge of G's singular spectrum.
  ``W_r`` is shipped with the weights, the way a checkpoint would carry it;
* prompts: ids uniform on ``[0, V-2]``; the rest of each row is the mask id
  ``V-1``.
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

from .configs import Config, FP32

# tensor ids inside a layer
T_ATTN_NORM, T_WQ, T_WK, T_WV, T_WO, T_FFN_NORM, T_WG, T_WU, T_WD, T_PU, T_PV = range(11)
# pseudo-layers
L_HEAD, L_TOKENS, L_STALE = -1, -2, -3


def seed_of(cfg_seed: int, layer: int, tensor_id: int) -> int:
    ss = np.random.SeedSequence([cfg_seed & 0xFFFFFFFF, (layer + 16) & 0xFFFFFFFF, tensor_id])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(seed: int, shape, std: float, device="cpu", dtype=torch.float32) -> torch.Tensor:
    x = torch.randn(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def storage_dtype(cfg: Config) -> torch.dtype:
    return torch.float32 if cfg.dtype == FP32 else torch.bfloat16


def _orthonormal(seed: int, n: int, r: int) -> torch.Tensor:
    a = normal(seed, (n, r), 1.0, "cpu", torch.float32).double()
    q, rr = torch.linalg.qr(a, mode="reduced")
    # fix the sign convention so the factor is unique
    q = q * torch.sign(torch.diagonal(rr)).unsqueeze(0)
    return q


def planted_value_projection(cfg: Config, layer: int, device="cpu"):
    """Return (W_V fp32 [d, n_v], W_r fp32 [d, r], sigma fp64 [r])."""
    d, nv, r, std = cfg.d_model, cfg.n_v, cfg.proxy_rank, cfg.weight_std
    u = _orthonormal(seed_of(cfg.seed, layer, T_PU), d, r)
    v = _orthonormal(seed_of(cfg.seed, layer, T_PV), nv, r)
    e = std * (math.sqrt(d) + math.sqrt(nv))
    j = torch.arange(r, dtype=torch.float64)
    sigma = e * (1.35 - 0.25 * j / max(r - 1, 1))
    wr = (u * sigma.unsqueeze(0)).to(torch.float32)
    g = normal(seed_of(cfg.seed, layer, T_WV), (d, nv), std, device, torch.float32)
    uf, vf = u.to(device=device, dtype=torch.float32), v.to(device=device, dtype=torch.float32)
    if r < nv:
        g = g - uf @ (uf.T @ g)
        g = g - (g @ vf) @ vf.T
    else:
        g.zero_()
    wv = g + (uf * sigma.to(device=device, dtype=torch.float32).unsqueeze(0)) @ vf.T
    return wv, wr.to(device), sigma


def layer_weights(cfg: Config, layer: int, device="cpu", gain_std: float = 0.0) -> Dict[str, torch.Tensor]:
    dt = storage_dtype(cfg)
    d, f, std = cfg.d_model, cfg.d_ffn, cfg.weight_std
    s = lambda t: seed_of(cfg.seed, layer, t)  # noqa: E731

    def gain(t):
        if gain_std <= 0:
            return torch.ones(d, dtype=torch.float32, device=device)
        return 1.0 + normal(s(t), (d,), gain_std, device)

    wv, wr, _ = planted_value_projection(cfg, layer, device)
    return {
        "attn_norm": gain(T_ATTN_NORM),
        "w_q": normal(s(T_WQ), (d, cfg.n_q), std, device, dt),
        "w_k": normal(s(T_WK), (d, cfg.n_v), std, device, dt),
        "w_v": wv.to(dt),
        "w_o": normal(s(T_WO), (cfg.n_q, d), std, device, dt),
        "ffn_norm": gain(T_FFN_NORM),
        "w_gate": normal(s(T_WG), (d, f), std, device, dt),
        "w_up": normal(s(T_WU), (d, f), std, device, dt),
        "w_down": normal(s(T_WD), (f, d), std, device, dt),
        "w_proxy": wr,
    }


def head_weights(cfg: Config, device="cpu", gain_std: float = 0.0) -> Dict[str, torch.Tensor]:
    dt = storage_dtype(cfg)
    d, v, std = cfg.d_model, cfg.vocab, cfg.weight_std
    s = lambda t: seed_of(cfg.seed, L_HEAD, t)  # noqa: E731
    if gain_std > 0:
        fn = 1.0 + normal(s(1), (d,), gain_std, device)
    else:
        fn = torch.ones(d, dtype=torch.float32, device=device)
    return {
        "embed": normal(s(0), (v, d), std, device, dt),
        "final_norm": fn,
        "lm_head": normal(s(2), (d, v), std, device, dt),
    }


def prompt_tokens(cfg: Config, device="cpu"):
    """tokens int32 [B, L] (prompt ids then mask ids) and committed uint8 [B, L]."""
    B, L, P = cfg.batch, cfg.seq_len, cfg.prompt_len
    g = _gen(seed_of(cfg.seed, L_TOKENS, 0), "cpu")
    ids = torch.randint(0, cfg.vocab - 1, (B, P), generator=g, dtype=torch.int64)
    tokens = torch.full((B, L), cfg.mask_id, dtype=torch.int32)
    tokens[:, :P] = ids.to(torch.int32)
    committed = torch.zeros((B, L), dtype=torch.uint8)
    committed[:, :P] = 1
    return tokens.to(device), committed.to(device)


def stale_layer_input(cfg: Config, device="cpu"):
    """Single-layer workload with a stale cache.

    Returns ``(h, h_stale, rows)``: the current layer input h ~ N(0,1) [B, L, d]
    in the storage dtype, the input the cache was built from
    (``h + stale_std * N(0,1)`` on ``rows``), and the sorted perturbed rows
    (``round(stale_frac * L)`` of them per sequence).
    """
    B, L, d = cfg.batch, cfg.seq_len, cfg.d_model
    dt = storage_dtype(cfg)
    h = normal(seed_of(cfg.seed, L_STALE, 0), (B, L, d), 1.0, device, torch.float32)
    noise = normal(seed_of(cfg.seed, L_STALE, 1), (B, L, d), cfg.stale_std, device, torch.float32)
    n_rows = int(round(cfg.stale_frac * L))
    g = _gen(seed_of(cfg.seed, L_STALE, 2), "cpu")
    rows = torch.stack([torch.randperm(L, generator=g)[:n_rows].sort().values for _ in range(B)])
    mask = torch.zeros((B, L, 1), dtype=torch.float32)
    mask.scatter_(1, rows.unsqueeze(-1), 1.0)
    hs = h + noise * mask.to(device)
    return h.to(dt), hs.to(dt), rows.to(torch.int32)
