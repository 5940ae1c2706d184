"""Test helpers: config -> oracle spec, tensors -> numpy, tolerance metric."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from sparse_kv_cache_value_amd import configs, inputs


def spec_of(cfg: configs.Config, **kw) -> oracle.Spec:
    base = dict(
        n_layers=cfg.n_layers, d_model=cfg.d_model, n_q_heads=cfg.n_q_heads,
        n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, d_ffn=cfg.d_ffn,
        vocab=cfg.vocab, seq_len=cfg.seq_len, block_len=cfg.block_len,
        proxy_rank=cfg.proxy_rank, rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
        bf16=(cfg.dtype == configs.BF16),
    )
    base.update(kw)
    return oracle.Spec(**base)


def policy_of(cfg: configs.Config, **kw) -> oracle.decode.Policy:
    base = dict(rho=cfg.rho, forced=cfg.forced, recent_k=cfg.recent_k, tau=cfg.tau,
                conf_threshold=cfg.conf_threshold, score=cfg.score,
                polestar=oracle.polestar.PolestarParams(cfg.n_clusters, cfg.kmeans_iters, cfg.top_clusters,
                                                        cfg.window_blocks))
    base.update(kw)
    return oracle.decode.Policy(**base)


def np32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float32).numpy()
    return np.asarray(t, np.float32)


def np_weights(w: dict) -> dict:
    return {k: np32(v) for k, v in w.items()}


def model_np(cfg: configs.Config, gain_std: float = 0.0, device="cpu"):
    layers = [np_weights(inputs.layer_weights(cfg, l, device, gain_std)) for l in range(cfg.n_layers)]
    head = np_weights(inputs.head_weights(cfg, device, gain_std))
    return layers, head


def rel_err(a, b) -> float:
    """max|a - b| / max|b| (the parity metric for float tensors)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def tiny_cfg(**kw) -> configs.Config:
    """Tiny model for brute-force checks: d = 8, 2 heads x 4, F = 16, V = 11, L = 6."""
    base = dict(name="brute", seed=11, n_layers=2, d_model=8, n_q_heads=2, n_kv_heads=2,
                head_dim=4, d_ffn=16, vocab=11, batch=1, seq_len=6, prompt_len=2,
                block_len=2, proxy_rank=3, dtype=configs.FP32, rho=(0.5, 0.34),
                weight_std=0.3)
    base.update(kw)
    return configs.Config(**base)
