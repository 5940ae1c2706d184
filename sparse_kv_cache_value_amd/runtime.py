"""Device-side model and decode-state helpers over the C-ABI.

``Model`` creates a libdllm model and hands it the (seeded, synthetic)
weights; ``State`` allocates the caller-owned decode state as torch tensors in
the layouts include/libdllm.h documents.  Nothing here computes any part of
the decoding step.
"""

from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import binding as B
from . import inputs
from .configs import BF16, FP32, Config, FORCED_BLOCK, FORCED_BLOCK_RECENT, FORCED_NONE, SCORE_POLESTAR

FORCED_RULE = {FORCED_NONE: B.DLLM_FORCED_NONE, FORCED_BLOCK: B.DLLM_FORCED_BLOCK,
               FORCED_BLOCK_RECENT: B.DLLM_FORCED_BLOCK_RECENT}


def dims_of(cfg: Config, max_batch: Optional[int] = None) -> B.DllmDims:
    return B.DllmDims(
        cfg.n_layers, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ffn, cfg.vocab,
        max_batch or cfg.batch, cfg.seq_len, cfg.block_len, cfg.proxy_rank,
        B.DLLM_FP32 if cfg.dtype == FP32 else B.DLLM_BF16, cfg.rms_eps, cfg.rope_theta)


class Model:
    """A libdllm model holding one config's weights (library-owned copies)."""

    def __init__(self, cfg: Config, device="cuda", gain_std: float = 0.0,
                 layers: Optional[List[Dict[str, torch.Tensor]]] = None,
                 head: Optional[Dict[str, torch.Tensor]] = None, max_batch: Optional[int] = None):
        self.cfg = cfg
        self.device = torch.device(device)
        self.h = B.dllm_create(dims_of(cfg, max_batch))
        for l in range(cfg.n_layers):
            w = layers[l] if layers is not None else inputs.layer_weights(cfg, l, self.device, gain_std)
            w = {k: (v.to(self.device).contiguous() if v is not None else None) for k, v in w.items()}
            B.dllm_init_layer(self.h, l, w)
            torch.cuda.current_stream().synchronize()
            del w
        hw = head if head is not None else inputs.head_weights(cfg, self.device, gain_std)
        hw = {k: v.to(self.device).contiguous() for k, v in hw.items()}
        B.dllm_init_head(self.h, hw["embed"], hw["final_norm"], hw["lm_head"])
        torch.cuda.current_stream().synchronize()

    def close(self):
        if self.h:
            B.dllm_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def first_block(committed: torch.Tensor, block_len: int) -> torch.Tensor:
    """First row of the first block that still holds a masked row, per sequence."""
    c = committed.to("cpu", torch.bool)
    Bn, L = c.shape
    out = torch.empty(Bn, dtype=torch.int32)
    for b in range(Bn):
        bs = 0
        while bs < L and bool(c[b, bs:bs + block_len].all()):
            bs += block_len
        out[b] = bs
    return out


class State:
    """Caller-owned decode state on the device."""

    def __init__(self, cfg: Config, batch: Optional[int] = None, device="cuda", tokens=None, committed=None):
        self.cfg = cfg
        dev = torch.device(device)
        Bn = batch or cfg.batch
        N, L, d, r = cfg.n_layers, cfg.seq_len, cfg.d_model, cfg.proxy_rank
        dt = inputs.storage_dtype(cfg)
        self.hidden = torch.zeros((N + 1, Bn, L, d), dtype=dt, device=dev)
        # keys in matrix-core fragment order, values row-major (include/libdllm.h)
        L32 = (L + 31) // 32 * 32
        dh = cfg.head_dim
        self.k_cache = torch.zeros((N, Bn, cfg.n_kv_heads, L32 // 32, dh // 16, 64, 8), dtype=dt, device=dev)
        self.v_cache = torch.zeros((N, Bn, cfg.n_kv_heads, L32, dh), dtype=dt, device=dev)
        self.proxy_cur = torch.zeros((N, Bn, L, r), dtype=torch.float64, device=dev)
        self.proxy_ref = torch.zeros_like(self.proxy_cur)
        self.score = torch.zeros((N, Bn, L), dtype=torch.float64, device=dev)
        if tokens is None:
            tokens, committed = inputs.prompt_tokens(cfg.with_(batch=Bn))
        self.tokens = tokens.to(dev, torch.int32).contiguous()
        self.committed = committed.to(dev, torch.uint8).contiguous()
        self.history = torch.full((Bn, L), -1, dtype=torch.int32, device=dev)
        self.n_history = torch.zeros(Bn, dtype=torch.int32, device=dev)
        self.n_new = torch.zeros(Bn, dtype=torch.int32, device=dev)
        self.block_start = first_block(self.committed, cfg.block_len).to(dev)
        self.full_next = torch.ones(Bn, dtype=torch.uint8, device=dev)
        self.max_entropy = torch.zeros(Bn, dtype=torch.float64, device=dev)
        self.batch = Bn
        self.c = B.DllmState(*[t.data_ptr() for t in (
            self.hidden, self.k_cache, self.v_cache, self.proxy_cur, self.proxy_ref, self.score, self.tokens,
            self.committed, self.history, self.n_history, self.n_new, self.block_start, self.full_next,
            self.max_entropy)], Bn)

    def tensors(self) -> Dict[str, torch.Tensor]:
        return {k: getattr(self, k) for k in (
            "hidden", "k_cache", "v_cache", "proxy_cur", "proxy_ref", "score", "tokens", "committed",
            "history", "n_history", "n_new", "block_start", "full_next", "max_entropy")}


def polestar_params(cfg: Config) -> B.DllmPolestarParams:
    return B.DllmPolestarParams(cfg.n_clusters, cfg.kmeans_iters, cfg.top_clusters, cfg.window_blocks,
                                1 if cfg.polestar_commit else 0, float(cfg.commit_alpha), cfg.tau_upd,
                                cfg.full_period)


class PolestarState:
    """Caller-owned Polestar state (include/libdllm.h, dllm_polestar_state)."""

    def __init__(self, cfg: Config, batch: Optional[int] = None, device="cuda"):
        dev = torch.device(device)
        Bn = batch or cfg.batch
        N, d, K, Hq = cfg.n_layers, cfg.d_model, cfg.n_clusters, cfg.n_q_heads
        W = cfg.window_blocks * cfg.block_len
        self.W = W
        self.log_attn = torch.zeros((N, Bn, K, Hq, W), dtype=torch.float64, device=dev)
        self.win_start = torch.full((N, Bn), -1, dtype=torch.int32, device=dev)
        self.centroids = torch.zeros((Bn, K, d), dtype=torch.float64, device=dev)
        self.norms = torch.zeros((Bn, W), dtype=torch.float64, device=dev)
        self.assign = torch.zeros((Bn, W), dtype=torch.int32, device=dev)
        self.codes = torch.zeros((Bn, W, d // 2), dtype=torch.uint8, device=dev)
        self.scales = torch.zeros((Bn, W, d // 16), dtype=torch.uint8, device=dev)
        self.queries = torch.zeros((Bn, K, cfg.n_q), dtype=inputs.storage_dtype(cfg), device=dev)
        self.kl = torch.zeros((Bn, K), dtype=torch.float64, device=dev)
        self.top = torch.zeros((Bn, cfg.top_clusters), dtype=torch.int32, device=dev)
        self.drift_sum = torch.zeros((Bn, cfg.block_len), dtype=torch.float64, device=dev)
        self.drift_cnt = torch.zeros((Bn, cfg.block_len), dtype=torch.int32, device=dev)
        self.drift_valid = torch.zeros(Bn, dtype=torch.int32, device=dev)
        self.upd_hist = torch.zeros((N, Bn), dtype=torch.int32, device=dev)
        self.c = B.DllmPolestarState(*[t.data_ptr() for t in (
            self.log_attn, self.win_start, self.centroids, self.norms, self.assign, self.codes, self.scales,
            self.queries, self.kl, self.top, self.drift_sum, self.drift_cnt, self.drift_valid, self.upd_hist)], 0)


def ce_params(cfg: Config) -> B.DllmCEParams:
    return B.DllmCEParams(cfg.ce_horizon, cfg.ce_q, cfg.ce_r, cfg.ce_p_v0, cfg.ce_kappa, cfg.ce_gamma)


class CEState:
    """Caller-owned Confidence Extrapolation state (include/libdllm.h, dllm_ce_state)."""

    def __init__(self, cfg: Config, batch: Optional[int] = None, device="cuda"):
        Bn = batch or cfg.batch
        self.kf = torch.zeros((Bn, cfg.block_len, 5), dtype=torch.float64, device=device)
        self.has = torch.zeros((Bn, cfg.block_len), dtype=torch.int32, device=device)
        self.c = B.DllmCEState(self.kf.data_ptr(), self.has.data_ptr())


def step(model: Model, state: State, mode: int = B.DLLM_MODE_AUTO, want_result: bool = True, stream=None,
         tau: Optional[float] = None, polestar_state: Optional[PolestarState] = None,
         ce_state: Optional[CEState] = None, sets_out=None, n_sets_out=None):
    """One dllm_step; a config with ce_horizon > 0 commits with Confidence
    Extrapolation and needs a CEState.  sets_out/n_sets_out (optional int32
    device tensors [N][B][L] / [N][B]) receive every layer's index set."""
    cfg = model.cfg
    ce = None
    if cfg.ce_horizon > 0:
        if ce_state is None:
            raise ValueError("Confidence Extrapolation needs a CEState")
        ce = ce_params(cfg)
    if cfg.score == SCORE_POLESTAR:
        if polestar_state is None:
            raise ValueError("the Polestar score needs a PolestarState")
        return B.dllm_step(model.h, state, mode, FORCED_RULE[cfg.forced], cfg.recent_k,
                           cfg.tau if tau is None else tau, cfg.conf_threshold, cfg.rho, want_result, stream,
                           B.DLLM_SCORE_POLESTAR_KL, polestar_params(cfg), polestar_state, ce, ce_state,
                           sets_out, n_sets_out)
    return B.dllm_step(model.h, state, mode, FORCED_RULE[cfg.forced], cfg.recent_k,
                       cfg.tau if tau is None else tau, cfg.conf_threshold, cfg.rho, want_result, stream,
                       ce=ce, ce_state=ce_state, sets_out=sets_out, n_sets_out=n_sets_out)
