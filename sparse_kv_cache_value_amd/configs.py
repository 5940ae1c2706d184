"""Workload configurations (shapes, seeds and decoding hyper-parameters).

Shapes follow the dLLMs the pages evaluate on (LLaDA-8B and Dream-7B); the
caching hyper-parameters follow each page:

* SPA-Cache ("Singular Proxy for Adaptive Caching in Diffusion Language
  Models", sections 1-3): value-proxy rank ``r`` and the per-layer update ratio
  rho(l), a piecewise Gaussian that is low for early and late layers and peaks
  at mid depth (section 2).  The ablation there reports a mean update ratio of
  16% with r = 128.
* EntropyCache (section 2, "procedure"): full pass next step when the maximum
  entropy of the tokens decoded this step exceeds tau; otherwise refresh the
  current mask block plus the k most recently decoded tokens.
* Polestar (section 2A): local window of prefix/current/suffix blocks,
  spherical k-means of the window, top drift clusters.

rho(l) is given here as a literal table (an input to both the library and the
oracle).  It was produced from the split-Gaussian reading
``rho(l) = 0.04 + (rho_pk - 0.04) * exp(-(l - mu)^2 / (2 sigma^2))`` with
``mu = (N-1)/2``, ``sigma = N/4`` below ``mu`` and ``N/6`` above it, and
``rho_pk`` solved so that the mean ratio is 0.16; the oracle re-derives it from
that formula in a test.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

# rho(l) for a 32-layer model (mean 0.16).
RHO_SPLIT_GAUSSIAN_32 = (
    0.07619438012868328, 0.08575398362567002, 0.09694175263254699,
    0.10976649371057867, 0.1241544551097386, 0.13993588813323293,
    0.1568368902508947, 0.1744784363584371, 0.19238403213040867,
    0.20999667222574084, 0.22670481900731126, 0.24187604324001516,
    0.2548959294172583, 0.26520900039928813, 0.2723579014714283,
    0.2760170059916142, 0.27544149541150276, 0.26730806352130165,
    0.2518744125416231, 0.23066633352543986, 0.20565378128933506,
    0.17895063212353987, 0.1525256511038249, 0.1279780591426117,
    0.10640932314697438, 0.0883966794742886, 0.07405131683670138,
    0.0631304505588074, 0.055169319824389745, 0.04960461493602131,
    0.04587118334470474, 0.04346499938608556,
)

FP32 = "fp32"
BF16 = "bf16"

# forced-set rules
FORCED_NONE = "none"            # pure SPA-Cache: drift alone picks rows
FORCED_BLOCK_RECENT = "block+recent"  # EntropyCache: mask block + recent k decoded
FORCED_BLOCK = "block"          # Polestar: the current block

# drift scores
SCORE_SPA = "spa_cos"
SCORE_POLESTAR = "polestar_kl"


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    batch: int
    seq_len: int
    prompt_len: int
    block_len: int
    proxy_rank: int
    dtype: str
    rho: Tuple[float, ...]          # per layer
    forced: str = FORCED_NONE
    recent_k: int = 0
    tau: float = float("inf")       # entropy gate threshold (nats); inf = never full
    conf_threshold: float = 0.9
    n_steps: int = 8
    score: str = SCORE_SPA
    weight_std: float = 0.02
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    # Polestar
    window_blocks: int = 3
    n_clusters: int = 16
    kmeans_iters: int = 10
    top_clusters: int = 4
    tau_upd: int = 0                # drift refresh every this many decoded tokens (0: every step)
    full_period: int = 0            # AUTO mode: a full pass every this many steps (0: never)
    polestar_commit: bool = False   # Polestar-Commit (Polestar section 2B) instead of the threshold commit
    commit_alpha: float = 1.0
    # Confidence Extrapolation (TSPD + CE section 2) on the threshold commit; horizon 0 = off
    ce_horizon: int = 0
    ce_q: float = 1e-4
    ce_r: float = 1e-3
    ce_p_v0: float = 1e-2
    ce_kappa: float = 2.0
    ce_gamma: float = 0.5
    # C2-style stale cache
    stale_frac: float = 0.0
    stale_std: float = 0.0

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def n_v(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_q(self) -> int:
        return self.n_q_heads * self.head_dim

    def k_layer(self, layer: int) -> int:
        """Rows refreshed at ``layer`` before the forced set is merged."""
        import math

        return int(math.floor(self.rho[layer] * self.seq_len + 0.5))

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def weight_bytes_per_layer(self) -> int:
        d, f = self.d_model, self.d_ffn
        n = d * (self.n_q + 2 * self.n_v) + self.n_q * d + 3 * d * f
        return n * (4 if self.dtype == FP32 else 2)


def _uniform(n_layers: int, rho: float):
    return tuple([rho] * n_layers)


# Tiny fp32 model: 2 layers, d=256, 4 heads x 64, SwiGLU 1024, vocab 1024,
# L = 64 prompt + 64 masked, block 32, 8 steps, r = 16, k = 16 rows per layer.
C1 = Config(
    name="tiny-fp32", seed=0, n_layers=2, d_model=256, n_q_heads=4,
    n_kv_heads=4, head_dim=64, d_ffn=1024, vocab=1024, batch=1, seq_len=128,
    prompt_len=64, block_len=32, proxy_rank=16, dtype=FP32,
    rho=_uniform(2, 16 / 128), n_steps=8,
)

# One LLaDA-8B-shaped layer with a stale cache on 30% of rows; k = 82 (16%).
C2 = Config(
    name="llada8b-1layer", seed=1, n_layers=1, d_model=4096, n_q_heads=32,
    n_kv_heads=32, head_dim=128, d_ffn=12288, vocab=126464, batch=1,
    seq_len=512, prompt_len=256, block_len=32, proxy_rank=128, dtype=BF16,
    rho=_uniform(1, 82 / 512), n_steps=1, stale_frac=0.3, stale_std=0.05,
)

# Full 32-layer LLaDA-8B shape, L = 1024, split-Gaussian rho(l), EntropyCache gate.
C3 = Config(
    name="llada8b-32l-L1024", seed=2, n_layers=32, d_model=4096, n_q_heads=32,
    n_kv_heads=32, head_dim=128, d_ffn=12288, vocab=126464, batch=1,
    seq_len=1024, prompt_len=512, block_len=32, proxy_rank=128, dtype=BF16,
    rho=RHO_SPLIT_GAUSSIAN_32, forced=FORCED_BLOCK_RECENT, recent_k=32,
    tau=2.0, n_steps=512,
)

# Dream-7B shape (GQA 28/4), batch 8, L = 2048, uniform 16% refresh.
C4 = Config(
    name="dream7b-28l-B8-L2048", seed=3, n_layers=28, d_model=3584,
    n_q_heads=28, n_kv_heads=4, head_dim=128, d_ffn=18944, vocab=152064,
    batch=8, seq_len=2048, prompt_len=1024, block_len=32, proxy_rank=128,
    dtype=BF16, rho=_uniform(28, 328 / 2048), forced=FORCED_BLOCK_RECENT,
    recent_k=32, n_steps=1024,
)

# Polestar drift path on the LLaDA-8B layer shape, batch 4, L = 4096.
C5 = Config(
    name="llada8b-polestar-B4-L4096", seed=4, n_layers=32, d_model=4096,
    n_q_heads=32, n_kv_heads=32, head_dim=128, d_ffn=12288, vocab=126464,
    batch=4, seq_len=4096, prompt_len=2048, block_len=32, proxy_rank=128,
    dtype=BF16, rho=_uniform(32, 0.0), forced=FORCED_BLOCK,
    score=SCORE_POLESTAR, n_steps=2048,
)

ALL = {c.name: c for c in (C1, C2, C3, C4, C5)}


def scaled(cfg: Config, **kw) -> Config:
    """A smaller variant of ``cfg`` for tests (same structure, fewer rows/layers)."""
    return cfg.with_(**kw)
