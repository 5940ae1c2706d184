"""Helpers for the GPU parity tests: models with host copies of their weights,
state snapshots in the oracle's layout, and the comparison rules (float
tolerance, selection tie bands)."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from helpers import np_weights, spec_of
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, inputs, runtime

TOL = {configs.FP32: 1e-4, configs.BF16: 2e-2}


def say(*a):
    print(*a, flush=True)


def build(cfg, gain_std=0.1):
    """Model on the GPU plus host (numpy fp32) copies of the same weights."""
    layers = [inputs.layer_weights(cfg, l, "cuda", gain_std) for l in range(cfg.n_layers)]
    head = inputs.head_weights(cfg, "cuda", gain_std)
    model = runtime.Model(cfg, "cuda", layers=layers, head=head)
    layers_np = [np_weights(w) for w in layers]
    head_np = np_weights(head)
    del layers, head
    torch.cuda.empty_cache()
    return model, layers_np, head_np


def unpack_k(k):
    """[N][B][G][L32/32][dh/16][64][8] fragment order -> [N, B, L32, G, dh]."""
    N_, B_, G_, T_, KS, _, _ = k.shape
    k = k.reshape(N_, B_, G_, T_, KS, 2, 32, 8)            # lane = key%32 + 32*((dim/8)%2)
    k = k.permute(0, 1, 3, 6, 2, 4, 5, 7)                  # N B T key G KS half j
    return k.reshape(N_, B_, T_ * 32, G_, KS * 16).numpy()


def unpack_v(v):
    """[N][B][G][L32][dh] row-major values -> [N, B, L32, G, dh]."""
    return v.permute(0, 1, 3, 2, 4).numpy()


class Snap:
    """Host copy of a State, in the oracle's per-sequence layout."""

    def __init__(self, st: runtime.State):
        torch.cuda.synchronize()
        t = {k: v.detach().cpu() for k, v in st.tensors().items()}
        self.H = t["hidden"].float().numpy()                                 # [N+1, B, L, d]
        L = self.H.shape[2]
        self.K = unpack_k(t["k_cache"].float())[:, :, :L]                      # [N, B, L, Hkv, dh]
        self.V = unpack_v(t["v_cache"].float())[:, :, :L]
        self.Pc = t["proxy_cur"].numpy()
        self.Pr = t["proxy_ref"].numpy()
        self.score = t["score"].numpy()
        self.tokens = t["tokens"].numpy().astype(np.int64)
        self.committed = t["committed"].numpy().astype(bool)
        self.history = t["history"].numpy()
        self.n_history = t["n_history"].numpy()
        self.n_new = t["n_new"].numpy()
        self.block_start = t["block_start"].numpy()
        self.full_next = t["full_next"].numpy()
        self.max_entropy = t["max_entropy"].numpy()


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0)) if b.size else 0.0


def assert_close(a, b, tol, what=""):
    e = rel(a, b)
    assert e <= tol, f"{what}: rel err {e:.3e} > {tol:.1e}"
    return e


def selection_band(s, forced, I_ref, k):
    """Rows excluded from exact comparison: non-forced rows whose score is
    within 1e-6 (relative) of the reference's last drift-picked score."""
    s = np.asarray(s, np.float64)
    forced = np.zeros(len(s), bool) if forced is None else np.asarray(forced, bool)
    picked = [i for i in I_ref if not forced[i]]
    if not picked:
        return set()
    last = min(s[i] for i in picked)
    if last == 0.0:
        return set()
    return {i for i in range(len(s)) if not forced[i] and abs(s[i] - last) <= 1e-6 * last}


def assert_same_selection(I_gpu, I_ref, s_ref, forced, k, what=""):
    I_gpu = [int(i) for i in I_gpu]
    I_ref = [int(i) for i in I_ref]
    assert len(I_gpu) == len(I_ref), f"{what}: |I| gpu {len(I_gpu)} vs oracle {len(I_ref)}"
    assert I_gpu == sorted(I_gpu), f"{what}: gpu indices not ascending"
    band = selection_band(s_ref, forced, I_ref, k)
    a = set(I_gpu) - band
    b = set(I_ref) - band
    assert a == b, f"{what}: selections differ outside the tie band: gpu-only {sorted(a - b)[:10]} oracle-only {sorted(b - a)[:10]}"
    return len(band)


# LM-head statistics are checked to 1e-5 of max|z| (logits accumulate in fp32
# on the device, fp64 in the oracle); a commit decision closer than that to
# flipping is left undecided
COMMIT_BAND = 1e-5


def commit_band(stats, masked, thr, rel=COMMIT_BAND):
    """Rows whose commit decision the float tolerance cannot decide: top-2 logit
    gap within rel*max|z|, confidence within rel of the threshold, or (masked:
    bool per row, the rows still masked) a most-confident fallback whose
    runner-up confidence is within rel of it."""
    z = stats["logits"]
    conf = np.asarray(stats["conf"], np.float64)
    out = set()
    for j in range(z.shape[0]):
        zz = np.sort(z[j])[-2:]
        scale = max(np.max(np.abs(z[j])), 1e-30)
        if zz[1] - zz[0] <= rel * scale:
            out.add(j)
        if abs(conf[j] - thr) <= rel * max(thr, 1e-30):
            out.add(j)
    if masked is not None:
        cand = [j for j in range(z.shape[0]) if masked[j]]
        if cand and not any(conf[j] >= thr for j in cand):
            best = max(conf[j] for j in cand)
            close = [j for j in cand if best - conf[j] <= rel * best]
            if len(close) > 1:
                out.update(close)
    return out


def assert_states_equal(a, b, what="", skip=()):
    """Two States hold bit-identical buffers (except those named in skip)."""
    torch.cuda.synchronize()
    for k, v in a.tensors().items():
        if k not in skip:
            assert torch.equal(v, getattr(b, k)), f"{what}: {k} differs"


def mode_of(full: bool) -> int:
    return B.DLLM_MODE_FULL if full else B.DLLM_MODE_SPARSE


def medium_cfg(**kw):
    """A small bf16 model: several MFMA tiles, ragged row counts, two layers."""
    base = dict(name="medium-bf16", seed=21, n_layers=2, d_model=512, n_q_heads=4, n_kv_heads=4,
                head_dim=128, d_ffn=1536, vocab=4096, batch=1, seq_len=160, prompt_len=96, block_len=32,
                proxy_rank=32, dtype=configs.BF16, rho=(0.16, 0.2), forced=configs.FORCED_BLOCK_RECENT,
                recent_k=8, tau=2.0, n_steps=4)
    base.update(kw)
    return configs.Config(**base)
