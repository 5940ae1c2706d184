"""LM-head row statistics (EntropyCache section 2: the O(V) decision) without
a logits buffer: for up to 288 rows the weight-streaming GEMM reduces each
128-column vocabulary slab to (max, lowest argmax, S, T) in its epilogue and
one kernel merges the slabs in a fixed order.  Against the logits of the same
GEMM (dllm_lm_head with logits requested) reduced on the host in fp64: the
max and argmax equal bit for bit, S and T to 1e-12 relative; and against the
oracle's statistics of the same hidden rows.  LLaDA-8B vocabulary (126464)
and a small one; 32 to 288 rows (one to nine row tiles, 64 rows per pass of
the epilogue)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_common import build, medium_cfg, say
from helpers import spec_of
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, runtime

pytestmark = pytest.mark.gpu


def _host_stats(z):
    z = z.astype(np.float64)
    m = z.max(axis=1)
    am = np.argmax(z, axis=1)
    e = np.exp(z - m[:, None])
    return m, am, e.sum(axis=1), (e * (z - m[:, None])).sum(axis=1)


@pytest.mark.parametrize("cfg", [medium_cfg(name="lm-medium", n_layers=1, batch=2),
                                 medium_cfg(name="lm-medium-b3", n_layers=1, batch=3),
                                 medium_cfg(name="lm-medium-b9", n_layers=1, batch=9),
                                 configs.C2.with_(n_layers=1),
                                 configs.C2.with_(name="lm-llada8b-b4", n_layers=1, batch=4)],
                         ids=lambda c: c.name)
def test_fused_lm_head_statistics(cfg):
    spec = spec_of(cfg)
    model, _, head = build(cfg)
    st = runtime.State(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    Bn, blk, V = st.batch, cfg.block_len, cfg.vocab
    fused = torch.zeros((Bn, blk, 4), dtype=torch.float64, device="cuda")
    plain = torch.zeros_like(fused)
    logits = torch.zeros((Bn, blk, V), dtype=torch.float32, device="cuda")
    B.dllm_lm_head(model.h, st, fused)
    B.dllm_lm_head(model.h, st, plain, logits)
    torch.cuda.synchronize()
    f = fused.cpu().numpy().reshape(-1, 4)
    z = logits.cpu().numpy().reshape(-1, V)
    m, am, S, T = _host_stats(z)
    assert np.array_equal(f[:, 0], m), "max"
    assert np.array_equal(f[:, 1].astype(np.int64), am), "argmax"
    assert np.max(np.abs(f[:, 2] / S - 1)) <= 1e-12, "S"
    assert np.max(np.abs(f[:, 3] - T) / np.abs(T)) <= 1e-12, "T"
    p = plain.cpu().numpy().reshape(-1, 4)
    assert np.array_equal(p[:, :2], f[:, :2])
    # the oracle on the same final hidden rows
    H = st.hidden[cfg.n_layers].float().cpu().numpy()
    bs = st.block_start.cpu().numpy()
    for b in range(Bn):
        rows = np.arange(bs[b], bs[b] + blk)
        so = oracle.lm_stats(H[b][rows], head["final_norm"], head["lm_head"], spec)
        fb = fused.cpu().numpy()[b]
        assert np.max(np.abs(fb[:, 0] - so["m"])) <= 1e-5 * np.max(np.abs(so["logits"]))
        assert np.max(np.abs(fb[:, 2] / so["S"] - 1)) <= 1e-5
        ent = np.log(fb[:, 2]) - fb[:, 3] / fb[:, 2]
        assert np.max(np.abs(ent - so["entropy"])) <= 1e-5
    say(f"{cfg.name}: {Bn * blk} rows x {V}: fused statistics match the logits and the oracle")
    model.close()
