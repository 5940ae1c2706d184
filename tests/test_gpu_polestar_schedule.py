"""Polestar refresh schedule (Polestar page, section 2A, schedule) on the
GPU: with tau_upd = 3 a layer's drift refresh runs on a window's first step
and then once three tokens were decoded since its last one; between refreshes
the index set is the current block alone and the stored proxy attention,
window start and refresh counter stay untouched.  The refresh decision is
checked against the oracle's rule on the GPU's own state at every layer, and
on refresh steps the index set against the oracle's selection on the GPU's
assignment and drift.  With full_period = 3 in AUTO mode every third step is
a full pass of every sequence, and an explicit SPARSE mode overrides it."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import polestar as ps
from gpu_common import build, medium_cfg, say
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, runtime

pytestmark = pytest.mark.gpu

SCHED = medium_cfg(name="medium-polestar-schedule", score=configs.SCORE_POLESTAR, forced=configs.FORCED_BLOCK,
                   recent_k=0, seed=33, batch=2, tau_upd=3, tau=float("inf"), n_steps=8)


def test_refresh_every_tau_upd_tokens():
    cfg = SCHED
    model, _, _ = build(cfg)
    st, pst = runtime.State(cfg), runtime.PolestarState(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL, polestar_state=pst)
    params = runtime.polestar_params(cfg)
    pp = ps.PolestarParams(cfg.n_clusters, cfg.kmeans_iters, cfg.top_clusters, cfg.window_blocks,
                           tau_upd=cfg.tau_upd)
    Bn, L, N, blk = cfg.batch, cfg.seq_len, cfg.n_layers, cfg.block_len
    idx = torch.zeros((Bn, L), dtype=torch.int32, device="cuda")
    n = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    pattern = []
    for t in range(cfg.n_steps):
        nh = st.n_history.cpu().numpy()
        nn = st.n_new.cpu().numpy()
        hist = st.history.cpu().numpy()
        rows0 = torch.zeros((Bn, L), dtype=torch.int32)
        n0 = torch.zeros(Bn, dtype=torch.int32)
        for b in range(Bn):
            rows0[b, :nn[b]] = torch.from_numpy(hist[b][nh[b] - nn[b]:nh[b]].copy())
            n0[b] = int(nn[b])
        B.dllm_embed(model.h, st, rows0.cuda(), n0.cuda())
        bs = st.block_start.cpu().numpy()
        for l in range(N):
            torch.cuda.synchronize()
            w0 = pst.win_start[l].cpu().numpy().copy()
            u0 = pst.upd_hist[l].cpu().numpy().copy()
            la0 = pst.log_attn[l].clone()
            B.dllm_polestar_drift(model.h, l, st, pst, params)
            B.dllm_polestar_select(model.h, l, st, pst, params, idx, n)
            torch.cuda.synchronize()
            I_all, n_all = idx.cpu().numpy(), n.cpu().numpy()
            kl, assign, top = pst.kl.cpu().numpy(), pst.assign.cpu().numpy(), pst.top.cpu().numpy()
            for b in range(Bn):
                ws = ps.window_start(int(bs[b]), L, blk, cfg.window_blocks)
                prev = ps.PolestarLayerState(logA=None if w0[b] < 0 else np.zeros(1), wstart=int(w0[b]),
                                             hist_at_update=int(u0[b]))
                due = ps.refresh_due(prev, ws, int(nh[b]), pp)
                I = list(I_all[b][:n_all[b]])
                block = list(range(int(bs[b]), min(int(bs[b]) + blk, L)))
                if due:
                    assert int(pst.win_start[l, b]) == ws and int(pst.upd_hist[l, b]) == int(nh[b])
                    want = ps.select_rows(np.array(block), ws, assign[b], top[b]).tolist()
                    assert I == want, f"t={t} l={l} b={b}: refresh index set"
                    assert list(top[b]) == list(ps.top_clusters(kl[b], cfg.top_clusters))
                else:
                    assert I == block, f"t={t} l={l} b={b}: without a refresh I must be the block"
                    assert int(pst.win_start[l, b]) == w0[b] and int(pst.upd_hist[l, b]) == u0[b]
                    assert torch.equal(pst.log_attn[l, b], la0[b]), f"t={t} l={l} b={b}: attention replaced"
                    assert np.all(kl[b] == 0.0) and int(pst.drift_valid[b]) == 0
                if l == 0:
                    pattern.append((t, b, due))
            B.dllm_sparse_layer(model.h, l, st, idx, n, Bn * pst.W)
        B.dllm_commit(model.h, st, cfg.conf_threshold, cfg.tau)
    say(f"refresh pattern (step, seq, due): {pattern}")
    dues = [d for (_, _, d) in pattern]
    assert any(dues) and not all(dues), "the schedule should both refresh and skip"
    model.close()


def test_periodic_full_pass():
    cfg = SCHED.with_(name="medium-polestar-full-period", tau_upd=0, full_period=3)
    model, _, _ = build(cfg)
    st, pst = runtime.State(cfg), runtime.PolestarState(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL, polestar_state=pst)
    modes = []
    for t in range(7):
        res = runtime.step(model, st, mode=B.DLLM_MODE_AUTO, polestar_state=pst)
        modes.append("F" if res.n_full == cfg.batch else ("S" if res.n_full == 0 else "?"))
    say(f"AUTO modes after the first full pass: {''.join(modes)}")
    assert "".join(modes) == "SSFSSFS"
    # an explicit SPARSE mode is not overridden, and still counts
    res = runtime.step(model, st, mode=B.DLLM_MODE_SPARSE, polestar_state=pst)
    assert res.n_full == 0
    res = runtime.step(model, st, mode=B.DLLM_MODE_AUTO, polestar_state=pst)
    assert res.n_full == cfg.batch
    model.close()
