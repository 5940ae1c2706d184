"""GPU parity: each entry point of the C-ABI against the oracle, layer by layer
(shadow mode: at every decision point the oracle's decision functions run on
the GPU's own inputs), for a full pass followed by sparse steps."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (TOL, Snap, assert_close, assert_same_selection, build, commit_band, medium_cfg, say)
from helpers import spec_of
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, runtime

pytestmark = pytest.mark.gpu

CFGS = {
    "c1-fp32": configs.C1.with_(n_steps=3),
    "medium-bf16": medium_cfg(),
    "medium-gqa": medium_cfg(name="medium-gqa", n_q_heads=8, n_kv_heads=2, head_dim=128, seed=22),
    "medium-dh64": medium_cfg(name="medium-dh64", n_q_heads=8, n_kv_heads=8, head_dim=64, seed=25, n_steps=2),
    "medium-l100": medium_cfg(name="medium-l100", seq_len=100, prompt_len=50, seed=26, n_steps=2),
    "medium-b2": medium_cfg(name="medium-b2", batch=2, seq_len=96, prompt_len=40, seed=23, n_steps=3),
    "medium-none": medium_cfg(name="medium-none", forced=configs.FORCED_NONE, recent_k=0, seed=24, n_steps=3),
}


def _forced_np(cfg, snap, b):
    L, blk = cfg.seq_len, cfg.block_len
    f = np.zeros(L, bool)
    if cfg.forced in (configs.FORCED_BLOCK, configs.FORCED_BLOCK_RECENT):
        bs = snap.block_start[b]
        f[bs:min(bs + blk, L)] = True
    if cfg.forced == configs.FORCED_BLOCK_RECENT:
        nh = snap.n_history[b]
        f[snap.history[b][max(0, nh - cfg.recent_k):nh]] = True
    return f


def _check_commit(cfg, spec, head, before, after, what):
    thr = cfg.conf_threshold
    for b in range(cfg.batch):
        bs = before.block_start[b]
        rows = np.arange(bs, min(bs + cfg.block_len, cfg.seq_len))
        if rows.size == 0:
            assert after.n_new[b] == 0
            continue
        st = oracle.lm_stats(after.H[cfg.n_layers][b][rows], head["final_norm"], head["lm_head"], spec)
        band = commit_band(st, ~before.committed[b][rows], thr)
        pos, tok, emax = oracle.commit(rows, st["conf"], st["argmax"], st["entropy"], before.committed[b], thr)
        cand_band = {int(rows[j]) for j in band}
        got_pos = [int(p) for p in after.history[b][before.n_history[b]:after.n_history[b]]]
        if cand_band & set(pos + got_pos):
            say(f"{what} b={b}: commit inside the tie band, skipped")
            continue
        assert got_pos == pos, f"{what} b={b}: committed {got_pos} vs oracle {pos}"
        assert [int(after.tokens[b][p]) for p in pos] == tok
        assert after.n_new[b] == len(pos)
        assert all(after.committed[b][p] for p in pos)
        assert abs(after.max_entropy[b] - emax) <= 1e-6 * max(1.0, emax), (after.max_entropy[b], emax)
        assert bool(after.full_next[b]) == (emax > cfg.tau)


def _check_full_pass(cfg, spec, layers, head, before, cur, tol, what):
    for b in range(cfg.batch):
        emb = head["embed"][before.tokens[b]]
        assert np.array_equal(cur.H[0][b], emb), f"{what}: embeddings"
        for l in range(cfg.n_layers):
            x = cur.H[l][b]
            out, K, V = oracle.layer_dense(x, layers[l], spec)
            e = assert_close(cur.H[l + 1][b], out, tol, f"{what} b={b} l={l} H")
            assert_close(cur.K[l][b], K, tol, f"{what} b={b} l={l} K")
            assert_close(cur.V[l][b], V, tol, f"{what} b={b} l={l} V")
            C = oracle.proxy(x, layers[l]["attn_norm"], layers[l]["w_proxy"])
            assert_close(cur.Pr[l][b], C, 1e-12, f"{what} proxy")
            assert np.array_equal(cur.Pr[l][b], cur.Pc[l][b])
            assert np.all(cur.score[l][b] == 0.0)
            say(f"{what} full pass b={b} l={l}: H rel err {e:.2e}")


@pytest.mark.parametrize("name", list(CFGS))
def test_layerwise_parity(name):
    torch.manual_seed(0)
    cfg = CFGS[name]
    say(f"== {name}")
    spec = spec_of(cfg)
    tol = TOL[cfg.dtype]
    model, layers, head = build(cfg)
    st = runtime.State(cfg)
    Bn, L, N = cfg.batch, cfg.seq_len, cfg.n_layers
    rule = runtime.FORCED_RULE[cfg.forced]

    before = Snap(st)
    res = runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    cur = Snap(st)
    assert res.n_full == Bn
    _check_full_pass(cfg, spec, layers, head, before, cur, tol, name)
    _check_commit(cfg, spec, head, before, cur, f"{name} step0")

    # the oracle's proxy at each row's last refresh, from the GPU's inputs
    P_or = [[oracle.proxy(cur.H[l][b], layers[l]["attn_norm"], layers[l]["w_proxy"]) for b in range(Bn)]
            for l in range(N)]
    dev = "cuda"
    idx = torch.zeros((Bn, L), dtype=torch.int32, device=dev)
    n = torch.zeros(Bn, dtype=torch.int32, device=dev)
    forced = torch.zeros((Bn, L), dtype=torch.uint8, device=dev)
    for t in range(1, cfg.n_steps + 1):
        S0 = Snap(st)
        if all(S0.block_start[b] >= L for b in range(Bn)):
            break
        B.dllm_forced_set(model.h, st, rule, cfg.recent_k, forced)
        fr = forced.cpu().numpy().astype(bool)
        for b in range(Bn):
            assert np.array_equal(fr[b], _forced_np(cfg, S0, b)), f"forced set b={b}"
        rows0 = torch.zeros((Bn, L), dtype=torch.int32)
        n0 = torch.zeros(Bn, dtype=torch.int32)
        for b in range(Bn):
            nh, nn = S0.n_history[b], S0.n_new[b]
            rows0[b, :nn] = torch.from_numpy(S0.history[b][nh - nn:nh].copy())
            n0[b] = nn
        prev_idx, prev_n = rows0.to(dev), n0.to(dev)
        B.dllm_embed(model.h, st, prev_idx, prev_n)
        for l in range(N):
            B.dllm_drift_score(model.h, l, st, prev_idx, prev_n)
            Sd = Snap(st)
            k = oracle.budget_k(cfg.rho[l], L)
            B.dllm_select(model.h, l, st, forced, None, cfg.rho[l], idx, n)
            I_all = idx.cpu().numpy()
            n_all = n.cpu().numpy()
            B.dllm_sparse_layer(model.h, l, st, idx, n)
            Sa = Snap(st)
            for b in range(Bn):
                x = Sd.H[l][b]
                C = oracle.proxy(x, layers[l]["attn_norm"], layers[l]["w_proxy"])
                s = oracle.drift(C, P_or[l][b])
                diff = np.abs(Sd.score[l][b] - s)
                assert np.all(diff <= 1e-10 * np.maximum(s, 1e-300) + 1e-15), \
                    f"{name} t={t} l={l} b={b}: drift max diff {diff.max():.3e}"
                I_or = oracle.select(s, fr[b], k)
                I_gpu = I_all[b][:n_all[b]]
                nb = assert_same_selection(I_gpu, I_or, s, fr[b], k, f"{name} t={t} l={l} b={b}")
                Kx, Vx, Hx = Sd.K[l][b].copy(), Sd.V[l][b].copy(), Sd.H[l + 1][b].copy()
                oracle.sparse_layer(x, Kx, Vx, Hx, I_gpu, layers[l], spec)
                mask = np.zeros(L, bool)
                mask[I_gpu] = True
                e = assert_close(Sa.H[l + 1][b][mask], Hx[mask], tol, f"{name} t={t} l={l} H")
                assert np.array_equal(Sa.H[l + 1][b][~mask], Sd.H[l + 1][b][~mask]), "rows outside I changed"
                assert_close(Sa.K[l][b][mask], Kx[mask], tol, "K rows")
                assert_close(Sa.V[l][b][mask], Vx[mask], tol, "V rows")
                assert np.array_equal(Sa.K[l][b][~mask], Sd.K[l][b][~mask])
                assert np.array_equal(Sa.Pr[l][b][mask], Sa.Pc[l][b][mask])
                assert np.all(Sa.score[l][b][mask] == 0.0)
                P_or[l][b][mask] = C[mask]
                say(f"{name} t={t} l={l} b={b}: |I|={len(I_gpu)} band={nb} H rel err {e:.2e}")
            prev_idx, prev_n = idx.clone(), n.clone()
        # LM head statistics against the oracle on the GPU's final hidden rows
        stats = torch.zeros((Bn, cfg.block_len, 4), dtype=torch.float64, device=dev)
        B.dllm_lm_head(model.h, st, stats)
        sg = stats.cpu().numpy()
        Sl = Snap(st)
        for b in range(Bn):
            bs = Sl.block_start[b]
            rows = np.arange(bs, min(bs + cfg.block_len, L))
            if rows.size == 0:
                continue
            so = oracle.lm_stats(Sl.H[N][b][rows], head["final_norm"], head["lm_head"], spec)
            band = commit_band(so, ~Sl.committed[b][rows], cfg.conf_threshold)
            nr = rows.size
            assert np.max(np.abs(sg[b, :nr, 0] - so["m"])) <= 1e-5 * np.max(np.abs(so["logits"]))
            assert np.max(np.abs(sg[b, :nr, 2] / so["S"] - 1)) <= 1e-5
            ent = np.log(sg[b, :nr, 2]) - sg[b, :nr, 3] / sg[b, :nr, 2]
            assert np.max(np.abs(ent - so["entropy"])) <= 1e-5
            for j in range(nr):
                if j not in band:
                    assert int(sg[b, j, 1]) == so["argmax"][j], f"argmax row {j}"
        B.dllm_commit(model.h, st, cfg.conf_threshold, cfg.tau)
        _check_commit(cfg, spec, head, S0, Snap(st), f"{name} t={t}")
    model.close()


@pytest.mark.parametrize("name", ["medium-bf16", "c1-fp32", "medium-b2"])
def test_step_equals_entry_point_composition(name):
    """dllm_step is bit-for-bit the composition of the per-function entry points."""
    cfg = CFGS[name]
    say(f"== step composition {name}")
    model, layers, head = build(cfg)
    Bn, L, N = cfg.batch, cfg.seq_len, cfg.n_layers
    rule = runtime.FORCED_RULE[cfg.forced]
    fmax = {configs.FORCED_NONE: 0, configs.FORCED_BLOCK: cfg.block_len,
            configs.FORCED_BLOCK_RECENT: cfg.block_len + cfg.recent_k}[cfg.forced]
    a = runtime.State(cfg)
    runtime.step(model, a, mode=B.DLLM_MODE_FULL)
    b_ = runtime.State(cfg)
    for k, v in a.tensors().items():
        getattr(b_, k).copy_(v)
    dev = "cuda"
    idx = [torch.zeros((Bn, L), dtype=torch.int32, device=dev) for _ in range(2)]
    n = [torch.zeros(Bn, dtype=torch.int32, device=dev) for _ in range(2)]
    forced = torch.zeros((Bn, L), dtype=torch.uint8, device=dev)
    for t in range(2):
        runtime.step(model, a, mode=B.DLLM_MODE_SPARSE)
        S0 = Snap(b_)
        B.dllm_forced_set(model.h, b_, rule, cfg.recent_k, forced)
        rows0 = torch.zeros((Bn, L), dtype=torch.int32)
        n0 = torch.zeros(Bn, dtype=torch.int32)
        for bb in range(Bn):
            nh, nn = S0.n_history[bb], S0.n_new[bb]
            rows0[bb, :nn] = torch.from_numpy(S0.history[bb][nh - nn:nh].copy())
            n0[bb] = nn
        pi, pn, pmax = rows0.to(dev), n0.to(dev), Bn * min(L, cfg.block_len)
        B.dllm_embed(model.h, b_, pi, pn)
        for l in range(N):
            B.dllm_drift_score(model.h, l, b_, pi, pn, pmax)
            k = oracle.budget_k(cfg.rho[l], L)
            B.dllm_select(model.h, l, b_, forced, None, cfg.rho[l], idx[l & 1], n[l & 1])
            rmax = Bn * min(L, max(k, fmax))
            B.dllm_sparse_layer(model.h, l, b_, idx[l & 1], n[l & 1], rmax)
            pi, pn, pmax = idx[l & 1], n[l & 1], rmax
        B.dllm_commit(model.h, b_, cfg.conf_threshold, cfg.tau)
        torch.cuda.synchronize()
        for k2, v in a.tensors().items():
            assert torch.equal(v, getattr(b_, k2)), f"t={t}: {k2} differs"
    model.close()


def test_determinism():
    """Two runs of the same steps give bit-identical states."""
    cfg = CFGS["medium-bf16"]
    model, _, _ = build(cfg)
    outs = []
    for _ in range(2):
        s = runtime.State(cfg)
        runtime.step(model, s, mode=B.DLLM_MODE_FULL)
        for _ in range(3):
            runtime.step(model, s, mode=B.DLLM_MODE_SPARSE)
        torch.cuda.synchronize()
        outs.append({k: v.clone() for k, v in s.tensors().items()})
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k
    model.close()
