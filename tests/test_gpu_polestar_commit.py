"""Polestar-Commit (Polestar page, section 2B) on the GPU against the oracle,
in shadow mode: at every sparse step the oracle's commit decision runs on the
GPU's own last-layer hidden rows (its LM-head statistics are recomputed in
fp64), last-layer cluster drift, assignment and top clusters, and the drift
history the GPU held before the step.  Commits, tokens, entropy gate, block
advance and the updated drift history must agree (decisions inside the
float tie band are skipped and reported).  The config makes every rule fire:
drift commits (small alpha), the most-confident fallback, and suffix-block
commits at the confidence threshold (eight top clusters).  Also: dllm_step with Polestar-Commit is bit-for-bit
the composition of the entry points."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import polestar as ps
from gpu_common import Snap, assert_states_equal, build, commit_band, medium_cfg, say
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, runtime

pytestmark = pytest.mark.gpu

PC = medium_cfg(name="medium-polestar-commit", score=configs.SCORE_POLESTAR, forced=configs.FORCED_BLOCK,
                recent_k=0, seed=31, batch=2, seq_len=224, prompt_len=96, top_clusters=8,
                conf_threshold=0.00125, polestar_commit=True, commit_alpha=1e-5, n_steps=10)
# (test_polestar_commit_decode replaces conf_threshold by a data-derived one)


def _ps_host(pst):
    torch.cuda.synchronize()
    return {k: getattr(pst, k).cpu().numpy().copy() for k in
            ("kl", "assign", "top", "drift_sum", "drift_cnt", "drift_valid", "win_start")}


def _check_step(cfg, spec, head, before, pb, after, pa, counts, what):
    L, blk, N = cfg.seq_len, cfg.block_len, cfg.n_layers
    thr, alpha = cfg.conf_threshold, cfg.commit_alpha
    assert np.all(pa["drift_valid"] == 0), f"{what}: drift_valid not cleared"
    for b in range(cfg.batch):
        bs = int(before.block_start[b])
        if bs >= L:
            assert after.n_new[b] == 0
            continue
        ws = ps.window_start(bs, L, blk, cfg.window_blocks)
        valid = int(pb["win_start"][N - 1, b]) == ws
        assert int(pa["win_start"][N - 1, b]) == ws
        rows = np.arange(bs, min(bs + blk, L))
        srows = np.arange(bs + blk, min(bs + 2 * blk, L))
        n = rows.size
        st = oracle.lm_stats(after.H[N][b][np.concatenate([rows, srows])], head["final_norm"], head["lm_head"],
                             spec)
        cur = {k: st[k][:n] for k in ("conf", "argmax", "entropy")}
        suf = {k: st[k][n:] for k in ("conf", "argmax", "entropy")}
        D = ps.token_drift(rows, ws, pa["assign"][b], pa["kl"][b]) if valid else None
        hit = valid and ps.suffix_hit(bs, blk, ws, pa["assign"][b], pa["top"][b])
        hs, hc = pb["drift_sum"][b][:n], pb["drift_cnt"][b][:n]
        pos, tok, emax, flags = ps.drift_commit(rows, cur, srows, suf, before.committed[b], thr, alpha, D, hs, hc,
                                                hit)
        # rows the float tolerance cannot decide
        both = np.concatenate([rows, srows])
        band = {int(both[j]) for j in commit_band(st, None, thr)}
        band |= {int(rows[j]) for j in commit_band({k: st[k][:n] for k in ('logits', 'conf')}, ~before.committed[b][rows], thr)}
        if D is not None:
            for j in range(n):
                if hc[j] > 0:
                    t = thr - cur["conf"][j]
                    dt = alpha * (t * t)
                    delta = D[j] - hs[j] / hc[j]
                    if abs(delta - dt) <= 1e-5 * abs(dt) + 1e-18:
                        band.add(int(rows[j]))
        got = [int(p) for p in after.history[b][before.n_history[b]:after.n_history[b]]]
        if band & set(pos + got):
            say(f"{what} b={b}: commit inside the tie band, skipped")
            continue
        assert got == pos, f"{what} b={b}: committed {got} vs oracle {pos} (hit={hit}, valid={valid})"
        assert [int(after.tokens[b][p]) for p in pos] == tok
        assert after.n_new[b] == len(pos)
        assert abs(after.max_entropy[b] - emax) <= 1e-6 * max(1.0, emax)
        assert bool(after.full_next[b]) == (emax > cfg.tau)
        # block advance: the oracle's rule on the committed map
        cm = before.committed[b].copy()
        cm[pos] = True
        nbs = bs
        while nbs < L and cm[nbs:nbs + blk].all():
            nbs += blk
        assert int(after.block_start[b]) == nbs, f"{what} b={b}: block start {after.block_start[b]} vs {nbs}"
        # drift history
        if nbs != bs:
            want_s, want_c = np.zeros(blk), np.zeros(blk, np.int64)
        else:
            want_s, want_c = pb["drift_sum"][b].copy(), pb["drift_cnt"][b].astype(np.int64)
            if D is not None:
                want_s[:n] = want_s[:n] + D
                want_c[:n] += 1
        assert np.array_equal(pa["drift_sum"][b], want_s), f"{what} b={b}: drift_sum"
        assert np.array_equal(pa["drift_cnt"][b].astype(np.int64), want_c), f"{what} b={b}: drift_cnt"
        by_drift = [j for j in range(n) if flags[j] and cur["conf"][j] < thr and D is not None and hc[j] > 0
                    and D[j] - hs[j] / hc[j] > alpha * ((thr - cur["conf"][j]) ** 2)]
        nd = len(by_drift)
        counts["drift"] += nd
        counts["suffix"] += sum(1 for p in pos if p >= bs + blk)
        counts["threshold"] += sum(1 for j in range(n) if flags[j] and cur["conf"][j] >= thr)
        counts["fallback"] += int(flags.sum()) - nd - sum(1 for j in range(n) if flags[j] and cur["conf"][j] >= thr)
        say(f"{what} b={b}: bs={bs} valid={valid} hit={hit} committed {pos} ({nd} by drift)")


def test_polestar_commit_decode():
    cfg = PC
    from helpers import spec_of
    spec = spec_of(cfg)
    model, _, head = build(cfg)
    st = runtime.State(cfg)
    pst = runtime.PolestarState(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL, polestar_state=pst)
    # threshold at the 80th percentile of the next block's confidences after
    # the full pass (random weights keep them near 1/V), so that suffix
    # commits can happen
    stats = torch.zeros((cfg.batch * cfg.block_len, 4), dtype=torch.float64, device="cuda")
    bs = st.block_start.clone()
    st.block_start.add_(cfg.block_len)
    B.dllm_lm_head(model.h, st, stats)
    st.block_start.copy_(bs)
    thr = float(np.quantile(1.0 / stats[:, 2].cpu().numpy(), 0.8))
    cfg = cfg.with_(conf_threshold=thr)
    model.cfg = cfg
    say(f"commit threshold {thr:.6e}")
    counts = {"drift": 0, "suffix": 0, "threshold": 0, "fallback": 0}
    for t in range(cfg.n_steps):
        before, pb = Snap(st), _ps_host(pst)
        if np.all(before.block_start >= cfg.seq_len):
            break
        runtime.step(model, st, mode=B.DLLM_MODE_SPARSE, polestar_state=pst)
        _check_step(cfg, spec, head, before, pb, Snap(st), _ps_host(pst), counts, f"t={t}")
    say(f"commits: {counts}")
    # every rule fired (threshold commits here are the suffix block's)
    assert counts["drift"] > 0 and counts["suffix"] > 0 and counts["fallback"] > 0, counts
    model.close()


def test_polestar_commit_step_equals_entry_points():
    cfg = PC
    model, _, _ = build(cfg)
    params = runtime.polestar_params(cfg)
    a, pa = runtime.State(cfg), runtime.PolestarState(cfg)
    runtime.step(model, a, mode=B.DLLM_MODE_FULL, polestar_state=pa)
    b_, pb = runtime.State(cfg), runtime.PolestarState(cfg)
    for k, v in a.tensors().items():
        getattr(b_, k).copy_(v)
    for k in ("log_attn", "win_start", "drift_sum", "drift_cnt", "drift_valid"):
        getattr(pb, k).copy_(getattr(pa, k))
    Bn, L, N = cfg.batch, cfg.seq_len, cfg.n_layers
    idx = torch.zeros((Bn, L), dtype=torch.int32, device="cuda")
    n = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    P0, s0 = a.proxy_ref.clone(), a.score.clone()
    for t in range(4):
        runtime.step(model, a, mode=B.DLLM_MODE_SPARSE, polestar_state=pa)
        nh, nn, hist = b_.n_history.cpu().numpy(), b_.n_new.cpu().numpy(), b_.history.cpu().numpy()
        rows0 = torch.zeros((Bn, L), dtype=torch.int32)
        n0 = torch.zeros(Bn, dtype=torch.int32)
        for bb in range(Bn):
            rows0[bb, :nn[bb]] = torch.from_numpy(hist[bb][nh[bb] - nn[bb]:nh[bb]].copy())
            n0[bb] = int(nn[bb])
        B.dllm_embed(model.h, b_, rows0.cuda(), n0.cuda())
        for l in range(N):
            B.dllm_polestar_drift(model.h, l, b_, pb, params)
            B.dllm_polestar_select(model.h, l, b_, pb, params, idx, n)
            B.dllm_sparse_layer(model.h, l, b_, idx, n, Bn * pb.W)
        B.dllm_polestar_commit(model.h, b_, pb, params, cfg.conf_threshold, cfg.tau)
        torch.cuda.synchronize()
        assert_states_equal(a, b_, f"t={t}", skip=("proxy_ref", "score"))
        assert torch.equal(a.proxy_ref, P0) and torch.equal(a.score, s0)
        for k in ("log_attn", "win_start", "assign", "kl", "top", "drift_sum", "drift_cnt", "drift_valid"):
            assert torch.equal(getattr(pa, k), getattr(pb, k)), f"t={t}: polestar {k} differs"
    model.close()


def test_polestar_commit_rejects_bad_alpha():
    cfg = PC
    model, _, _ = build(cfg)
    st, pst = runtime.State(cfg), runtime.PolestarState(cfg)
    p = runtime.polestar_params(cfg)
    p.commit_alpha = -1.0
    with pytest.raises(B.DllmError):
        B.dllm_polestar_commit(model.h, st, pst, p, cfg.conf_threshold, cfg.tau)
    model.close()
