"""Whole decodes on the GPU next to the oracle's decode loop, free-running:
dllm_step and oracle.decode.step each advance their own state from the same
prompt, with no shadowing.  Per step: the mode (full or sparse), every
layer's index set, every layer's hidden states, keys and values, the commits,
tokens, history, entropy gate and block advance.  Decisions the float
tolerance cannot decide (selection and commit tie bands) would end the
comparison if they went different ways, since the two decodes then
legitimately part; the test reports how many steps it compared and requires
all of them on these seeds.

Also: the Polestar drift path refuses an entropy gate that fired for some
sequences only, and a Polestar-Commit step that commits more than a block
(current block plus suffix block) re-embeds every committed row."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_common import (TOL, Snap, assert_close, assert_same_selection, assert_states_equal, build, commit_band,
                        medium_cfg, say)
from helpers import policy_of, spec_of
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, inputs, runtime

pytestmark = pytest.mark.gpu


def _free_running(cfg, steps, what):
    spec = spec_of(cfg)
    tol = TOL[cfg.dtype]
    model, layers, head = build(cfg)
    N, L, Bn = cfg.n_layers, cfg.seq_len, cfg.batch
    assert Bn == 1
    st = runtime.State(cfg)
    tok0, com0 = inputs.prompt_tokens(cfg)
    sq = oracle.decode.SeqState(spec, tok0.numpy()[0], com0.numpy()[0])
    pol = policy_of(cfg)
    sets = torch.zeros((N, Bn, L), dtype=torch.int32, device="cuda")
    nsets = torch.zeros((N, Bn), dtype=torch.int32, device="cuda")
    compared = 0
    for t in range(steps):
        before = Snap(st)
        committed_before = sq.committed.copy()
        res = runtime.step(model, st, mode=B.DLLM_MODE_AUTO, sets_out=sets, n_sets_out=nsets)
        info = oracle.decode.step(sq, layers, head, spec, pol)
        g = Snap(st)
        assert res.n_full == int(info["full"]), f"{what} t={t}: mode"
        S_all, n_all = sets.cpu().numpy(), nsets.cpu().numpy()
        parted = False
        for l in range(N):
            I_gpu = S_all[l, 0, :n_all[l, 0]]
            if info["full"]:
                assert np.array_equal(I_gpu, np.arange(L)), f"{what} t={t} l={l}: full-pass index set"
            else:
                k = oracle.budget_k(cfg.rho[l], L)
                nb = assert_same_selection(I_gpu, info["sets"][l], info["scores"][l], info["forced"], k,
                                           f"{what} t={t} l={l}")
                if nb and not np.array_equal(I_gpu, info["sets"][l]):
                    parted = True
            assert_close(g.H[l + 1][0], sq.H[l + 1], tol, f"{what} t={t} l={l} H")
            assert_close(g.K[l][0], sq.K[l], tol, f"{what} t={t} l={l} K")
            assert_close(g.V[l][0], sq.V[l], tol, f"{what} t={t} l={l} V")
        assert np.array_equal(g.H[0][0], np.asarray(head["embed"])[before.tokens[0]]), f"{what} t={t}: embeddings"
        rows = info["rows"]
        band = commit_band(info["stats"], ~committed_before[rows], pol.conf_threshold) if rows.size else set()
        got = [int(p) for p in g.history[0][before.n_history[0]:g.n_history[0]]]
        if {int(rows[j]) for j in band} & set(info["pos"] + got) and got != info["pos"]:
            parted = True
        else:
            assert got == info["pos"], f"{what} t={t}: committed {got} vs oracle {info['pos']}"
            assert g.history[0][:g.n_history[0]].tolist() == sq.history
            assert np.array_equal(g.tokens[0], sq.tokens), f"{what} t={t}: tokens"
            assert np.array_equal(g.committed[0], sq.committed), f"{what} t={t}: committed"
            assert int(g.block_start[0]) == sq.block_start
            assert int(g.n_new[0]) == sq.n_new
            assert abs(g.max_entropy[0] - info["emax"]) <= 1e-6 * max(1.0, info["emax"])
            assert bool(g.full_next[0]) == bool(sq.full_next)
        say(f"{what} t={t}: full={info['full']} commits {got} E={g.max_entropy[0]:.4f} "
            f"|I|={[int(x) for x in n_all[:, 0]]}")
        if parted:
            say(f"{what}: a tie-band decision at step {t}; the decodes may part, comparison ends")
            break
        compared += 1
    model.close()
    return compared


@pytest.mark.parametrize("tau", [float("inf"), 0.0], ids=["tau-inf", "tau-0"])
def test_c1_free_running_decode(tau):
    """The tiny fp32 config, all 8 steps: step 0 full, then sparse (tau = inf)
    or full at every step (tau = 0: every commit's entropy is positive)."""
    cfg = configs.C1.with_(tau=tau)
    n = _free_running(cfg, cfg.n_steps, f"C1 tau={tau}")
    assert n == cfg.n_steps, f"compared {n} of {cfg.n_steps} steps"


def test_medium_fp32_free_running_decode():
    """A wider fp32 model (several matrix tiles, d = 512) with the EntropyCache
    forced set (current block + the 8 most recent commits) and budgets of 16%
    and 20%, tau = inf: 6 free-running steps."""
    cfg = medium_cfg(name="medium-fp32-free", dtype=configs.FP32, tau=float("inf"), seed=41, n_steps=6)
    n = _free_running(cfg, cfg.n_steps, "medium")
    assert n == cfg.n_steps, f"compared {n} of {cfg.n_steps} steps"


PS = medium_cfg(name="medium-polestar-b2", score=configs.SCORE_POLESTAR, forced=configs.FORCED_BLOCK, recent_k=0,
                seed=33, batch=2, seq_len=224, prompt_len=96, n_steps=3)


def test_polestar_mixed_gate_rejected():
    """With the Polestar score, AUTO mode and the gate set for one sequence of
    two, dllm_step returns DLLM_E_UNSUPPORTED and leaves the state as it was;
    both set or both clear run normally."""
    cfg = PS
    model, _, _ = build(cfg)
    st, pst = runtime.State(cfg), runtime.PolestarState(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL, polestar_state=pst)
    st.full_next.copy_(torch.tensor([1, 0], dtype=torch.uint8))
    keep = {k: v.clone() for k, v in st.tensors().items()}
    with pytest.raises(B.DllmError) as e:
        runtime.step(model, st, mode=B.DLLM_MODE_AUTO, polestar_state=pst)
    assert e.value.status == B.DLLM_E_UNSUPPORTED
    say(f"rejected: {e.value}")
    torch.cuda.synchronize()
    for k, v in st.tensors().items():
        assert torch.equal(v, keep[k]), f"{k} changed by a rejected step"
    st.full_next.fill_(1)
    r = runtime.step(model, st, mode=B.DLLM_MODE_AUTO, polestar_state=pst, tau=float("inf"))
    assert r.n_full == 2
    r = runtime.step(model, st, mode=B.DLLM_MODE_AUTO, polestar_state=pst, tau=float("inf"))
    assert r.n_full == 0
    model.close()


PCX = medium_cfg(name="medium-polestar-commit-wide", score=configs.SCORE_POLESTAR, forced=configs.FORCED_BLOCK,
                 recent_k=0, seed=34, batch=2, seq_len=224, prompt_len=96, top_clusters=16,
                 polestar_commit=True, commit_alpha=1.0, n_steps=4)


def test_polestar_commit_more_than_a_block():
    """Polestar-Commit with every cluster refreshed (so a suffix centroid is
    always among them) and threshold 0 at the second sparse step: the whole
    current block and the whole next block commit in one step (63 tokens per
    sequence).  The next step's layer-0 input must be the embedding of every
    committed token (all rows, bitwise), and dllm_step must equal the
    composition of the entry points."""
    cfg = PCX
    model, _, head = build(cfg)
    params = runtime.polestar_params(cfg)
    a, pa = runtime.State(cfg), runtime.PolestarState(cfg)
    runtime.step(model, a, mode=B.DLLM_MODE_FULL, polestar_state=pa)
    b_, pb = runtime.State(cfg), runtime.PolestarState(cfg)
    for k, v in a.tensors().items():
        getattr(b_, k).copy_(v)
    for k in ("log_attn", "win_start", "drift_sum", "drift_cnt", "drift_valid", "upd_hist"):
        getattr(pb, k).copy_(getattr(pa, k))
    Bn, L, N, blk = cfg.batch, cfg.seq_len, cfg.n_layers, cfg.block_len
    idx = torch.zeros((Bn, L), dtype=torch.int32, device="cuda")
    n = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    P0, s0 = a.proxy_ref.clone(), a.score.clone()
    embed = head["embed"]
    wide = False
    for t, thr in enumerate((0.9, 0.0, 0.9)):
        model.cfg = cfg.with_(conf_threshold=thr)
        tokens_before = a.tokens.cpu().numpy()
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
        B.dllm_polestar_commit(model.h, b_, pb, params, thr, cfg.tau)
        g = Snap(a)
        nnew = g.n_new.tolist()
        say(f"t={t} thr={thr}: commits per sequence {nnew}, block starts {g.block_start.tolist()}")
        if t == 1:
            wide = max(nnew) > blk
        # the layer-0 input of the step: the embedding of every token the step
        # started from (at t = 2, including the wide commit's)
        for bb in range(Bn):
            assert np.array_equal(g.H[0][bb], embed[tokens_before[bb]]), f"t={t} b={bb}: layer-0 input"
        assert_states_equal(a, b_, f"t={t}", skip=("proxy_ref", "score"))
        assert torch.equal(a.proxy_ref, P0) and torch.equal(a.score, s0)
    assert wide, "the threshold-0 step committed no more than a block"
    model.close()
