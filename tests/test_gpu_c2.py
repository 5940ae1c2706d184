"""Full-size single LLaDA-8B-shaped layer (d=4096, 32x128 heads, SwiGLU 12288,
vocab 126464, L=512) with a stale cache on 30% of the rows: drift scores and
the 16% selection must match the oracle exactly, the sparse layer within the
bf16 tolerance, and the commit exactly (shadow mode)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Snap, assert_close, assert_same_selection, build, commit_band, say
from helpers import spec_of
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, inputs, runtime

pytestmark = pytest.mark.gpu


def test_c2_stale_cache_layer():
    cfg = configs.C2
    spec = spec_of(cfg)
    L = cfg.seq_len
    say("== C2: building model")
    model, layers, head = build(cfg, gain_std=0.0)
    W = layers[0]
    h, hc, rows_s = inputs.stale_layer_input(cfg, "cuda")
    st = runtime.State(cfg)
    dev = "cuda"
    # cache from a pass over every row of the stale input
    st.hidden[0].copy_(hc)
    B.dllm_drift_score(model.h, 0, st)
    idx = torch.zeros((1, L), dtype=torch.int32, device=dev)
    n = torch.zeros(1, dtype=torch.int32, device=dev)
    B.dllm_select(model.h, 0, st, None, None, 1.0, idx, n)
    B.dllm_sparse_layer(model.h, 0, st, idx, n)
    s0 = Snap(st)
    hc_np = hc.float().cpu().numpy()[0]
    h_np = h.float().cpu().numpy()[0]
    out_c, Kc, Vc = oracle.layer_dense(hc_np, W, spec)
    e0 = assert_close(s0.H[1][0], out_c, 2e-2, "cache pass H")
    assert_close(s0.K[0][0], Kc, 2e-2, "cache pass K")
    say(f"C2 cache pass: H rel err {e0:.2e}")
    # the current input differs on the stale rows only
    st.hidden[0].copy_(h)
    rows = torch.zeros((1, L), dtype=torch.int32)
    rows[0, :rows_s.shape[1]] = rows_s[0]
    nr = torch.tensor([rows_s.shape[1]], dtype=torch.int32)
    B.dllm_drift_score(model.h, 0, st, rows.to(dev), nr.to(dev))
    k = oracle.budget_k(cfg.rho[0], L)
    assert k == 82
    B.dllm_select(model.h, 0, st, None, None, cfg.rho[0], idx, n)
    sd = Snap(st)
    I_gpu = idx[0, :int(n[0])].cpu().numpy()
    B.dllm_sparse_layer(model.h, 0, st, idx, n)
    sa = Snap(st)
    # drift from the two inputs alone
    C = oracle.proxy(h_np, W["attn_norm"], W["w_proxy"])
    P = oracle.proxy(hc_np, W["attn_norm"], W["w_proxy"])
    s = oracle.drift(C, P)
    stale = set(rows_s[0].tolist())
    assert all((s[i] > 0) == (i in stale) for i in range(L))
    diff = np.abs(sd.score[0][0] - s)
    assert np.all(diff <= 1e-10 * s + 1e-15), f"drift max diff {diff.max():.3e}"
    I_or = oracle.select(s, None, k)
    nb = assert_same_selection(I_gpu, I_or, s, None, k, "C2 selection")
    picked = sorted(s[I_or])
    say(f"C2: |I|={len(I_gpu)} band={nb} score gap at the cut {picked[0]:.3e} -> next "
        f"{max(s[i] for i in range(L) if i not in set(I_or.tolist())):.3e}")
    # sparse layer in shadow mode (GPU cache) and free-running (oracle cache)
    Kx, Vx, Hx = sd.K[0][0].copy(), sd.V[0][0].copy(), sd.H[1][0].copy()
    oracle.sparse_layer(h_np, Kx, Vx, Hx, I_gpu, W, spec)
    mask = np.zeros(L, bool)
    mask[I_gpu] = True
    e1 = assert_close(sa.H[1][0][mask], Hx[mask], 2e-2, "C2 sparse layer (shadow)")
    Ko, Vo, Ho = Kc.copy(), Vc.copy(), out_c.copy()
    oracle.sparse_layer(h_np, Ko, Vo, Ho, I_or, W, spec)
    e2 = assert_close(sa.H[1][0], Ho, 2e-2, "C2 sparse layer (free-running)")
    assert np.array_equal(sa.H[1][0][~mask], sd.H[1][0][~mask])
    say(f"C2 sparse layer: shadow rel err {e1:.2e}, free-running {e2:.2e}")
    # LM head on the 32 block rows and the commit
    stats = torch.zeros((1, cfg.block_len, 4), dtype=torch.float64, device=dev)
    B.dllm_lm_head(model.h, st, stats)
    sg = stats.cpu().numpy()[0]
    bs = int(sa.block_start[0])
    assert bs == 256
    rws = np.arange(bs, bs + cfg.block_len)
    so = oracle.lm_stats(sa.H[1][0][rws], head["final_norm"], head["lm_head"], spec)
    band = commit_band(so, None, cfg.conf_threshold)
    assert np.max(np.abs(sg[:, 0] - so["m"])) <= 1e-5 * np.max(np.abs(so["logits"]))
    assert np.max(np.abs(sg[:, 2] / so["S"] - 1)) <= 1e-5
    for j in range(cfg.block_len):
        if j not in band:
            assert int(sg[j, 1]) == so["argmax"][j]
    ent = np.log(sg[:, 2]) - sg[:, 3] / sg[:, 2]
    assert np.max(np.abs(ent - so["entropy"])) <= 1e-6
    say(f"C2 LM head: entropy {ent.min():.4f}..{ent.max():.4f} (ln V = {np.log(cfg.vocab):.4f}), "
        f"max conf {np.max(1 / sg[:, 2]):.2e}")
    B.dllm_commit(model.h, st, cfg.conf_threshold, cfg.tau)
    s1 = Snap(st)
    pos, tok, emax = oracle.commit(rws, so["conf"], so["argmax"], so["entropy"], sa.committed[0],
                                   cfg.conf_threshold)
    got = [int(p) for p in s1.history[0][:int(s1.n_history[0])]]
    if not ({int(rws[j]) for j in band} & set(pos + got)):
        assert got == pos and [int(s1.tokens[0][p]) for p in pos] == tok
    assert len(got) == 1  # random init: fallback commit of the most confident row
    model.close()
