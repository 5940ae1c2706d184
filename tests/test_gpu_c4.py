"""Full-size Dream-7B-shaped model (28 layers, d=3584, GQA 28/4 x 128, SwiGLU
18944, vocab 152064), batch 8, L=2048 (1024 prompt + 1024 masked), 16%
uniform refresh with forced = current block + 32 recent: one full pass and
one sparse step through the C-ABI entry points, checked against the oracle on
sampled sequences and layers (every row of them) in shadow mode (the oracle's functions applied to
the GPU's own state at each decision point)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_common import assert_close, assert_same_selection, commit_band, say, unpack_k, unpack_v
from helpers import np_weights, spec_of
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, inputs, runtime

pytestmark = pytest.mark.gpu

SEQS = (0, 7)


def _slice(st, l, b):
    """Host copies of sequence b's layer-l slices (layer input, output, K, V, proxies, score)."""
    torch.cuda.synchronize()
    L = st.cfg.seq_len
    return {
        "x": st.hidden[l, b].float().cpu().numpy(),
        "h": st.hidden[l + 1, b].float().cpu().numpy(),
        "K": unpack_k(st.k_cache[l:l + 1, b:b + 1].float().cpu())[0, 0, :L],
        "V": unpack_v(st.v_cache[l:l + 1, b:b + 1].float().cpu())[0, 0, :L],
        "Pr": st.proxy_ref[l, b].cpu().numpy(),
        "Pc": st.proxy_cur[l, b].cpu().numpy(),
        "score": st.score[l, b].cpu().numpy(),
    }


def test_c4_full_size_sampled():
    cfg = configs.C4
    spec = spec_of(cfg)
    N, Bn, L = cfg.n_layers, cfg.batch, cfg.seq_len
    check = (0, N - 1)
    say("== C4: building the 28-layer model on the GPU")
    model = runtime.Model(cfg, "cuda")
    W = {l: np_weights(inputs.layer_weights(cfg, l, "cuda")) for l in check}
    head = np_weights(inputs.head_weights(cfg, "cuda"))
    torch.cuda.empty_cache()
    st = runtime.State(cfg)
    say("C4: full pass (B=8, L=2048)")
    runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    P_or = {}  # the oracle's proxy of each checked row's input at its last refresh
    for l in check:
        for b in SEQS:
            # every row of the layer (M = B*L = 16384 on the device: the row-blocked GEMM)
            s = _slice(st, l, b)
            out, Kx, Vx = oracle.layer_dense(s["x"], W[l], spec)
            e = assert_close(s["h"], out, 2e-2, f"full pass l={l} b={b} H")
            assert_close(s["K"], Kx, 2e-2, f"full pass l={l} b={b} K")
            assert_close(s["V"], Vx, 2e-2, f"full pass l={l} b={b} V")
            C = oracle.proxy(s["x"], W[l]["attn_norm"], W[l]["w_proxy"])
            assert_close(s["Pr"], C, 1e-12, f"full pass l={l} b={b} proxy")
            P_or[(l, b)] = C
            say(f"C4 full pass l={l} b={b}: all {L} rows, H rel err {e:.2e}")

    # one sparse step through the entry points
    dev = "cuda"
    rule = runtime.FORCED_RULE[cfg.forced]
    forced = torch.zeros((Bn, L), dtype=torch.uint8, device=dev)
    B.dllm_forced_set(model.h, st, rule, cfg.recent_k, forced)
    fr = forced.cpu().numpy().astype(bool)
    nh = st.n_history.cpu().numpy()
    nn = st.n_new.cpu().numpy()
    hist = st.history.cpu().numpy()
    rows0 = torch.zeros((Bn, L), dtype=torch.int32)
    n0 = torch.zeros(Bn, dtype=torch.int32)
    for b in range(Bn):
        assert nn[b] == 1
        rows0[b, :nn[b]] = torch.from_numpy(hist[b][nh[b] - nn[b]:nh[b]].copy())
        n0[b] = int(nn[b])
    pi, pn = rows0.to(dev), n0.to(dev)
    idx = [torch.zeros((Bn, L), dtype=torch.int32, device=dev) for _ in range(2)]
    n = [torch.zeros(Bn, dtype=torch.int32, device=dev) for _ in range(2)]
    committed0 = st.committed.cpu().numpy().astype(bool)
    hist_n0 = st.n_history.cpu().numpy().copy()
    bs0 = st.block_start.cpu().numpy().copy()
    B.dllm_embed(model.h, st, pi, pn)
    k = oracle.budget_k(cfg.rho[0], L)
    for l in range(N):
        B.dllm_drift_score(model.h, l, st, pi, pn)
        pre = {b: _slice(st, l, b) for b in SEQS} if l in check else None
        B.dllm_select(model.h, l, st, forced, None, cfg.rho[l], idx[l & 1], n[l & 1])
        B.dllm_sparse_layer(model.h, l, st, idx[l & 1], n[l & 1])
        if pre is not None:
            I_all = idx[l & 1].cpu().numpy()
            n_all = n[l & 1].cpu().numpy()
            for b in SEQS:
                s0 = pre[b]
                s1 = _slice(st, l, b)
                C = oracle.proxy(s0["x"], W[l]["attn_norm"], W[l]["w_proxy"])
                sc = oracle.drift(C, P_or[(l, b)])  # exactly 0 where the input is unchanged
                diff = np.abs(s0["score"] - sc)
                assert np.all(diff <= 1e-10 * np.maximum(sc, 1e-300) + 1e-15), f"l={l} b={b} drift"
                I_or = oracle.select(sc, fr[b], k)
                I_gpu = I_all[b][:n_all[b]]
                band = assert_same_selection(I_gpu, I_or, sc, fr[b], k, f"C4 l={l} b={b}")
                Kx, Vx, Hx = s0["K"].copy(), s0["V"].copy(), s0["h"].copy()
                oracle.sparse_layer(s0["x"], Kx, Vx, Hx, I_gpu, W[l], spec)
                mask = np.zeros(L, bool)
                mask[I_gpu] = True
                e = assert_close(s1["h"][mask], Hx[mask], 2e-2, f"C4 l={l} b={b} sparse H")
                assert_close(s1["K"][mask], Kx[mask], 2e-2, f"C4 l={l} b={b} K rows")
                assert_close(s1["V"][mask], Vx[mask], 2e-2, f"C4 l={l} b={b} V rows")
                assert np.array_equal(s1["h"][~mask], s0["h"][~mask]), "rows outside I changed"
                assert np.array_equal(s1["Pr"][mask], s1["Pc"][mask])
                say(f"C4 sparse l={l} b={b}: |I|={len(I_gpu)} (k={k}) band={band} rel err {e:.2e}")
        pi, pn = idx[l & 1], n[l & 1]
    stats = torch.zeros((Bn, cfg.block_len, 4), dtype=torch.float64, device=dev)
    B.dllm_lm_head(model.h, st, stats)
    B.dllm_commit(model.h, st, cfg.conf_threshold, cfg.tau)
    sg = stats.cpu().numpy()
    hist1 = st.history.cpu().numpy()
    hn1 = st.n_history.cpu().numpy()
    tok1 = st.tokens.cpu().numpy()
    for b in SEQS:
        rows = np.arange(bs0[b], bs0[b] + cfg.block_len)
        hN = st.hidden[N, b].float().cpu().numpy()[rows]
        so = oracle.lm_stats(hN, head["final_norm"], head["lm_head"], spec)
        assert np.max(np.abs(sg[b, :, 0] - so["m"])) <= 1e-5 * np.max(np.abs(so["logits"]))
        ent = np.log(sg[b, :, 2]) - sg[b, :, 3] / sg[b, :, 2]
        assert np.max(np.abs(ent - so["entropy"])) <= 1e-5
        band = commit_band(so, ~committed0[b][rows], cfg.conf_threshold)
        pos, tok, _ = oracle.commit(rows, so["conf"], so["argmax"], so["entropy"], committed0[b],
                                    cfg.conf_threshold)
        got = [int(p) for p in hist1[b][hist_n0[b]:hn1[b]]]
        if not ({int(rows[j]) for j in band} & set(pos + got)):
            assert got == pos and [int(tok1[b][p]) for p in pos] == tok
        say(f"C4 commit b={b}: {got}")
    model.close()
