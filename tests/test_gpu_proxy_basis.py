"""In-library proxy basis (SPA-Cache, method step 1: W_r = U_r S_r of the
value projection) on the GPU against the oracle's fp64 truncated SVD of the
same stored W_V: the drift scores (1 - cos) the two bases give agree to
1e-12 (the subspace iteration converges to the same singular subspace and
values; column signs do not change a cosine), W_r W_r^T agrees (a
basis-independent form), and the column norms are the singular values.
dllm_init_layer without a supplied basis derives it and the layer's drift
scores match those of a model given the oracle's basis.  Shapes: the tiny
fp32 model, a bf16 d = 512 model with n_v = 512 and with GQA n_v = 128."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_common import medium_cfg, say
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, inputs, runtime

pytestmark = pytest.mark.gpu

CFGS = [configs.C1, medium_cfg(name="basis-bf16", n_layers=1),
        medium_cfg(name="basis-gqa", n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=64)]


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_derived_basis_matches_svd(cfg):
    model = runtime.Model(cfg, "cuda")
    w = inputs.layer_weights(cfg, 0, "cuda")
    wv = w["w_v"].contiguous()
    d, r = cfg.d_model, cfg.proxy_rank
    out = torch.zeros((d, r), dtype=torch.float64, device="cuda")
    B.dllm_derive_proxy_basis(model.h, wv, out)
    torch.cuda.synchronize()
    wr = out.cpu().numpy()
    wr_o, s = oracle.proxy_basis(wv.double().cpu().numpy(), r)
    norms = np.sqrt(np.sum(wr * wr, axis=0))
    assert np.max(np.abs(norms - s[:r]) / s[:r]) < 1e-12, "column norms are not the singular values"
    g1, g2 = wr @ wr.T, wr_o @ wr_o.T
    assert np.max(np.abs(g1 - g2)) < 1e-12 * np.max(np.abs(g2)), "W_r W_r^T differs"
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, d))
    y = x + 0.2 * rng.standard_normal((64, d))
    g = 1.0 + 0.1 * rng.standard_normal(d)
    d_gpu = oracle.drift(oracle.proxy(x, g, wr), oracle.proxy(y, g, wr))
    d_or = oracle.drift(oracle.proxy(x, g, wr_o), oracle.proxy(y, g, wr_o))
    err = float(np.max(np.abs(d_gpu - d_or)))
    say(f"{cfg.name}: W_V {tuple(wv.shape)}, r = {r}: max drift difference {err:.2e}")
    assert err < 1e-12
    model.close()


def test_init_layer_derives_basis():
    """dllm_init_layer with w_proxy = NULL: the layer's drift scores equal those
    of a model given the oracle's basis (both stored in fp32)."""
    cfg = CFGS[1]
    w = inputs.layer_weights(cfg, 0, "cuda")
    head = inputs.head_weights(cfg, "cuda")
    wr_o, _ = oracle.proxy_basis(w["w_v"].double().cpu().numpy(), cfg.proxy_rank)
    w_given = dict(w, w_proxy=torch.from_numpy(wr_o).float().cuda())
    w_none = dict(w, w_proxy=None)
    ma = runtime.Model(cfg, "cuda", layers=[w_given], head=head)
    mb = runtime.Model(cfg, "cuda", layers=[w_none], head=head)
    sa, sb = runtime.State(cfg), runtime.State(cfg)
    rng = np.random.default_rng(4)
    h = torch.from_numpy(rng.standard_normal((cfg.batch, cfg.seq_len, cfg.d_model))).to(sa.hidden.dtype).cuda()
    for s_ in (sa, sb):
        s_.hidden[0].copy_(h)
    B.dllm_drift_score(ma.h, 0, sa, None, None)
    B.dllm_drift_score(mb.h, 0, sb, None, None)
    h2 = (h.double() + 0.3 * torch.randn_like(h.double())).to(h.dtype)
    for s_ in (sa, sb):
        s_.hidden[0].copy_(h2)
        s_.proxy_ref[0].copy_(s_.proxy_cur[0])
    B.dllm_drift_score(ma.h, 0, sa, None, None)
    B.dllm_drift_score(mb.h, 0, sb, None, None)
    torch.cuda.synchronize()
    da, db = sa.score[0].cpu().numpy(), sb.score[0].cpu().numpy()
    err = float(np.max(np.abs(da - db)))
    say(f"init_layer-derived basis: max drift difference {err:.2e} (scores up to {da.max():.3f})")
    assert err < 1e-6
    ma.close()
    mb.close()


def test_derived_basis_full_size():
    """The LLaDA-8B layer shape: W_V 4096 x 4096 (bf16), r = 128, 136-column
    subspace, 200 steps; against numpy's fp64 SVD."""
    import time
    cfg = configs.C2
    model = runtime.Model(cfg, "cuda", layers=[dict(inputs.layer_weights(cfg, 0, "cuda"), w_proxy=None)])
    wv = inputs.layer_weights(cfg, 0, "cuda")["w_v"].contiguous()
    out = torch.zeros((cfg.d_model, cfg.proxy_rank), dtype=torch.float64, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    B.dllm_derive_proxy_basis(model.h, wv, out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    wr = out.cpu().numpy()
    t1 = time.perf_counter()
    wr_o, s = oracle.proxy_basis(wv.double().cpu().numpy(), cfg.proxy_rank)
    dt_cpu = time.perf_counter() - t1
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, cfg.d_model))
    y = x + 0.2 * rng.standard_normal(x.shape)
    g = np.ones(cfg.d_model)
    err = float(np.max(np.abs(oracle.drift(oracle.proxy(x, g, wr), oracle.proxy(y, g, wr)) -
                              oracle.drift(oracle.proxy(x, g, wr_o), oracle.proxy(y, g, wr_o)))))
    norms = np.sqrt(np.sum(wr * wr, axis=0))
    say(f"full size: GPU derivation {dt:.2f} s, numpy SVD {dt_cpu:.1f} s, max drift difference {err:.2e}, "
        f"max singular value error {np.max(np.abs(norms - s[:cfg.proxy_rank]) / s[:cfg.proxy_rank]):.2e}")
    assert err < 1e-12
    model.close()
