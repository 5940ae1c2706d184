"""Degenerate cases of the sparse step on the GPU, through the C-ABI.

* An empty index set (every count zero, with the host row bound exact, loose or
  the default) leaves the hidden states, keys, values, proxies and scores
  bitwise unchanged; with two sequences, an empty first sequence and a
  non-empty second one change only the second's listed rows.
* Drift closed forms (SPA-Cache method step 1, the cosine of the rank-r value
  proxy against the cached one): a row whose layer input did not change scores
  exactly 0; a row scaled by 2 (exact in bf16 and in the fp64 proxy) also
  scores exactly 0, since the cosine ignores the row's scale; a negated row
  scores 2 (cosine -1).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_common import TOL, Snap, assert_close, build, medium_cfg, say
from helpers import spec_of
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import runtime

pytestmark = pytest.mark.gpu

MED = medium_cfg(name="edge-medium", seed=31, n_steps=1)
MED_B2 = medium_cfg(name="edge-b2", batch=2, seq_len=96, prompt_len=40, seed=32, n_steps=1)


def _same(a: Snap, b: Snap, what: str, seqs=None):
    for name in ("H", "K", "V", "Pc", "Pr", "score"):
        x, y = getattr(a, name), getattr(b, name)
        if seqs is not None:
            x, y = x[:, seqs], y[:, seqs]
        assert np.array_equal(x, y), f"{what}: {name} changed"


@pytest.mark.parametrize("cfg", [MED, MED_B2], ids=lambda c: c.name)
def test_empty_selection_changes_nothing(cfg):
    model, layers, _ = build(cfg)
    st = runtime.State(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    Bn, L = cfg.batch, cfg.seq_len
    idx = torch.zeros((Bn, L), dtype=torch.int32, device="cuda")
    n = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    before = Snap(st)
    for layer in range(cfg.n_layers):
        for max_rows in (0, 1, 7):
            say(f"{cfg.name}: empty I at layer {layer}, max_rows={max_rows}")
            B.dllm_sparse_layer(model.h, layer, st, idx, n, max_rows=max_rows)
            B.dllm_drift_score(model.h, layer, st, idx, n, max_rows=max_rows)
            _same(before, Snap(st), f"layer {layer} max_rows {max_rows}")
    if Bn == 2:
        # sequence 0 empty, sequence 1 refreshes three rows
        rows = np.array([5, 40, 95], np.int32)
        idx_h = np.zeros((Bn, L), np.int32)
        idx_h[1, :3] = rows
        idx.copy_(torch.from_numpy(idx_h))
        n.copy_(torch.tensor([0, 3], dtype=torch.int32))
        spec = spec_of(cfg)
        B.dllm_sparse_layer(model.h, 0, st, idx, n)
        after = Snap(st)
        _same(before, after, "sequence 0 with an empty list", seqs=[0])
        Kx, Vx, Hx = before.K[0][1].copy(), before.V[0][1].copy(), before.H[1][1].copy()
        oracle.sparse_layer(before.H[0][1], Kx, Vx, Hx, rows.astype(np.int64), layers[0], spec)
        assert_close(after.H[1][1][rows], Hx[rows], TOL[cfg.dtype], "sequence 1 rows")
        mask = np.ones(L, bool)
        mask[rows] = False
        assert np.array_equal(after.H[1][1][mask], before.H[1][1][mask]), "sequence 1: rows outside I changed"
    model.close()


def test_drift_closed_forms():
    cfg = MED
    model, _, _ = build(cfg)
    st = runtime.State(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    Bn, L = cfg.batch, cfg.seq_len
    cap = Bn * L  # the full pass's row bound: the proxy kernels run the same split
    for layer in range(cfg.n_layers):
        say(f"drift closed forms, layer {layer}")
        # unchanged inputs, every row listed
        B.dllm_drift_score(model.h, layer, st, None, None, max_rows=cap)
        s = Snap(st)
        assert np.all(s.score[layer] == 0.0), "unchanged rows must score exactly 0"
        assert np.array_equal(s.Pc[layer], s.Pr[layer]), "unchanged rows must reproduce the cached proxy"
        # row 7 doubled (exact), row 11 negated (exact)
        with torch.no_grad():
            st.hidden[layer, 0, 7] *= 2
            st.hidden[layer, 0, 11].neg_()
        rows = torch.zeros((Bn, L), dtype=torch.int32, device="cuda")
        rows[0, :2] = torch.tensor([7, 11], dtype=torch.int32)
        n = torch.tensor([2], dtype=torch.int32, device="cuda")
        B.dllm_drift_score(model.h, layer, st, rows, n, max_rows=cap)
        s = Snap(st)
        assert s.score[layer][0][7] == 0.0, f"scaled row: drift {s.score[layer][0][7]!r}, want exactly 0"
        assert np.array_equal(s.Pc[layer][0][7], 2.0 * s.Pr[layer][0][7]), "scaled row: proxy must double exactly"
        assert abs(s.score[layer][0][11] - 2.0) <= 1e-12, f"negated row: drift {s.score[layer][0][11]!r}, want 2"
        assert np.array_equal(s.Pc[layer][0][11], -s.Pr[layer][0][11]), "negated row: proxy must flip sign"
        others = np.ones(L, bool)
        others[[7, 11]] = False
        assert np.all(s.score[layer][0][others] == 0.0), "rows not listed keep their score"
    model.close()
