"""One sparse layer at every row-count regime of the kernels.

The gathered-row GEMMs pick their kernel and tiling from the row count M
(1..384 rows: the weight-streaming kernel with 1..12 row tiles and split K;
more rows: the row-blocked kernel); attention runs 1..33 query tiles per head
over a 1024-key cache.  Each case refreshes a
random index set of M rows spread over the batch and compares the new hidden
rows, keys and values with the oracle's sparse layer on the same inputs.  The
host row bound ``max_rows`` is passed both exact and loose (the kernels read
the true count on the device).
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

# (rows in batch 0, rows in batch 1, extra slack on the host bound)
CASES = [(1, 0, 0), (17, 16, 0), (50, 40, 0), (40, 57, 5), (70, 65, 0), (100, 91, 0), (120, 73, 0),
         (128, 128, 0), (140, 131, 0), (150, 133, 9), (190, 162, 0), (200, 184, 0), (240, 145, 0), (256, 256, 0)]


def _run_cases(cfg, cases, prep=None):
    torch.manual_seed(0)
    spec = spec_of(cfg)
    tol = TOL[cfg.dtype]
    model, layers, head = build(cfg)
    st = runtime.State(cfg)
    Bn, L = cfg.batch, cfg.seq_len
    runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    if prep is not None:
        prep(st)
    rng = np.random.default_rng(7)
    dev = "cuda"
    for case in cases:
        counts, slack = case[:-1], case[-1]
        M = sum(counts)
        idx_h = np.zeros((Bn, L), np.int32)
        for b in range(Bn):
            idx_h[b, :counts[b]] = np.sort(rng.choice(L, counts[b], replace=False))
        idx = torch.from_numpy(idx_h).to(dev)
        n = torch.tensor(counts, dtype=torch.int32, device=dev)
        say(f"{cfg.name}: M={M} {counts} max_rows={M + slack}")
        Sd = Snap(st)
        B.dllm_sparse_layer(model.h, 0, st, idx, n, max_rows=M + slack)
        Sa = Snap(st)
        for b in range(Bn):
            I = idx_h[b, :counts[b]].astype(np.int64)
            x = Sd.H[0][b]
            Kx, Vx, Hx = Sd.K[0][b].copy(), Sd.V[0][b].copy(), Sd.H[1][b].copy()
            oracle.sparse_layer(x, Kx, Vx, Hx, I, layers[0], spec)
            mask = np.zeros(L, bool)
            mask[I] = True
            if I.size:
                e = assert_close(Sa.H[1][b][mask], Hx[mask], tol, f"M={M} b={b} H")
                assert_close(Sa.K[0][b][mask], Kx[mask], tol, f"M={M} b={b} K")
                assert_close(Sa.V[0][b][mask], Vx[mask], tol, f"M={M} b={b} V")
                say(f"  b={b} |I|={I.size} H rel err {e:.2e}")
            assert np.array_equal(Sa.H[1][b][~mask], Sd.H[1][b][~mask]), "rows outside I changed"
            assert np.array_equal(Sa.K[0][b][~mask], Sd.K[0][b][~mask]), "keys outside I changed"
    model.close()


def test_sparse_layer_row_counts():
    """Every GEMM row-tile count, batch 2."""
    cfg = medium_cfg(name="rows-bf16", n_layers=1, batch=2, seq_len=256, prompt_len=128, seed=31, n_steps=1)
    _run_cases(cfg, CASES)


@pytest.mark.parametrize("heads,dh", [(8, 64), (4, 128)])
def test_attention_long_cache(heads, dh):
    """L = 1024 (GQA 2:1) with 1..1024 selected rows."""
    cfg = medium_cfg(name=f"split-h{heads}-d{dh}", n_layers=1, batch=1, seq_len=1024, prompt_len=512,
                     n_q_heads=heads, n_kv_heads=heads // 2, head_dim=dh, seed=33, n_steps=1)
    _run_cases(cfg, [(1, 0), (37, 3), (200, 0), (700, 0), (1024, 0)])


def _scale_key_tiles(st):
    """Layer-0 keys of 32-key tile t scaled by 2^(t % 3), tile 5 by 2^3 more
    (powers of two: exact in bf16).  Each query's score maximum then grows by
    far more than 8 (log2 units) inside a wave's key range and stays put over
    other tiles, so the attention kernels' running-maximum update, their
    output rescale and its skip all run on sharply peaked softmaxes."""
    k = st.k_cache[0]  # [B][G][T][KS][64][8], fragment order
    T = k.shape[2]
    f = torch.tensor([2.0 ** (t % 3) for t in range(T)], dtype=torch.float32)
    f[min(5, T - 1)] *= 8.0
    k.mul_(f.view(1, 1, T, 1, 1, 1).to(device=k.device, dtype=k.dtype))


@pytest.mark.parametrize("heads,kv,dh", [(4, 2, 128), (8, 4, 64), (8, 2, 64)])
def test_attention_score_range(heads, kv, dh):
    """L = 1024 keys whose tiles are scaled 1x to 32x: the multi-head kernel
    (2 query heads per KV head) and the grouped-query kernel (4 per KV head)
    against the oracle's sparse layer on the same scaled cache."""
    cfg = medium_cfg(name=f"range-h{heads}-kv{kv}-d{dh}", n_layers=1, batch=1, seq_len=1024, prompt_len=512,
                     n_q_heads=heads, n_kv_heads=kv, head_dim=dh, seed=39, n_steps=1)
    _run_cases(cfg, [(37, 0), (200, 0), (700, 0)], prep=_scale_key_tiles)


def test_wide_layer_shapes():
    """d = 2048, SwiGLU 5632 (K split 8 and 11 ways, 32..88 slabs), GQA 2:1;
    1..288 rows."""
    cfg = medium_cfg(name="wide-bf16", n_layers=1, batch=2, seq_len=256, prompt_len=128, d_model=2048,
                     n_q_heads=16, n_kv_heads=8, head_dim=128, d_ffn=5632, seed=35, n_steps=1)
    _run_cases(cfg, [(1, 0, 0), (20, 20, 0), (64, 36, 3), (90, 70, 0), (110, 90, 0), (140, 110, 0), (150, 138, 0)])
