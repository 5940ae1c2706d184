"""Diagnostics through the C-ABI: the streaming-read probe gives a rate
between a sanity floor and the published HBM peak (8 TB/s), and rejects a
buffer below its minimum; the per-class events of a step cover every class a
sparse step launches."""

from __future__ import annotations

import pytest
import torch

from gpu_common import say
from sparse_kv_cache_value_amd import binding as B
from sparse_kv_cache_value_amd import configs, runtime

pytestmark = pytest.mark.gpu


def test_stream_probe_rate():
    buf = torch.full((512 << 20,), 3, dtype=torch.uint8, device="cuda")
    scratch = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    gbs = B.dllm_stream_probe(buf, scratch, reps=2)
    say(f"streaming read {gbs:.0f} GB/s")
    assert 1000.0 < gbs < 8000.0 * 1.05
    with pytest.raises(B.DllmError):
        B.dllm_stream_probe(buf[: 128 << 20], scratch, reps=2)


def test_profile_classes_of_a_sparse_step():
    cfg = configs.C1
    model = runtime.Model(cfg, "cuda")
    st = runtime.State(cfg)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    B.dllm_profile(model.h, True)
    runtime.step(model, st, mode=B.DLLM_MODE_SPARSE, want_result=False)
    torch.cuda.synchronize()
    prof = B.dllm_profile_read(model.h)
    B.dllm_profile(model.h, False)
    model.close()
    n = cfg.n_layers
    assert prof["gemm"]["launches"] == 4 * n
    assert prof["select"]["launches"] == n
    assert prof["proxy"]["launches"] == n
    assert prof["attention"]["launches"] == n
    # one sequence: the selection and the gather are one launch (select
    # class); then the QKV / O / down epilogues (+ SwiGLU on the fp32 path)
    assert cfg.batch == 1
    assert prof["rows"]["launches"] == (4 if cfg.dtype == configs.FP32 else 3) * n
    assert prof["decide"]["launches"] >= 4
    assert all(v["ms"] >= 0.0 for v in prof.values())
