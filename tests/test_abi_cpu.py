"""The C-ABI library loads, exports every function include/libdllm.h declares,
and rejects bad arguments before touching the device (CPU only)."""

import ctypes
import os
import re

import pytest

from sparse_kv_cache_value_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libdllm.h")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dllm_\w+)\s*\(", text, re.M)))


def _lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libdllm.so not built")
    return B.lib()


def test_header_declares_the_entry_points():
    names = declared()
    for n in ("dllm_create", "dllm_destroy", "dllm_init_layer", "dllm_init_head", "dllm_drift_score",
              "dllm_select", "dllm_sparse_layer", "dllm_lm_head", "dllm_commit", "dllm_step",
              "dllm_last_error", "dllm_embed", "dllm_forced_set"):
        assert n in names
    assert set(names) == set(B.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for n in declared():
        assert hasattr(lib, n), n


def _dims(**kw):
    base = dict(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64, d_ffn=1024, vocab=1024,
                max_batch=1, seq_len=128, block_len=32, proxy_rank=16, dtype=B.DLLM_FP32,
                rms_eps=1e-5, rope_theta=1e4)
    base.update(kw)
    return B.DllmDims(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=63), B.DLLM_E_SHAPE),
    (dict(head_dim=36), B.DLLM_E_SHAPE),
    (dict(head_dim=48), B.DLLM_E_SHAPE),
    (dict(d_model=8224), B.DLLM_E_SHAPE),
    (dict(n_q_heads=6, n_kv_heads=4), B.DLLM_E_SHAPE),
    (dict(seq_len=9000), B.DLLM_E_SHAPE),
    (dict(block_len=65), B.DLLM_E_SHAPE),
    (dict(proxy_rank=129), B.DLLM_E_SHAPE),
    (dict(dtype=7), B.DLLM_E_ARG),
    (dict(n_layers=0), B.DLLM_E_ARG),
    (dict(d_model=250), B.DLLM_E_SHAPE),
    (dict(dtype=B.DLLM_BF16, vocab=1000), B.DLLM_E_SHAPE),
])
def test_create_rejects_bad_dims(kw, status):
    lib = _lib()
    h = ctypes.c_void_p()
    st = lib.dllm_create(ctypes.byref(_dims(**kw)), ctypes.byref(h))
    assert st == status
    assert h.value is None
    assert lib.dllm_last_error().decode() != ""


def test_null_arguments_are_rejected():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.dllm_create(None, ctypes.byref(h)) == B.DLLM_E_ARG
    assert lib.dllm_destroy(None) == B.DLLM_OK
    assert lib.dllm_init_layer(None, 0, None, None) == B.DLLM_E_ARG
    assert lib.dllm_init_head(None, None, None, None, None) == B.DLLM_E_ARG
    assert lib.dllm_drift_score(None, 0, None, None, None, 0, None) == B.DLLM_E_ARG
    assert lib.dllm_select(None, 0, None, None, None, 0.1, None, None, None) == B.DLLM_E_ARG
    assert lib.dllm_sparse_layer(None, 0, None, None, None, 0, None) == B.DLLM_E_ARG
    assert lib.dllm_lm_head(None, None, None, None, None) == B.DLLM_E_ARG
    assert lib.dllm_commit(None, None, 0.9, 2.0, None) == B.DLLM_E_ARG
    assert lib.dllm_step(None, None, None, None, None) == B.DLLM_E_ARG
    assert "NULL" in lib.dllm_last_error().decode()


def test_product_path_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libdllm.so")
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_hip_failure_maps_to_dllm_e_hip():
    """A HIP runtime failure (here: no device on this host) comes back as
    DLLM_E_HIP with the runtime's own error text, and no model."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: hipGetDevice succeeds")
    lib = _lib()
    h = ctypes.c_void_p()
    st = lib.dllm_create(ctypes.byref(_dims()), ctypes.byref(h))
    assert st == B.DLLM_E_HIP
    assert h.value is None
    msg = lib.dllm_last_error().decode()
    assert msg.startswith("hipGetDevice: ") and len(msg) > len("hipGetDevice: "), msg
