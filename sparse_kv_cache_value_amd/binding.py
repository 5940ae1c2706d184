"""ctypes binding of libdllm's C-ABI (include/libdllm.h), same names.

Argument marshalling only: tensors are passed as raw device pointers, every
computation runs in the library's HIP kernels.  Importing this module does not
load the library; the first call does, and raises if ``libdllm.so`` has not
been built (``python -m sparse_kv_cache_value_amd.build``).
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdllm.so")

(DLLM_OK, DLLM_E_ARG, DLLM_E_SHAPE, DLLM_E_STATE, DLLM_E_NOMEM, DLLM_E_HIP, DLLM_E_UNSUPPORTED,
 DLLM_E_NUMERIC) = 0, -1, -2, -3, -4, -5, -6, -7
DLLM_PROXY_ITERS = 200
DLLM_FP32, DLLM_BF16 = 0, 1
DLLM_MODE_AUTO, DLLM_MODE_FULL, DLLM_MODE_SPARSE = 0, 1, 2
DLLM_FORCED_NONE, DLLM_FORCED_BLOCK, DLLM_FORCED_BLOCK_RECENT = 0, 1, 2
DLLM_SCORE_SPA_COS, DLLM_SCORE_POLESTAR_KL = 0, 1

_i32, _f32, _f64, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_void_p


class DllmDims(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "d_ffn", "vocab",
        "max_batch", "seq_len", "block_len", "proxy_rank", "dtype")] + [("rms_eps", _f32), ("rope_theta", _f32)]


class DllmLayerWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "attn_norm", "w_q", "w_k", "w_v", "w_o", "ffn_norm", "w_gate", "w_up", "w_down", "w_proxy")]


class DllmState(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "hidden", "k_cache", "v_cache", "proxy_cur", "proxy_ref", "score", "tokens", "committed",
        "history", "n_history", "n_new", "block_start", "full_next", "max_entropy")] + [("batch", _i32)]


class DllmPolestarParams(ctypes.Structure):
    _fields_ = [("n_clusters", _i32), ("kmeans_iters", _i32), ("top_clusters", _i32), ("window_blocks", _i32),
                ("drift_commit", _i32), ("commit_alpha", _f64), ("tau_upd", _i32), ("full_period", _i32)]


class DllmPolestarState(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "log_attn", "win_start", "centroids", "norms", "assign", "codes", "scales", "queries", "kl", "top",
        "drift_sum", "drift_cnt", "drift_valid", "upd_hist")] + [("steps_since_full", _i32)]


class DllmCEParams(ctypes.Structure):
    _fields_ = [("horizon", _i32), ("q", _f64), ("r", _f64), ("p_v0", _f64), ("kappa", _f64), ("gamma", _f64)]


class DllmCEState(ctypes.Structure):
    _fields_ = [("kf", _vp), ("has", _vp)]


class DllmStepParams(ctypes.Structure):
    _fields_ = [("mode", _i32), ("forced_rule", _i32), ("recent_k", _i32), ("tau", _f64),
                ("conf_threshold", _f64), ("rho_h", ctypes.POINTER(_f64)), ("score", _i32),
                ("polestar", ctypes.POINTER(DllmPolestarParams)),
                ("polestar_state", ctypes.POINTER(DllmPolestarState)),
                ("ce", ctypes.POINTER(DllmCEParams)), ("ce_state", ctypes.POINTER(DllmCEState)),
                ("sets_out", _vp), ("n_sets_out", _vp)]


class DllmStepResult(ctypes.Structure):
    _fields_ = [("n_full", _i32), ("n_committed", _i32), ("n_active", _i32), ("max_entropy", _f64)]


(DLLM_PROF_GEMM, DLLM_PROF_LMHEAD, DLLM_PROF_ATTN, DLLM_PROF_PROXY, DLLM_PROF_SELECT, DLLM_PROF_ROWS,
 DLLM_PROF_POLESTAR, DLLM_PROF_DECIDE, DLLM_PROF_N) = range(9)
PROF_NAMES = ("gemm", "lm_head", "attention", "proxy", "select", "rows", "polestar", "decide")


class DllmKernelStats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("ms", _f64), ("bytes", _f64), ("flops", _f64)]


# name -> (restype, argtypes)
SIGNATURES = {
    "dllm_last_error": (ctypes.c_char_p, []),
    "dllm_create": (_i32, [ctypes.POINTER(DllmDims), ctypes.POINTER(_vp)]),
    "dllm_destroy": (_i32, [_vp]),
    "dllm_init_layer": (_i32, [_vp, _i32, ctypes.POINTER(DllmLayerWeights), _vp]),
    "dllm_init_head": (_i32, [_vp, _vp, _vp, _vp, _vp]),
    "dllm_embed": (_i32, [_vp, ctypes.POINTER(DllmState), _vp, _vp, _vp]),
    "dllm_drift_score": (_i32, [_vp, _i32, ctypes.POINTER(DllmState), _vp, _vp, _i32, _vp]),
    "dllm_select": (_i32, [_vp, _i32, ctypes.POINTER(DllmState), _vp, _vp, _f64, _vp, _vp, _vp]),
    "dllm_sparse_layer": (_i32, [_vp, _i32, ctypes.POINTER(DllmState), _vp, _vp, _i32, _vp]),
    "dllm_lm_head": (_i32, [_vp, ctypes.POINTER(DllmState), _vp, _vp, _vp]),
    "dllm_commit": (_i32, [_vp, ctypes.POINTER(DllmState), _f64, _f64, _vp]),
    "dllm_commit_ce": (_i32, [_vp, ctypes.POINTER(DllmState), ctypes.POINTER(DllmCEParams),
                              ctypes.POINTER(DllmCEState), _f64, _f64, _vp]),
    "dllm_forced_set": (_i32, [_vp, ctypes.POINTER(DllmState), _i32, _i32, _vp, _vp]),
    "dllm_polestar_drift": (_i32, [_vp, _i32, ctypes.POINTER(DllmState), ctypes.POINTER(DllmPolestarState),
                                   ctypes.POINTER(DllmPolestarParams), _vp]),
    "dllm_polestar_select": (_i32, [_vp, _i32, ctypes.POINTER(DllmState), ctypes.POINTER(DllmPolestarState),
                                    ctypes.POINTER(DllmPolestarParams), _vp, _vp, _vp]),
    "dllm_polestar_commit": (_i32, [_vp, ctypes.POINTER(DllmState), ctypes.POINTER(DllmPolestarState),
                                    ctypes.POINTER(DllmPolestarParams), _f64, _f64, _vp]),
    "dllm_step": (_i32, [_vp, ctypes.POINTER(DllmState), ctypes.POINTER(DllmStepParams),
                         ctypes.POINTER(DllmStepResult), _vp]),
    "dllm_profile": (_i32, [_vp, _i32]),
    "dllm_profile_read": (_i32, [_vp, ctypes.POINTER(DllmKernelStats)]),
    "dllm_stream_probe": (_i32, [_vp, ctypes.c_size_t, _vp, _i32, ctypes.POINTER(_f64), _vp]),
    "dllm_derive_proxy_basis": (_i32, [_vp, _vp, _i32, _vp, _vp]),
    "dllm_derive_proxy_basis_noalloc": (_i32, [_vp, _vp, _i32, _vp, _vp]),
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_kv_cache_value_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


class DllmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libdllm status {status}: {msg}")
        self.status = status


def _check(status: int):
    if status != DLLM_OK:
        raise DllmError(status, lib().dllm_last_error().decode())


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dllm_last_error() -> str:
    return lib().dllm_last_error().decode()


def dllm_create(dims: DllmDims) -> int:
    h = _vp()
    _check(lib().dllm_create(ctypes.byref(dims), ctypes.byref(h)))
    return h.value


def dllm_destroy(m: int):
    _check(lib().dllm_destroy(m))


def dllm_init_layer(m: int, layer: int, w: dict, stream=None):
    lw = DllmLayerWeights(*[_p(w[k]) for k in (
        "attn_norm", "w_q", "w_k", "w_v", "w_o", "ffn_norm", "w_gate", "w_up", "w_down", "w_proxy")])
    _check(lib().dllm_init_layer(m, layer, ctypes.byref(lw), _stream(stream)))


def dllm_init_head(m: int, embed, final_norm, lm_head, stream=None):
    _check(lib().dllm_init_head(m, _p(embed), _p(final_norm), _p(lm_head), _stream(stream)))


def dllm_embed(m: int, state, rows=None, n_rows=None, stream=None):
    _check(lib().dllm_embed(m, ctypes.byref(state.c), _p(rows), _p(n_rows), _stream(stream)))


def dllm_drift_score(m: int, layer: int, state, rows=None, n_rows=None, max_rows: int = 0, stream=None):
    _check(lib().dllm_drift_score(m, layer, ctypes.byref(state.c), _p(rows), _p(n_rows), max_rows,
                                  _stream(stream)))


def dllm_select(m: int, layer: int, state, forced, full, rho: float, idx, n_sel, stream=None):
    _check(lib().dllm_select(m, layer, ctypes.byref(state.c), _p(forced), _p(full), float(rho), _p(idx),
                             _p(n_sel), _stream(stream)))


def dllm_sparse_layer(m: int, layer: int, state, idx, n_sel, max_rows: int = 0, stream=None):
    _check(lib().dllm_sparse_layer(m, layer, ctypes.byref(state.c), _p(idx), _p(n_sel), max_rows,
                                   _stream(stream)))


def dllm_lm_head(m: int, state, stats_out=None, logits_out=None, stream=None):
    _check(lib().dllm_lm_head(m, ctypes.byref(state.c), _p(stats_out), _p(logits_out), _stream(stream)))


def dllm_commit(m: int, state, conf_threshold: float, tau: float, stream=None):
    _check(lib().dllm_commit(m, ctypes.byref(state.c), float(conf_threshold), float(tau), _stream(stream)))


def dllm_commit_ce(m: int, state, ce: DllmCEParams, ce_state, conf_threshold: float, tau: float, stream=None):
    _check(lib().dllm_commit_ce(m, ctypes.byref(state.c), ctypes.byref(ce), ctypes.byref(ce_state.c),
                                float(conf_threshold), float(tau), _stream(stream)))


def dllm_forced_set(m: int, state, rule: int, recent_k: int, forced, stream=None):
    _check(lib().dllm_forced_set(m, ctypes.byref(state.c), rule, recent_k, _p(forced), _stream(stream)))


def dllm_polestar_drift(m: int, layer: int, state, ps, params: DllmPolestarParams, stream=None):
    _check(lib().dllm_polestar_drift(m, layer, ctypes.byref(state.c), ctypes.byref(ps.c), ctypes.byref(params),
                                     _stream(stream)))


def dllm_polestar_select(m: int, layer: int, state, ps, params: DllmPolestarParams, idx, n_sel, stream=None):
    _check(lib().dllm_polestar_select(m, layer, ctypes.byref(state.c), ctypes.byref(ps.c), ctypes.byref(params),
                                      _p(idx), _p(n_sel), _stream(stream)))


def dllm_polestar_commit(m: int, state, ps, params: DllmPolestarParams, conf_threshold: float, tau: float,
                         stream=None):
    _check(lib().dllm_polestar_commit(m, ctypes.byref(state.c), ctypes.byref(ps.c), ctypes.byref(params),
                                      float(conf_threshold), float(tau), _stream(stream)))


def dllm_step(m: int, state, mode: int, forced_rule: int, recent_k: int, tau: float, conf_threshold: float,
              rho, want_result: bool = True, stream=None, score: int = DLLM_SCORE_SPA_COS,
              polestar: Optional[DllmPolestarParams] = None, polestar_state=None,
              ce: Optional[DllmCEParams] = None, ce_state=None, sets_out=None,
              n_sets_out=None) -> Optional[DllmStepResult]:
    """sets_out [N][B][L] / n_sets_out [N][B] (int32 device tensors, both or
    neither): every layer's index set of the step."""
    rho_arr = (_f64 * len(rho))(*[float(r) for r in rho])
    p = DllmStepParams(mode, forced_rule, recent_k, float(tau), float(conf_threshold),
                       ctypes.cast(rho_arr, ctypes.POINTER(_f64)), score,
                       ctypes.pointer(polestar) if polestar is not None else None,
                       ctypes.pointer(polestar_state.c) if polestar_state is not None else None,
                       ctypes.pointer(ce) if ce is not None else None,
                       ctypes.pointer(ce_state.c) if ce_state is not None else None,
                       _p(sets_out) if sets_out is not None else None,
                       _p(n_sets_out) if n_sets_out is not None else None)
    res = DllmStepResult() if want_result else None
    _check(lib().dllm_step(m, ctypes.byref(state.c), ctypes.byref(p),
                           ctypes.byref(res) if res is not None else None, _stream(stream)))
    return res


def dllm_profile(m: int, enable: bool, classes=None):
    """Per-class event timing on (`classes`: names from PROF_NAMES, default
    all) or off."""
    if not enable:
        mask = 0
    elif classes is None:
        mask = (1 << DLLM_PROF_N) - 1
    else:
        mask = 0
        for c in classes:
            mask |= 1 << PROF_NAMES.index(c)
    _check(lib().dllm_profile(m, mask))


def dllm_derive_proxy_basis(m: int, w_v, w_r_out, iters: int = DLLM_PROXY_ITERS, stream=None):
    """W_r [d][r] fp64 into w_r_out from the device value projection w_v."""
    _check(lib().dllm_derive_proxy_basis(m, _p(w_v), int(iters), _p(w_r_out), _stream(stream)))


def dllm_derive_proxy_basis_noalloc(m: int, w_v, w_r_out, iters: int = DLLM_PROXY_ITERS, stream=None):
    """dllm_derive_proxy_basis with the library's fixed per-device workspace
    (no device allocation in the call)."""
    _check(lib().dllm_derive_proxy_basis_noalloc(m, _p(w_v), int(iters), _p(w_r_out), _stream(stream)))


def dllm_stream_probe(buf, scratch, reps: int = 3, stream=None) -> float:
    """Achievable streaming-read GB/s over the device tensor `buf`
    (>= 256 MiB); `scratch` is a device tensor of >= 8 KiB."""
    out = _f64(0.0)
    _check(lib().dllm_stream_probe(_p(buf), buf.numel() * buf.element_size(), _p(scratch), int(reps),
                                   ctypes.byref(out), _stream(stream)))
    return out.value


def dllm_profile_read(m: int) -> dict:
    arr = (DllmKernelStats * DLLM_PROF_N)()
    _check(lib().dllm_profile_read(m, arr))
    return {PROF_NAMES[i]: {"launches": arr[i].launches, "ms": arr[i].ms, "bytes": arr[i].bytes,
                            "flops": arr[i].flops} for i in range(DLLM_PROF_N)}
