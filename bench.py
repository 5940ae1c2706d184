#!/usr/bin/env python3
"""Benchmark: generated tokens/s of one dLLM denoising step under approximate
KV caching on one MI355X, LLaDA-8B-shaped model (32 layers, d=4096, 32 heads,
SwiGLU 12288, vocab 126464), batch 1, L = 1024 (512 prompt + 512 masked,
block 32), per-layer update ratio rho(l) (mean 16%), value-proxy rank 128,
forced rows = current block + 32 most recent decoded tokens.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  Weights are seeded random init (synthetic); with them
every confidence is far below the 0.9 threshold, so each step commits one
token (TPF = 1) and the maximum entropy (~10.9 nats) always exceeds tau = 2,
i.e. the EntropyCache gate as specified fires on every step.  The headline
(`value`) is therefore the sparse step with the gate disabled (tau = inf:
every step after the prefill is a sparse refresh); the gate-as-specified run
(a full pass every step) is reported under `run_full_gate`.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dLLM gen tokens/s (LLaDA-8B-shape, L=1024, 16% refresh) + % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
CAL_ELEMS = 64 << 20  # fp32 elements of the calibration copy (256 MiB read + 256 MiB written)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_llada8b_sparse_step.json")
BF16_PEAK_TFLOPS = 2516.6


def _ensure_built():
    from sparse_kv_cache_value_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from sparse_kv_cache_value_amd import build
        build.build()


def gemm_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, if it was
    taken with the current GEMM sources (else None)."""
    try:
        from sparse_kv_cache_value_amd import prof_summary
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if rec.get("source_hash") != prof_summary.gemm_source_hash():
            return None
        return rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError, KeyError):
        return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_info():
    """BLAS library numpy uses and its thread count (threadpoolctl)."""
    out = {}
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        out["name"] = blas.get("name")
        out["version"] = blas.get("version")
    except Exception:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                out.setdefault("name", p.get("internal_api"))
                out["internal_api"] = p.get("internal_api")
                out["threads"] = p.get("num_threads")
                break
    except Exception:  # pragma: no cover
        pass
    return out


def cpu_baseline(cfg, budget_s: float = 25.0):
    """The oracle on the host cores, on a bounded sample of the same workload:
    one sparse step of the 32-layer model (proxy of every row, drift,
    selection, sparse layer on the selected rows, for each of the 32 layers,
    then LM-head statistics of the block) with every layer using layer 0's
    weights (same shapes and work); synthetic mid-decode cache."""
    import numpy as np
    import torch
    import oracle
    from oracle.decode import layer_refresh
    from sparse_kv_cache_value_amd import inputs

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    spec = oracle.Spec(n_layers=cfg.n_layers, d_model=cfg.d_model, n_q_heads=cfg.n_q_heads,
                       n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, d_ffn=cfg.d_ffn, vocab=cfg.vocab,
                       seq_len=cfg.seq_len, block_len=cfg.block_len, proxy_rank=cfg.proxy_rank,
                       rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta, bf16=True)
    W = {k: v.float().numpy() for k, v in inputs.layer_weights(cfg, 0, "cpu").items()}
    head = {k: v.float().numpy() for k, v in inputs.head_weights(cfg, "cpu").items()}
    L, d = cfg.seq_len, cfg.d_model
    g = torch.Generator().manual_seed(7)
    x = oracle.round_bf16(torch.randn(L, d, generator=g).numpy())
    K = oracle.round_bf16(torch.randn(L, cfg.n_kv_heads, cfg.head_dim, generator=g).numpy())
    V = oracle.round_bf16(torch.randn(L, cfg.n_kv_heads, cfg.head_dim, generator=g).numpy())
    H = oracle.round_bf16(torch.randn(L, d, generator=g).numpy())
    P = oracle.proxy(x + 0.05 * torch.randn(L, d, generator=g).numpy(), W["attn_norm"], W["w_proxy"])
    forced = np.zeros(L, bool)
    forced[cfg.prompt_len:cfg.prompt_len + cfg.block_len] = True
    forced[cfg.prompt_len - cfg.recent_k:cfg.prompt_len] = True
    t0 = time.perf_counter()
    n_layers_done = 0
    for l in range(cfg.n_layers):
        k = oracle.budget_k(cfg.rho[l], L)
        layer_refresh(x, K, V, H, P, W, spec, k, forced)
        n_layers_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    t_layers = time.perf_counter() - t0
    t1 = time.perf_counter()
    rows = np.arange(cfg.prompt_len, cfg.prompt_len + cfg.block_len)
    oracle.lm_stats(H[rows], head["final_norm"], head["lm_head"], spec)
    t_head = time.perf_counter() - t1
    step_s = t_layers * cfg.n_layers / n_layers_done + t_head
    return {
        "value": round(1.0 / step_s, 6),
        "unit": "tokens/s",
        "cores": int(threads),
        "cpu_model": _cpu_model(),
        "blas": _blas_info(),
        "kind": "oracle",
        "sample": (f"one sparse step of the 32-layer LLaDA-8B-shaped model: oracle proxy/drift/select/sparse layer "
                   f"on {n_layers_done} of {cfg.n_layers} layers (layer-0 weights each, "
                   f"{t_layers:.1f} s, scaled x{cfg.n_layers / n_layers_done:.2f}) + LM-head stats on 32 rows "
                   f"({t_head:.1f} s); TPF = 1, batch 1"),
        "seconds_per_step": round(step_s, 3),
    }


WORKLOADS = {
    "C1": "tiny fp32 dLLM: 2 layers, d=256, 4x64 heads, SwiGLU 1024, vocab 1024, batch 1, L=128 "
          "(64 prompt + 64 masked, block 32), r=16, k=16 refreshed rows/layer",
    "C2": "one LLaDA-8B-shaped layer (d=4096, 32x128, SwiGLU 12288) + LM head 4096x126464 on the 32 block "
          "rows, batch 1, L=512 (256 + 256 masked), k=82 rows, r=128",
    "C4": "Dream-7B-shaped GQA model: 28 layers, d=3584, 28/4 heads x 128, SwiGLU 18944, vocab 152064, "
          "batch 8, L=2048 (1024 + 1024 masked), 328 rows/layer per sequence (16%), r=128, "
          "forced = block + recent 32, gate disabled",
    "C5": "Polestar drift path on the LLaDA-8B layer shape: 32 layers, batch 4, L=4096 (2048 + 2048 masked), "
          "window 96, 16 spherical k-means centroids x 10 iterations, NVFP4 residual codes, top-4 clusters",
    "C5-commit": "C5 with Polestar-Commit (drift-delta rule, alpha = 1, tau_s = 0.9, suffix-block commit): "
                 "LM head over the current and next block",
}

WORKLOADS["C2-ce"] = ("C2 with Confidence Extrapolation on the threshold commit (horizon 2, q = 1e-4, r = 1e-3, "
                      "p_v0 = 1e-2, kappa = 2, gamma = 0.5)")

# the config object behind each name
CONFIG_OF = {"C5-commit": lambda c: c.C5.with_(polestar_commit=True, commit_alpha=1.0),
             "C2-ce": lambda c: c.C2.with_(ce_horizon=2)}


def class_table(prof, steps, achievable, ms_per_step):
    """Per-phase figures from the library's per-class HIP events: ms per step,
    launches, achieved algorithmic GB/s and TFLOP/s, and the fraction of the
    HBM peak and of the measured streaming-read rate."""
    out = {}
    busy = 0.0
    for k, v in prof.items():
        if v["launches"] == 0:
            continue
        busy += v["ms"]
        gbs = v["bytes"] / (v["ms"] * 1e-3) / 1e9 if v["ms"] > 0 else None
        out[k] = {"ms_per_step": round(v["ms"] / steps, 4),
                  "launches_per_step": round(v["launches"] / steps, 2),
                  "GB_per_s": round(gbs, 1) if gbs is not None else None,
                  "TFLOP_per_s": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["ms"] > 0 else None,
                  "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4) if gbs is not None else None,
                  "achievable_frac": round(gbs / achievable, 4) if gbs is not None and achievable else None}
    # launch gaps, host work and any launch outside the classes
    out["unprofiled"] = {"ms_per_step": round(ms_per_step - busy / steps, 4)}
    return out


def achievable_read_gbs():
    """Best streaming-read rate of this device (dllm_stream_probe over 1 GiB)."""
    import torch
    from sparse_kv_cache_value_amd import binding as B
    buf = torch.full((1 << 30,), 7, dtype=torch.uint8, device="cuda")
    scratch = torch.zeros(1 << 13, dtype=torch.uint8, device="cuda")
    gbs = B.dllm_stream_probe(buf, scratch, reps=3)
    del buf, scratch
    torch.cuda.empty_cache()
    return gbs


def bench_config(name, steps, warmup, achievable=None):
    """Sparse steps of one of the other configs (the per-config figures of the
    scope table's measurement row): tokens/s, TPF, per-layer us, the kernel
    classes, and the GEMM class against its roofline (HBM, or the bf16 MFMA
    peak where the GEMMs are compute-bound)."""
    import torch
    from sparse_kv_cache_value_amd import binding as B
    from sparse_kv_cache_value_amd import configs, runtime

    cfg = CONFIG_OF[name](configs) if name in CONFIG_OF else getattr(configs, name)
    model = runtime.Model(cfg, "cuda")
    st = runtime.State(cfg)
    ps = runtime.PolestarState(cfg) if cfg.score == configs.SCORE_POLESTAR else None
    cs = runtime.CEState(cfg) if cfg.ce_horizon > 0 else None
    stream = torch.cuda.current_stream()
    runtime.step(model, st, mode=B.DLLM_MODE_FULL, polestar_state=ps, ce_state=cs)
    for _ in range(warmup):
        runtime.step(model, st, mode=B.DLLM_MODE_SPARSE, want_result=False, polestar_state=ps, ce_state=cs)
    torch.cuda.synchronize()
    def run(classes):
        nh = int(st.n_history.sum())
        B.dllm_profile(model.h, True, classes)
        t0 = time.perf_counter()
        for _ in range(steps):
            runtime.step(model, st, mode=B.DLLM_MODE_SPARSE, want_result=False, polestar_state=ps, ce_state=cs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        prof = B.dllm_profile_read(model.h)
        B.dllm_profile(model.h, False)
        return wall, int(st.n_history.sum()) - nh, prof

    # timed steps with events on the GEMM classes only, then the same number
    # of steps with every class for the per-phase table
    wall, tokens, prof = run(["gemm", "lm_head"])
    wall_all, _, prof_all = run(None)
    model.close()
    del st, ps, cs, model
    torch.cuda.empty_cache()
    ms = 1e3 * wall / steps
    classes = class_table(prof_all, steps, achievable, 1e3 * wall_all / steps)
    g = prof["gemm"]
    gb = g["bytes"] / (g["ms"] * 1e-3) / 1e9 if g["ms"] > 0 else 0.0
    tf = g["flops"] / (g["ms"] * 1e-3) / 1e12 if g["ms"] > 0 else 0.0
    # intensity above the machine balance (peak FLOP/s over peak B/s): MFMA-bound
    mfma_bound = g["bytes"] > 0 and g["flops"] / g["bytes"] > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gb / HBM_PEAK_GBS, 4),
                "frac_of_achievable": round(gb / achievable, 4) if achievable else None}
    roof["kernel"] = "layer GEMMs (gemm class)"
    lm_ms = prof["lm_head"]["ms"] / steps
    return {
        "workload": WORKLOADS[name],
        "dtype": "f32" if cfg.dtype == configs.FP32 else "bf16",
        "tokens_per_s": round(tokens / wall, 3),
        "ms_per_step": round(ms, 4),
        "tpf": round(tokens / steps / cfg.batch, 3),
        "per_layer_sparse_us": round(1e3 * (ms - lm_ms) / cfg.n_layers, 2),
        "steps": steps,
        "roofline": roof,
        "kernel_classes": classes,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--full-steps", type=int, default=3, help="steps timed with the gate as specified")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the short per-config runs (C1, C2, C4, C5) reported under other_configs")
    ap.add_argument("--config", choices=sorted(set(WORKLOADS) - {"C3"}),
                    help="only the per-config sparse-step figures of this config (--steps timed steps, "
                         "--warmup untimed), printed as one JSON line; for profiling one config")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 256 MiB device copy before the timed steps (untimed), the reference kernel for "
                         "the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    _ensure_built()
    if args.config:
        torch.cuda.set_device(0)
        print(json.dumps({"config": args.config, **bench_config(args.config, args.steps, args.warmup,
                                                                achievable_read_gbs())}), flush=True)
        return
    from sparse_kv_cache_value_amd import binding as B
    from sparse_kv_cache_value_amd import configs, runtime

    cfg = configs.C3
    masked = cfg.seq_len - cfg.prompt_len
    if args.warmup + 5 * args.steps + args.full_steps + 1 > masked:
        print("too many steps for 512 masked tokens", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    achievable = achievable_read_gbs()
    t_init = time.perf_counter()
    model = runtime.Model(cfg, "cuda")
    st = runtime.State(cfg)
    init_s = time.perf_counter() - t_init
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.ones(CAL_ELEMS, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # prefill: step 0 is a full pass (and commits)
    runtime.step(model, st, mode=B.DLLM_MODE_FULL)
    for _ in range(args.warmup):
        runtime.step(model, st, mode=B.DLLM_MODE_SPARSE, want_result=False)
    torch.cuda.synchronize()
    nh0 = int(st.n_history.sum())

    # Run B (headline): sparse refresh every step, gate disabled (tau = inf).
    # The library's per-class HIP events bracket every kernel launch on the
    # step's stream during the timed region.
    def run_sparse(n, profile, classes=None):
        nh = int(st.n_history.sum())
        B.dllm_profile(model.h, profile, classes)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(n):
            runtime.step(model, st, mode=B.DLLM_MODE_SPARSE, want_result=False)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        prof = B.dllm_profile_read(model.h) if profile else None
        B.dllm_profile(model.h, False)
        return wall, ev0.elapsed_time(ev1), int(st.n_history.sum()) - nh, prof

    # timed steps: events on the dominant class (layer GEMMs + LM head) only;
    # three runs of K steps each, the median run is reported
    runs = [run_sparse(args.steps, True, ["gemm", "lm_head"]) for _ in range(3)]
    run_ms = [1e3 * r[0] / args.steps for r in runs]
    wall, gpu_ms, tokens, prof = sorted(runs, key=lambda r: r[0])[1]
    ms_per_step = 1e3 * wall / args.steps
    # per-phase table: the same number of steps with events on every class
    wall_all, _, _, prof_all = run_sparse(args.steps, True)
    # and without any events, for their overhead
    wall_np, _, tokens_np, _ = run_sparse(args.steps, False)

    # Run A: gate as specified (tau = 2 nats, AUTO mode reads the flag each step)
    torch.cuda.synchronize()
    nfull = 0
    nh_a = int(st.n_history.sum())
    ta = time.perf_counter()
    for _ in range(args.full_steps):
        res = runtime.step(model, st, mode=B.DLLM_MODE_AUTO, want_result=True)
        nfull += res.n_full
    torch.cuda.synchronize()
    full_s = time.perf_counter() - ta
    full_ms = 1e3 * full_s / max(args.full_steps, 1)
    full_tokens = int(st.n_history.sum()) - nh_a

    g = prof["gemm"]
    lm = prof["lm_head"]
    dom_ms = g["ms"] + lm["ms"]
    dom_launches = g["launches"] + lm["launches"]
    dom_bytes = g["bytes"] + lm["bytes"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9 if dom_ms > 0 else 0.0
    per_step = class_table(prof_all, args.steps, achievable, 1e3 * wall_all / args.steps)
    step_bytes = (g["bytes"] + lm["bytes"]) / args.steps
    out = {
        "metric": METRIC,
        "value": round(tokens / wall, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "timed_runs_ms_per_step": [round(x, 4) for x in run_ms],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, uniform random prompt ids)",
        "config": {
            "workload": "LLaDA-8B-shaped dLLM sparse denoising step: 32 layers, d=4096, 32x128 heads, "
                        "SwiGLU 12288, vocab 126464, batch 1, L=1024 (512 prompt + 512 masked, block 32), "
                        "rho(l) split Gaussian mean 16%, value proxy r=128, forced = block + recent 32, "
                        "gate disabled (tau=inf)",
            "global_batch": 1, "seq_len": cfg.seq_len, "layers": cfg.n_layers,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gemm_stream_kernel, gemm_bf16_kernel (layer GEMMs + LM head)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_of_achievable": round(achieved / achievable, 4),
            "traffic": gemm_traffic(),
            "launches": dom_launches,
            "avg_launch_us": round(1e3 * dom_ms / max(dom_launches, 1), 3),
            "algorithmic_bytes_per_launch": round(dom_bytes / max(dom_launches, 1), 1),
        },
        "achievable_read_GB_per_s": round(achievable, 1),
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 4),
        "ms_per_step_without_kernel_events": round(1e3 * wall_np / args.steps, 4),
        "tokens_per_s_without_kernel_events": round(tokens_np / wall_np, 3),
        "tokens_timed": tokens,
        "tpf": round(tokens / args.steps, 3),
        "per_layer_sparse_us": round(1e3 * (ms_per_step - lm["ms"] / args.steps) / cfg.n_layers, 2),
        "kernel_classes": per_step,
        "step_weight_bytes_GB": round(step_bytes / 1e9, 3),
        "run_full_gate": {"tau": cfg.tau, "ms_per_step": round(full_ms, 3),
                          "tokens_per_s": round(full_tokens / full_s, 3) if full_s > 0 else None,
                          "tokens": full_tokens, "full_pass_fraction": nfull / max(args.full_steps, 1)},
        "speedup_sparse_vs_full": round(full_ms / ms_per_step, 3),
        "init_s": round(init_s, 1),
    }
    model.close()
    del st, model
    torch.cuda.empty_cache()
    if not args.no_other_configs:
        # the other configs of the scope table, a few sparse steps each
        out["other_configs"] = {}
        for name, n, w in (("C1", 20, 3), ("C2", 20, 3), ("C2-ce", 20, 3), ("C4", 8, 2), ("C5", 8, 2),
                           ("C5-commit", 8, 2)):
            out["other_configs"][name] = bench_config(name, n, w, achievable)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
