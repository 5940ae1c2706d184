"""Summaries of rocprofv3 output for the decoding step (text for profiles/).

    python -m sparse_kv_cache_value_amd.prof_summary kernels <kernel_trace.csv> [steps]
        per-step kernel time breakdown over the last `steps` sparse steps

    python -m sparse_kv_cache_value_amd.prof_summary traffic <fetch.csv> <write.csv> [steps]
        FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the GEMM launches of the
        last `steps` steps, each scaled by what the same counter reads for the
        256 MiB calibration copy that bench.py --copy-calibration runs; prints
        the JSON record bench.py reads for roofline.traffic.

A step ends at its LM-head merge kernel (one per step).
"""

from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
CAL_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("gemm.hip", "common.h"):  # the GEMM kernels' device code
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _name(s: str) -> str:
    return re.sub(r"\(.*", "", s)


def _steps(rows, key_start, key_end, name_key, nsteps):
    # a step ends with its commit kernel
    ks = sorted(rows, key=lambda r: int(r[key_start]))
    ends = [i for i, r in enumerate(ks) if "commit_kernel" in r[name_key]]
    if len(ends) < nsteps + 1:
        raise SystemExit(f"trace has {len(ends)} steps, need {nsteps + 1}")
    sel = ends[-nsteps - 1:]
    return ks, sel


def kernels(path: str, nsteps: int = 10) -> str:
    rows = list(csv.DictReader(open(path)))
    ks, sel = _steps(rows, "Start_Timestamp", "End_Timestamp", "Kernel_Name", nsteps)
    agg = defaultdict(lambda: [0, 0.0])
    busy = 0.0
    for a, b in zip(sel[:-1], sel[1:]):
        for r in ks[a + 1:b + 1]:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            n = _name(r["Kernel_Name"])
            agg[n][0] += 1
            agg[n][1] += d
            busy += d
    # from the first kernel of the first selected step (the host work between
    # bench passes before it is not part of the steps)
    span = (int(ks[sel[-1]]["End_Timestamp"]) - int(ks[sel[0] + 1]["Start_Timestamp"])) / 1e3
    out = [f"steps {nsteps}: span/step {span / nsteps:.1f} us, kernel busy/step {busy / nsteps:.1f} us, "
           f"gaps/step {(span - busy) / nsteps:.1f} us",
           f"{'kernel':64s} {'launches/step':>13s} {'avg_us':>8s} {'us/step':>9s}"]
    for n, (c, t) in sorted(agg.items(), key=lambda x: -x[1][1]):
        out.append(f"{n[:64]:64s} {c / nsteps:13.1f} {t / c:8.2f} {t / nsteps:9.1f}")
    gc = sum(c for n, (c, t) in agg.items() if "gemm" in n)
    gt = sum(t for n, (c, t) in agg.items() if "gemm" in n)
    if gc:
        out.append(f"gemm class (every gemm_* launch, layer GEMMs + LM head): {gc / nsteps:.1f} launches/step, "
                   f"average {gt / gc:.2f} us per launch, {gt / nsteps:.1f} us/step")
    return "\n".join(out)


CAL_GRID = (CAL_BYTES // 4) // 4  # fp32 elements, four per thread in torch's vectorised kernel


def _counter(path, counter):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    by = {}
    for r in rows:
        by[r["Dispatch_Id"]] = (int(r["Start_Timestamp"]), _name(r["Kernel_Name"]), float(r["Counter_Value"]),
                                int(r["Grid_Size"]))
    return by


def traffic(fetch_csv: str, write_csv: str, nsteps: int = 3) -> dict:
    rec = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        by = _counter(path, counter)
        seq = sorted(by.values())
        cal = [v for (_, n, v, g) in seq if "elementwise" in n and "Fill" not in n and g == CAL_GRID]
        if not cal:
            raise SystemExit(f"{counter}: no calibration copy dispatch in {path}")
        factor = (sum(cal) / len(cal)) * 1024 / CAL_BYTES
        ends = [i for i, (_, n, _, _) in enumerate(seq) if "lm_merge" in n]
        sel = ends[-nsteps - 1:]
        vals = [v for (_, n, v, _) in seq[sel[0] + 1:sel[-1] + 1] if "gemm" in n]
        rec[counter] = {"kib_per_launch": sum(vals) / len(vals), "launches": len(vals), "copy_factor": factor}
    fetch = rec["FETCH_SIZE"]["kib_per_launch"] * 1024 / rec["FETCH_SIZE"]["copy_factor"]
    write = rec["WRITE_SIZE"]["kib_per_launch"] * 1024 / rec["WRITE_SIZE"]["copy_factor"]
    run = ("rocprofv3 --pmc {c} --kernel-include-regex 'gemm|lm_merge|elementwise' --output-format csv "
           "-d <out_{c}> -o run -- python3 bench.py --steps 3 --warmup 1 --full-steps 0 --no-cpu-baseline "
           "--no-other-configs --copy-calibration")
    cmds = [run.format(c="FETCH_SIZE"), run.format(c="WRITE_SIZE"),
            "python -m sparse_kv_cache_value_amd.prof_summary traffic <out_FETCH_SIZE>/run_counter_collection.csv "
            "<out_WRITE_SIZE>/run_counter_collection.csv 3"]
    return {"commands (from /tmp, TMPDIR=/tmp)": cmds,
            "kernel_class": "gemm (layer GEMMs + LM head)", "steps": nsteps, "counters": rec,
            "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
            "traffic_bytes_per_launch": round(fetch + write), "source_hash": gemm_source_hash()}


def sq_table(path: str, top: int = 10) -> str:
    """Per-kernel ratios from one rocprofv3 --pmc pass of SQ counters:
    SQ_VALU_MFMA_BUSY_CYCLES / (4 SQ_BUSY_CU_CYCLES) (share of SIMD cycles the
    matrix pipe is busy, 4 SIMDs per CU), and SQ_WAIT_ANY, SQ_WAIT_INST_LDS,
    SQ_ACTIVE_INST_LDS over SQ_WAVE_CYCLES (share of wave cycles waiting on any
    counter, waiting on LDS, issuing LDS)."""
    rows = list(csv.DictReader(open(path)))
    agg, disp = defaultdict(lambda: defaultdict(float)), defaultdict(set)
    for r in rows:
        n = _name(r["Kernel_Name"])
        agg[n][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[n].add(r["Dispatch_Id"])
    out = [f"{'kernel':48s} {'dispatches':>10s} {'mfma_busy':>9s} {'wait_any':>8s} {'wait_lds':>8s} {'lds_issue':>9s}"]
    for n, c in sorted(agg.items(), key=lambda x: -x[1].get("SQ_WAVE_CYCLES", 0.0))[:top]:
        wc = max(c["SQ_WAVE_CYCLES"], 1.0)
        out.append(f"{n[:48]:48s} {len(disp[n]):10d} {c['SQ_VALU_MFMA_BUSY_CYCLES'] / max(4 * c['SQ_BUSY_CU_CYCLES'], 1):9.3f} "
                   f"{c['SQ_WAIT_ANY'] / wc:8.3f} {c['SQ_WAIT_INST_LDS'] / wc:8.3f} {c['SQ_ACTIVE_INST_LDS'] / wc:9.3f}")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "kernels":
        print(kernels(sys.argv[2], int(sys.argv[3]) if len(sys.argv) > 3 else 10))
    elif len(sys.argv) >= 3 and sys.argv[1] == "sq":
        print(sq_table(sys.argv[2]))
    elif len(sys.argv) >= 4 and sys.argv[1] == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]) if len(sys.argv) > 4 else 3), indent=1))
    else:
        raise SystemExit(__doc__)
