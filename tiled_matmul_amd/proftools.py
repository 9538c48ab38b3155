"""Summaries of rocprofv3 output for the committed profiles (host tool, no GPU).

    python -m tiled_matmul_amd.proftools stats <kernel_trace.csv> [--skip-first N]
        per-kernel dispatch count and average / median / min / p90 / max duration (us), optionally without
        each kernel's first N dispatches (the warm-up launches of a timed run)
    python -m tiled_matmul_amd.proftools traffic --fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --kernel SUBSTR \
        --workload NAME --plan-kernel ID --out profiles/traffic_<kernel>_<workload>.json
        HBM bytes per launch of the kernel whose name contains SUBSTR, from FETCH_SIZE and
        WRITE_SIZE counter runs (KiB per dispatch), each scaled by the ratio of the known size
        of a plain copy kernel to what the same counter read for it; stamped with the source
        hash of planner kernel ID (ring4_256, gemv_lds, ...) and, with --grid G --block B, the
        launch shape it was measured on.
    python -m tiled_matmul_amd.proftools trace <kernel_trace.csv> --kernel SUBSTR --plan-kernel ID \
        --workload NAME --skip-first N --grid G --block B --command "..." --out profiles/trace_<ID>_<NAME>.json
        duration statistics of the kernel whose name contains SUBSTR (without its first N
        dispatches), stamped like a traffic summary, for bench.py to report beside its own
        HIP-event timing
    python -m tiled_matmul_amd.proftools sha ID
        that source hash: the shared device headers and the file that defines kernel ID
    python -m tiled_matmul_amd.proftools mfma <run_counter_collection.csv> <run_kernel_trace.csv> \
        --kernel SUBSTR [--peak-tflops P]
        per dispatch of the kernel whose name contains SUBSTR, from one rocprofv3 run with
        --kernel-trace and --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
        SQ_INSTS_VALU_MFMA_MOPS_F8 SQ_INSTS_VALU_MFMA_MOPS_F6F4 SQ_LDS_IDX_ACTIVE
        SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE: the average engine clock (busy cycles of one XCD
        over the traced duration), the MFMA utilisation (MFMA-busy cycles over the busy cycles
        of all 1024 SIMDs), the MFMA flops the counters saw (512 per counted op), the rate
        against the peak at 2.4 GHz and at the measured clock, and LDS activity
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# Device sources every kernel is built with (types, waits, tile order, epilogues, MFMA steps).
# The host planner is not hashed: a summary records the launch it was measured on (kernel,
# grid, block), which bench.py compares with the launch it makes.
SHARED_SOURCES = ("common.hpp", "launch.hpp", "mfma_step.hpp")
# Planner kernel id -> the file that defines it.
KERNEL_SOURCE = {
    "zero_fill": "gemm_simple.hip", "simple_64": "gemm_simple.hip", "mfma_128": "gemm_simple.hip",
    "pipe_256": "gemm_pipe.hip", "pipe_128": "gemm_pipe.hip", "persist_256": "gemm_pipe.hip",
    "persist_128": "gemm_pipe.hip", "spec_256": "gemm_pipe.hip", "pingpong_256": "gemm_pingpong.hip",
    "ring8_256": "gemm_ring.hip", "ring4_256": "gemm_ring.hip", "splitk_reduce": "gemm_ring.hip",
    "dtv_256": "gemm_dtv.hip", "roles_256x128": "gemm_roles.hip", "gemv": "gemv.hip", "gemv_lds": "gemv.hip",
    "mx_ring_256": "gemm_mx.hip", "mx_simple_64": "gemm_mx.hip",
    "attn_simple": "attention.hip", "attn_mfma": "attention.hip", "attn_pipe": "attention.hip",
}


def kernel_source_sha(kernel: str | None = None) -> str:
    """Hash of the sources kernel `kernel` (a planner id) is built from: identifies the code a
    profile was taken on.  Without a kernel (or for an unknown id): every source."""
    files = sorted(os.listdir(CSRC))
    if kernel in KERNEL_SOURCE:
        files = [*SHARED_SOURCES, KERNEL_SOURCE[kernel]]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def kernel_durations(path):
    """{kernel name: [duration ns, ...] in launch order} from a kernel trace CSV."""
    d = defaultdict(list)
    for r in _rows(path):
        name = r.get("Kernel_Name") or r.get("Name")
        if "Start_Timestamp" in r and "End_Timestamp" in r:
            start, end = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            d[name].append((start, end - start))
    return {k: [dur for _, dur in sorted(v)] for k, v in d.items()}


def kernel_durations_by_launch(path):
    """{(kernel name, workgroups, threads per workgroup): [duration ns, ...] in launch order}
    (the trace's grid size counts threads, so workgroups = grid size / workgroup size)."""
    d = defaultdict(list)
    for r in _rows(path):
        name = r.get("Kernel_Name") or r.get("Name")
        wg = int(r["Workgroup_Size_X"])
        key = (name, int(r["Grid_Size_X"]) // wg, wg)
        d[key].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return {k: [dur for _, dur in sorted(v)] for k, v in d.items()}


def duration_quantiles(ns):
    """Average, median, min, 90th percentile (nearest rank) and max of durations in ns, in us."""
    v = sorted(ns)
    p90 = v[min(len(v) - 1, max(0, -(-9 * len(v) // 10) - 1))]
    return {"avg": statistics.mean(v) / 1e3, "median": statistics.median(v) / 1e3, "min": v[0] / 1e3,
            "p90": p90 / 1e3, "max": v[-1] / 1e3}


def counter_per_dispatch(path, counter, substr):
    """Average over dispatches of `counter` for kernels whose name contains substr."""
    per = defaultdict(float)
    for r in _rows(path):
        if r["Counter_Name"] == counter and substr in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for a kernel containing {substr!r} in {path}")
    return statistics.mean(per.values()), len(per)


XCDS, CUS, SIMDS, PEAK_GHZ = 8, 256, 1024, 2.4


def mfma_summary(counters, trace, substr, peak_tflops=2500.0):
    """Averages over the dispatches of the kernel whose name contains substr of the counters
    of one --kernel-trace --pmc run (one row per dispatch and counter, summed over the XCDs)
    and the derived rates (see the module docstring)."""
    dur = {}
    for r in _rows(trace):
        if substr in r["Kernel_Name"]:
            dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = defaultdict(dict)
    for r in _rows(counters):
        if substr in r["Kernel_Name"]:
            per[r["Dispatch_Id"]][r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted(set(per) & set(dur), key=int)
    if not ids:
        raise SystemExit(f"no dispatch of a kernel containing {substr!r}")
    out = defaultdict(list)
    for i in ids:
        c, ns = per[i], dur[i]
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS                  # busy cycles of one XCD
        flops = 512.0 * sum(c.get(k, 0.0) for k in ("SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                                      "SQ_INSTS_VALU_MFMA_MOPS_F8",
                                                      "SQ_INSTS_VALU_MFMA_MOPS_F6F4"))
        ghz = cyc / ns
        out["us"].append(ns / 1e3)
        out["ghz"].append(ghz)
        out["mfma_util"].append(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS))
        out["lds_util"].append(c.get("SQ_LDS_IDX_ACTIVE", 0.0) / (cyc * CUS))
        out["lds_bank_conflict"].append(c.get("SQ_LDS_BANK_CONFLICT", 0.0))
        out["flops"].append(flops)
        out["tflops"].append(flops / ns / 1e3)
        out["frac_peak"].append(flops / ns / 1e3 / peak_tflops)
        out["frac_peak_at_clock"].append(flops / ns / 1e3 / (peak_tflops * ghz / PEAK_GHZ))
    res = {k: statistics.mean(v) for k, v in out.items()}
    res["dispatches"] = len(ids)
    return res


def trace_summary(trace, substr, plan_kernel, workload, skip_first, grid, block, command, out=None):
    """Durations of the dispatches of the kernel whose name contains substr (all matching
    names pooled, in launch order, the first skip_first dropped), as a summary bench.py reads."""
    v = [x for name, d in kernel_durations(trace).items() if substr in name for x in d]
    if len(v) <= skip_first:
        raise SystemExit(f"{len(v)} dispatches of a kernel containing {substr!r}, skip {skip_first}")
    v = v[skip_first:]
    q = duration_quantiles(v)
    res = {"kernel": substr, "plan_kernel": plan_kernel, "workload": workload,
           "kernel_source_sha": kernel_source_sha(plan_kernel), "grid": grid, "block": block,
           "command": command, "skip_first": skip_first, "dispatches": len(v),
           **{f"{k}_us": val for k, val in q.items()}}
    if out:
        with open(out, "w") as f:
            json.dump(res, f, indent=1)
    return res


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace")
    s.add_argument("--skip-first", type=int, default=0)
    s.add_argument("--by-launch", action="store_true",
                   help="one row per kernel and launch shape (workgroups x threads)")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--workload",
              "--plan-kernel", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--grid", type=int)
    t.add_argument("--block", type=int)
    tr = sub.add_parser("trace")
    tr.add_argument("trace")
    for a_ in ("--kernel", "--plan-kernel", "--workload", "--command", "--out"):
        tr.add_argument(a_, required=True)
    tr.add_argument("--skip-first", type=int, default=0)
    tr.add_argument("--grid", type=int)
    tr.add_argument("--block", type=int)
    h = sub.add_parser("sha")
    h.add_argument("kernel")
    m = sub.add_parser("mfma")
    m.add_argument("counters")
    m.add_argument("trace")
    m.add_argument("--kernel", required=True)
    m.add_argument("--peak-tflops", type=float, default=2500.0)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--copy-bytes", type=int, required=True)
    a = ap.parse_args()
    if a.cmd == "sha":
        print(kernel_source_sha(a.kernel))
        return
    if a.cmd == "mfma":
        print(json.dumps(mfma_summary(a.counters, a.trace, a.kernel, a.peak_tflops)))
        return
    if a.cmd == "trace":
        print(json.dumps(trace_summary(a.trace, a.kernel, a.plan_kernel, a.workload, a.skip_first,
                                       a.grid, a.block, a.command, a.out), indent=1))
        return
    if a.cmd == "stats":
        if a.by_launch:
            groups = {f"{n[:90]} | {g} x {b}": v for (n, g, b), v in kernel_durations_by_launch(a.trace).items()}
            print("| Kernel | Launch | Calls | Avg (us) | Median (us) | Min (us) | p90 (us) | Max (us) |")
            print("|---|---|---|---|---|---|---|---|")
        else:
            groups = {n[:90]: v for n, v in kernel_durations(a.trace).items()}
            print("| Kernel | Calls | Avg (us) | Median (us) | Min (us) | p90 (us) | Max (us) |")
            print("|---|---|---|---|---|---|---|")
        for name, v in sorted(groups.items(), key=lambda x: -sum(x[1])):
            v = v[a.skip_first:] if len(v) > a.skip_first else v
            q = duration_quantiles(v)
            print(f"| {name} | {len(v)} | {q['avg']:.2f} | {q['median']:.2f} | {q['min']:.2f} | "
                  f"{q['p90']:.2f} | {q['max']:.2f} |")
        return
    fetch, nf = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write, nw = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cfetch, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cwrite, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_scale = a.copy_bytes / (cfetch * 1024.0)
    w_scale = a.copy_bytes / (cwrite * 1024.0)
    out = {
        "kernel": a.kernel, "plan_kernel": a.plan_kernel, "workload": a.workload,
        "kernel_source_sha": kernel_source_sha(a.plan_kernel), "grid": a.grid, "block": a.block,
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "dispatches": [nf, nw],
        "copy_calibration": {"bytes": a.copy_bytes, "fetch_kib": cfetch, "write_kib": cwrite,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "hbm_read_bytes_per_launch": fetch * 1024.0 * f_scale,
        "hbm_write_bytes_per_launch": write * 1024.0 * w_scale,
    }
    out["hbm_bytes_per_launch"] = out["hbm_read_bytes_per_launch"] + out["hbm_write_bytes_per_launch"]
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
