"""Benchmark of the bf16 GEMM C = A * B^T on one MI355X.

One step = one gemm_bf16 call (the whole GEMM: every tile, the full K loop, the epilogue)
on one set of synthetic inputs already resident in device memory.  The headline workload
is the square 4096^3 GEMM (bf16 inputs N(0,1), fp32 output); the decode GEMV
(M=1, N=K=4096, fp32 output) is measured in a second leg and reported in "gemv".

Timing: W untimed warm-up steps, then K steps between two torch.cuda.synchronize() calls,
timed with HIP events recorded on the stream the kernels are launched on (the library
launches on torch's current stream).  The engine clock is not steady over a short run: from
idle, back-to-back 4096^3 GEMMs run ~104-108 us each for the first ~2 ms, then the clock drops
and they take ~113-128 us for a while, and only after many milliseconds settle near ~104 us.
A run of 5 warm-up and 20 timed steps therefore averages across that drop; the defaults
(300 warm-up, 5000 timed steps) time the settled state.  The amdgpu driver's clock reading is
sampled at the start and end of the timed region and every 2 ms in between (`sclk_mhz`;
in a region of a few milliseconds it mostly shows the clock of what ran before, so the rate
against the peak scaled to that clock, `roofline.frac_at_sclk`, is given only for regions of
0.1 s or more).  Inputs
rotate over several buffer sets whose total exceeds the 256 MB Infinity Cache, so no step
finds its operands in a cache left warm by the previous one.  The GEMV leg captures its
launches in a HIP graph (one kernel is a few microseconds, below the Python launch overhead)
and times graph replays; beside it, the same way, a plain streaming read of the same 32 MiB
buffers and an empty kernel (libtmm_ceiling.so) measure what any single launch can reach on
those bytes (`gemv.ceiling`).  Where a rocprofv3 kernel-trace summary of the same kernel,
sources and launch is committed under profiles/, `roofline.trace` gives the rates its traced
durations imply.

cpu_baseline: the CPU oracle (plain fp64 triple loop, OpenMP over rows) timed on a bounded
sample of the same workload: a band of rows of C, all N columns, the full K.  Its rows are
also compared with the GPU output under the acceptance bound.

Prints ONE JSON line.  `python bench.py --gpus N` with N > 1 exits with status 2: the
bench measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import tiled_matmul_amd as tm  # noqa: E402
from tiled_matmul_amd import roofline as rl  # noqa: E402
from tiled_matmul_amd import synth  # noqa: E402
from tiled_matmul_amd.proftools import kernel_source_sha  # noqa: E402

HBM_TB_S = rl.MI355X_BF16.hbm_tb_s
MFMA_TFLOPS = rl.MI355X_BF16.peak_tflops
MALL_BYTES = 256 * 2 ** 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def make_sets(name, torch, min_bytes, la=0, lb=0, pitch=None):
    """Enough copies of the workload's operands (and outputs) to exceed min_bytes.  Device
    operands are (M, K) and (N, K), or (batch, M, K) and (batch, N, K) for a batched
    workload (rows `pitch` elements apart if given, the padding NaN); the host arrays returned
    are batch item 0's."""
    w = synth.WORKLOADS[name]
    M, N, K, out, batch = w["M"], w["N"], w["K"], w["out"], w["batch"]
    items = [synth.make_operands(name, item=b, lda=pitch, ldb=pitch) for b in range(batch)]
    A, B = items[0]
    if batch == 1:
        Ad, Bd = to_dev(A, torch), to_dev(B, torch)
    else:
        Ad = to_dev(np.stack([a for a, _ in items]), torch)
        Bd = to_dev(np.stack([b for _, b in items]), torch)
    # MN-major operands: the same values stored transposed (K x M, K x N)
    if la == tm.GEMM_LAYOUT_MN_MAJOR:
        Ad = Ad.transpose(-1, -2).contiguous()
    if lb == tm.GEMM_LAYOUT_MN_MAJOR:
        Bd = Bd.transpose(-1, -2).contiguous()
    out_t = torch.float32 if out == tm.GEMM_OUT_FP32 else torch.bfloat16
    cshape = (M, N) if batch == 1 else (batch, M, N)
    per = Ad.numel() * 2 + Bd.numel() * 2 + batch * M * N * (4 if out == tm.GEMM_OUT_FP32 else 2)
    n = max(1, -(-min_bytes // per))
    sets = []
    for i in range(n):
        a = Ad if i == 0 else Ad.clone()
        b = Bd if i == 0 else Bd.clone()
        sets.append((a, b, torch.empty(cshape, dtype=out_t, device="cuda")))
    return (A, B), sets


# Shortest timed region whose clock readings are used to scale the peak (seconds).
SCLK_MIN_REGION_S = 0.1


class SclkSampler:
    """The engine clock the amdgpu driver reports (the level marked current in pp_dpm_sclk): one
    reading as the timed region starts, one as it ends (after the final synchronize), and
    readings every 2 ms in between from a host thread; no GPU call."""

    def __init__(self):
        import glob
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.mhz = []
        self.start = self.end = None

    def read(self):
        import re
        try:
            with open(self.path) as f:
                m = re.search(r"(\d+)\s*[Mm]hz\s*\*", f.read())
            return int(m.group(1)) if m else None
        except OSError:
            return None

    def _run(self):
        while not self._stop.wait(0.002):
            v = self.read()
            if v is not None:
                self.mhz.append(v)

    def __enter__(self):
        import threading
        if self.path:
            self.start = self.read()
            self._stop = threading.Event()
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._t.join()
            self.end = self.read()

    def summary(self, wall_s=None):
        """Median, mean, min and max MHz over every reading (start and end included), or None
        where sysfs does not expose the clock.  The driver's reading trails the clock, so in a
        region of a few milliseconds it mostly shows the clock of what ran just before."""
        v = sorted(x for x in [self.start, *self.mhz, self.end] if x is not None)
        if not v:
            return None
        return {"median": v[len(v) // 2], "mean": round(sum(v) / len(v), 1), "min": v[0], "max": v[-1],
                "start": self.start, "end": self.end, "samples": len(v),
                "timed_region_s": None if wall_s is None else round(wall_s, 4),
                "source": "pp_dpm_sclk (the amdgpu driver's current level): at the start and end of the "
                          "timed region and every 2 ms in between"}


def time_steps(launch, nsets, steps, warmup, torch, sampler=None, chunk=0):
    """Average ms per step over `steps` timed steps after `warmup` untimed ones, the wall time,
    the sampled engine clock and, with chunk > 0, the us per step of each run of `chunk`
    consecutive steps (events between them; the launches stay back to back)."""
    for i in range(warmup):
        launch(i % nsets)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps // chunk + 1)] if chunk > 0 else []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sampler = sampler or SclkSampler()
    with sampler:
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            if chunk > 0 and i % chunk == 0:
                marks[i // chunk].record()
            launch(i % nsets)
        if chunk > 0 and steps % chunk == 0:
            marks[-1].record()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    per_chunk = [round(marks[j].elapsed_time(marks[j + 1]) * 1e3 / chunk, 2) for j in range(len(marks) - 1)
                 if chunk > 0 and (j + 1) * chunk <= steps]
    return start.elapsed_time(end) / steps, wall, sampler.summary(wall), per_chunk


def traffic_for(kernel, workload, grid=None, block=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current sources of the kernel and (where the summary records it) the same launch
    shape of its first kernel; else None.  "a+b" (a call of two kernels) sums both."""
    total = 0
    for i, part in enumerate(kernel.split("+")):
        path = os.path.join(ROOT, "profiles", f"traffic_{part}_{workload}.json")
        if not os.path.exists(path):
            return None
        with open(path) as f:
            t = json.load(f)
        if t.get("kernel_source_sha") != kernel_source_sha(part):
            return None
        if i == 0 and t.get("grid") is not None and (t.get("grid"), t.get("block")) != (grid, block):
            return None
        total += t.get("hbm_bytes_per_launch")
    return total


def trace_for(kernel, workload, grid=None, block=None):
    """The committed rocprofv3 kernel-trace summary of this kernel on this workload
    (profiles/trace_<kernel>_<workload>.json), if it was taken on the current sources of the
    kernel and the same launch shape; else None."""
    path = os.path.join(ROOT, "profiles", f"trace_{kernel}_{workload}.json")
    if "+" in kernel or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha(kernel):
        return None
    if t.get("grid") is not None and (t.get("grid"), t.get("block")) != (grid, block):
        return None
    t["source"] = os.path.relpath(path, ROOT)
    return t


def traced_rate(t, work, peak, unit_scale):
    """Rates from a trace summary: `work` (FLOPs or bytes) per launch over its average and
    median durations, scaled by unit_scale, and their fractions of `peak`."""
    if t is None:
        return None
    avg = work / (t["avg_us"] * 1e-6) / unit_scale
    med = work / (t["median_us"] * 1e-6) / unit_scale
    return {"avg_us": t["avg_us"], "median_us": t["median_us"], "achieved_avg": avg,
            "achieved_median": med, "frac_avg": avg / peak, "frac_median": med / peak,
            "dispatches": t["dispatches"], "command": t["command"], "source": t["source"]}


def gemm_leg(args, torch):
    name = args.workload
    w = synth.WORKLOADS[name]
    M, N, K, out, batch = w["M"], w["N"], w["K"], w["out"], w["batch"]
    sA, sB, sC = (M * K, N * K, M * N) if batch > 1 else (0, 0, 0)
    la = tm.GEMM_LAYOUT_MN_MAJOR if args.a_layout == "mn" else tm.GEMM_LAYOUT_K_MAJOR
    lb = tm.GEMM_LAYOUT_MN_MAJOR if args.b_layout == "mn" else tm.GEMM_LAYOUT_K_MAJOR
    lda = M if la == tm.GEMM_LAYOUT_MN_MAJOR else K
    ldb = N if lb == tm.GEMM_LAYOUT_MN_MAJOR else K
    pitch = None
    if args.pad_pitch:
        if la != tm.GEMM_LAYOUT_K_MAJOR or lb != tm.GEMM_LAYOUT_K_MAJOR:
            raise SystemExit("--pad-pitch takes K-major operands")
        pitch = lda = ldb = -(-K // 64) * 64
        if batch > 1:
            sA, sB = M * pitch, N * pitch
    log(f"[bench] generating {name} operands")
    (A, B), sets = make_sets(name, torch, args.rotate_mb * 2 ** 20, la, lb, pitch)
    variant = tm.VARIANTS[args.variant]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = None
    sk_ws = None
    if args.streamk is not None:
        # stream-K with atomic work claiming: a zeroed workspace of the size the plan gives
        rc, ws_bytes, dp, sk, slots, grid = tm.gemm_bf16_streamk_plan(
            args.streamk, batch, M, N, K, sets[0][0], lda, sA, sets[0][1], ldb, sB, sets[0][2], N, sC, out, cus)
        block = 256
        # its own instances of the ring kernel: no trace or traffic summary of the static
        # kernel applies to it
        kname = "ring4_256 stream-K"
        sk_ws = torch.zeros(max(ws_bytes // 4, 64), dtype=torch.int32, device="cuda")
        splits = {"streamk_mode": args.streamk, "whole_tiles": dp, "cut_tiles": sk, "slots": slots}
    elif args.splits is not None:
        # split K: plan with an unbounded workspace, then allocate what the plan needs
        rc, splits, kname, grid = tm.gemm_bf16_splitk_plan(
            la, lb, args.splits, batch, M, N, K, sets[0][0], lda, sA, sets[0][1], ldb, sB,
            sets[0][2], N, sC, out, 1 << 12, 1 << 62, cus)
        block = 256
        ws_bytes = splits * batch * M * N * 4
        ws = torch.empty(max(ws_bytes // 4, 4), dtype=torch.float32, device="cuda")
        if splits > 1:
            kname += "+splitk_reduce"
    else:
        rc, kname, grid, block = tm.gemm_bf16_layout_plan(
            la, lb, variant, batch, M, N, K, sets[0][0], lda, sA, sets[0][1], ldb, sB, sets[0][2],
            N, sC, out, cus)
    if rc != 0:
        raise SystemExit(f"variant {args.variant} cannot run {name}: {tm.gemm_bf16_status_string(rc)}")

    def launch(i):
        a, b, c = sets[i]
        if sk_ws is not None:
            tm.gemm_bf16_streamk(args.streamk, batch, M, N, K, a, lda, sA, b, ldb, sB, c, N, sC, out, sk_ws,
                                 sk_ws.numel() * 4)
        elif splits is not None:
            tm.gemm_bf16_splitk(la, lb, args.splits, batch, M, N, K, a, lda, sA, b, ldb, sB, c, N,
                                sC, out, ws, ws_bytes)
        else:
            tm.gemm_bf16_layout(la, lb, variant, batch, M, N, K, a, lda, sA, b, ldb, sB, c, N,
                                sC, out)

    log(f"[bench] timing {name}: kernel {kname}, {len(sets)} rotating buffer sets, "
        f"{args.warmup} warm-up + {args.steps} timed steps")
    ms, wall, sclk, per_chunk = time_steps(launch, len(sets), args.steps, args.warmup, torch,
                                           chunk=args.chunk)
    flops = rl.flops(M, N, K, batch)
    tflops = flops / (ms * 1e-3) / 1e12
    obytes = 4 if out == tm.GEMM_OUT_FP32 else 2
    nbytes = batch * rl.algorithmic_bytes(M, N, K, obytes)
    return {
        "name": name, "batch": batch, "M": M, "N": N, "K": K,
        "layouts": f"A {args.a_layout}-major, B {args.b_layout}-major"
                   + (f", row pitch {pitch} elements (128-byte aligned rows)" if pitch else ""),
        "out": "fp32" if out == 0 else "bf16",
        "kernel": kname, "grid": grid, "block": block, "ms": ms, "wall_s": wall,
        "splits": splits, "sclk": sclk, "per_chunk": per_chunk,
        "tflops": tflops, "flops": flops, "bytes": nbytes, "A": A, "B": B, "sets": sets,
    }


FP8_MFMA_TFLOPS = 5000.0   # MI355X dense fp8 (MXFP8) MFMA peak


def mx_leg(args, torch):
    """The block-scaled 8-bit GEMM (gemm_mx) on an MX workload, rotating input sets."""
    name = args.workload
    w = synth.MX_WORKLOADS[name]
    M, N, K, fa, fb, out = w["M"], w["N"], w["K"], w["fa"], w["fb"], w["out"]
    log(f"[bench] generating {name} operands")
    A, SA, B, SB = synth.make_mx_operands(name)
    per = A.size + SA.size + B.size + SB.size + M * N * (4 if out == tm.GEMM_OUT_FP32 else 2)
    nsets = max(1, -(-(args.rotate_mb * 2 ** 20) // per))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    base = [dev(A), dev(SA), dev(B), dev(SB)]
    out_t = torch.float32 if out == tm.GEMM_OUT_FP32 else torch.bfloat16
    sets = [([t if i == 0 else t.clone() for t in base]) + [torch.empty((M, N), dtype=out_t, device="cuda")]
            for i in range(nsets)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    a, sa, b, sb, c = sets[0]
    rc, kname, grid, block = tm.gemm_mx_plan(0, fa, fb, M, N, K, a, K, sa, K // 32, b, K, sb, K // 32,
                                             c, N, out, cus)
    if rc != 0:
        raise SystemExit(f"gemm_mx cannot run {name}: {tm.gemm_bf16_status_string(rc)}")

    def launch(i):
        a, sa, b, sb, c = sets[i]
        tm.gemm_mx(fa, fb, M, N, K, a, K, sa, K // 32, b, K, sb, K // 32, c, N, out)

    log(f"[bench] timing {name}: kernel {kname}, {nsets} rotating buffer sets, "
        f"{args.warmup} warm-up + {args.steps} timed steps")
    ms, wall, sclk, _ = time_steps(launch, nsets, args.steps, args.warmup, torch)
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    fmt = {0: "e4m3", 1: "e5m2"}
    return {
        "metric": "MXFP8 GEMM TFLOP/s (block-scaled 8-bit, fp32 accumulate)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"mx-{fmt[fa]}x{fmt[fb]}", "data": "synthetic",
        "config": {"workload": f"{name}: C = A B^T, M={M} N={N} K={K}, A {fmt[fa]} and B "
                               f"{fmt[fb]} with E8M0 scales per 32 k, fp32 accumulate, "
                               f"{'fp32' if out == 0 else 'bf16'} out",
                   "kernel": kname, "grid": grid, "block": block, "rotating_buffer_sets": nsets},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP8_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / FP8_MFMA_TFLOPS,
                     "traffic": traffic_for(kname, name, grid, block), "flops_per_launch": flops},
        "kernel_source_sha": kernel_source_sha(kname),
        "sclk_mhz": sclk,
    }


def attention_leg(args, torch):
    """The attention forward (attention_fwd) on an attention workload, rotating input sets."""
    name = args.workload
    w = synth.ATTN_WORKLOADS[name]
    B, Hq, Hkv, Lq, Lk, d, causal, out = (w[k] for k in ("B", "Hq", "Hkv", "Lq", "Lk", "d", "causal", "out"))
    log(f"[bench] generating {name} inputs")
    Q, K, V = synth.make_attention_inputs(name)
    per = (Q.size + K.size + V.size) * 2 + Q.size * (4 if out == tm.GEMM_OUT_FP32 else 2)
    nsets = max(1, -(-(args.rotate_mb * 2 ** 20) // per))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    base = [dev(Q), dev(K), dev(V)]
    out_t = torch.float32 if out == tm.GEMM_OUT_FP32 else torch.bfloat16
    sets = [[t if i == 0 else t.clone() for t in base] + [torch.empty(Q.shape, dtype=out_t, device="cuda")]
            for i in range(nsets)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    q, k, v, o = sets[0]
    rc, kname, grid, block = tm.attention_fwd_plan(0, B, Hq, Hkv, Lq, Lk, d, q, k, v, o, w["scale"],
                                                   causal, out, cus)
    if rc != 0:
        raise SystemExit(f"attention_fwd cannot run {name}: {tm.gemm_bf16_status_string(rc)}")

    def launch(i):
        q, k, v, o = sets[i]
        tm.attention_fwd(B, Hq, Hkv, Lq, Lk, d, q, k, v, o, None, w["scale"], causal, out)

    log(f"[bench] timing {name}: kernel {kname}, {nsets} rotating buffer sets")
    ms, wall, sclk, _ = time_steps(launch, nsets, args.steps, args.warmup, torch)
    # FLOPs of the two products over the (query, key) pairs the mask allows
    pairs = sum(min(Lk, max(0, i + (Lk - Lq) + 1)) for i in range(Lq)) if causal else Lq * Lk
    flops = 4.0 * B * Hq * pairs * d
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "attention forward TFLOP/s (bf16 MFMA, fp32 softmax and accumulation)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{name}: B={B} Hq={Hq} Hkv={Hkv} Lq={Lq} Lk={Lk} d={d} "
                               f"{'causal' if causal else 'full'}, {'fp32' if out == 0 else 'bf16'} out",
                   "kernel": kname, "grid": grid, "block": block, "rotating_buffer_sets": nsets},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_TFLOPS, "traffic": traffic_for(kname, name, grid, block),
                     "flops_per_launch": flops},
        "kernel_source_sha": kernel_source_sha(kname),
        "sclk_mhz": sclk,
    }


def gemm_roofline(res):
    """The roof that binds this workload (by its arithmetic intensity against the ridge) and
    the achieved rate against it."""
    ai = res["flops"] / res["bytes"]
    bound = rl.bound(rl.MI355X_BF16, ai)
    if bound == "hbm":
        gbs = res["bytes"] / (res["ms"] * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": gbs, "peak": HBM_TB_S * 1e3, "unit": "GB/s",
             "frac": gbs / (HBM_TB_S * 1e3)}
    else:
        r = {"bound": "mfma", "achieved": res["tflops"], "peak": MFMA_TFLOPS, "unit": "TFLOP/s",
             "frac": res["tflops"] / MFMA_TFLOPS}
    if bound == "mfma" and res.get("sclk"):
        # the same rate against the dense peak scaled to the clock the amdgpu driver reported;
        # only over a region long enough for that reading to follow the clock (it trails by
        # milliseconds, so a short region mostly reads the idle level of what ran before)
        if (res["sclk"].get("timed_region_s") or 0.0) >= SCLK_MIN_REGION_S:
            r["frac_at_sclk"] = res["tflops"] / (MFMA_TFLOPS * res["sclk"]["median"] / 2400.0)
        else:
            r["frac_at_sclk"] = None
    tr = trace_for(res["kernel"], res["name"], res["grid"], res["block"])
    if bound == "hbm":
        r["trace"] = traced_rate(tr, res["bytes"], HBM_TB_S * 1e3, 1e9)
    else:
        r["trace"] = traced_rate(tr, res["flops"], MFMA_TFLOPS, 1e12)
    r.update({"traffic": traffic_for(res["kernel"], res["name"], res["grid"], res["block"]),
              "flops_per_launch": res["flops"], "algorithmic_bytes_per_launch": res["bytes"],
              "intensity_flop_per_byte": ai})
    return r


def gemv_leg(args, torch, name="gemv_m1"):
    w = synth.WORKLOADS[name]
    M, N, K, out = w["M"], w["N"], w["K"], w["out"]
    log(f"[bench] generating {name} operands")
    (A, B), sets = make_sets(name, torch, 2 * MALL_BYTES + 32 * 2 ** 20)
    n = len(sets)

    def launch(i):
        a, b, c = sets[i]
        tm.gemm_bf16(M, N, K, a, K, b, K, c, N, out)

    for i in range(n):      # fills the per-device cache before capture
        launch(i)
    torch.cuda.synchronize()
    reps = max(1, args.gemv_launches // n)
    launches = reps * n * args.gemv_replays
    us = graph_time_us(torch, launch, n, reps, args.gemv_replays)
    nbytes = rl.algorithmic_bytes(M, N, K, 4 if out == tm.GEMM_OUT_FP32 else 2)
    gbs = nbytes / (us * 1e-6) / 1e9
    _, kname, grid, block = tm.gemm_bf16_plan(0, 1, M, N, K, sets[0][0], K, 0, sets[0][1], K, 0,
                                              sets[0][2], N, 0, out)
    ceiling = None if args.no_ceiling else ceiling_leg(args, torch, [b for _, b, _ in sets])
    if ceiling is not None:
        # the same comparison on equal footing: the GEMV's algorithmic bytes per second against
        # the plain read's bytes per second
        ceiling["gemv_frac_of_stream_read"] = gbs / ceiling["stream_read"]["gbs"]
    return {
        "metric": f"GB/s and % of HBM peak, decode GEMV M={M} N={N} K={K} (bf16 in, "
                  f"{'fp32' if out == tm.GEMM_OUT_FP32 else 'bf16'} out)",
        "workload": name,
        "value": gbs, "unit": "GB/s", "us_per_launch": us, "launches": launches,
        "kernel": kname, "grid": grid, "block": block, "rotating_weight_buffers": n,
        "timing": "HIP events around replays of a captured HIP graph of back-to-back launches",
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_TB_S * 1e3, "unit": "GB/s",
                     "frac": gbs / (HBM_TB_S * 1e3), "traffic": traffic_for(kname, name, grid, block),
                     "algorithmic_bytes_per_launch": nbytes,
                     "trace": traced_rate(trace_for(kname, name, grid, block), nbytes, HBM_TB_S * 1e3, 1e9)},
        "ceiling": ceiling,
    }


def graph_time_us(torch, launch, n, reps, replays):
    """us per launch of `launch(i)` for i over range(n), repeated reps times, captured in one
    HIP graph and replayed `replays` times between two events (after one untimed replay)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            for i in range(n):
                launch(i)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (reps * n * replays)


def ceiling_leg(args, torch, bufs):
    """What one launch can reach on the GEMV's bytes: the best cold streaming read of one
    32 MiB buffer (rotating over the same buffers the GEMV's weights live in, more than twice
    the Infinity Cache) over a few launch shapes, and the cost of an empty launch; both timed
    like the GEMV, as back-to-back launches replayed from a HIP graph."""
    from tiled_matmul_amd import ceiling as cl
    nbytes = bufs[0].numel() * bufs[0].element_size()
    n = len(bufs)
    reps = max(1, args.gemv_launches // n)
    sink = torch.zeros(2048 * 1024 // 64, dtype=torch.float32, device="cuda")
    shapes = {}
    for grid in (256, 512, 1024, 2048):
        for block in (256, 1024):
            us = graph_time_us(torch, lambda i: cl.stream_read(bufs[i], nbytes, sink, grid, block), n, reps,
                               args.gemv_replays)
            shapes[f"{grid}x{block}"] = round(us, 3)
    best = min(shapes, key=shapes.get)
    floor = {}
    for grid, block in ((1, 64), (256, 1024)):
        floor[f"{grid}x{block}"] = round(graph_time_us(torch, lambda i: cl.launch_floor(grid, block), n, reps,
                                                       args.gemv_replays), 3)
    us = shapes[best]
    return {"stream_read": {"bytes": nbytes, "us": us, "gbs": nbytes / (us * 1e-6) / 1e9,
                            "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / (HBM_TB_S * 1e3),
                            "best_launch": best, "us_by_launch": shapes,
                            "kernel": "ceiling_stream_read (16-byte non-temporal loads, 4 in flight per thread)"},
            "launch_floor_us": floor,
            "timing": "HIP events around replays of a captured HIP graph of back-to-back launches"}


def cpu_baseline_leg(res, args, torch):
    """The oracle, as it stands, on a band of rows of the same GEMM."""
    import oracle
    from oracle import check as ck
    A, B, K, N = res["A"], res["B"], res["K"], res["N"]
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.gemm(A, B, K=K, rows=list(range(threads)), nthreads=threads)   # one row per thread
    t_probe = max(time.perf_counter() - t0, 1e-3)
    rows = int(min(res["M"], max(threads, args.cpu_seconds / t_probe * threads)))
    rows = max(threads, (rows // threads) * threads)
    sel = list(range(rows))
    log(f"[bench] cpu_baseline: oracle on {rows} rows x {N} x {K} with {threads} threads")
    t0 = time.perf_counter()
    C_ref, Mag = oracle.gemm(A, B, K=K, rows=sel, nthreads=threads)
    t = time.perf_counter() - t0
    flops = 2.0 * rows * N * K
    # time_steps launches set i % nsets for timed step i, so the last timed launch used this set
    assert args.steps >= 1
    out = res["sets"][(args.steps - 1) % len(res["sets"])][2]
    if res["batch"] > 1:
        out = out[0]          # the sample is drawn from batch item 0
    got = out[:rows].cpu()
    got = got.numpy() if got.dtype == torch.float32 else got.view(torch.int16).numpy().view(np.uint16)
    od = 0 if res["out"] == "fp32" else 1
    par = ck.check(got, C_ref, Mag, K, od)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    single = {}
    for name in ("single_tile_128", "gemv_m1"):
        w = synth.WORKLOADS[name]
        a1, b1 = synth.make_operands(name)
        t0 = time.perf_counter()
        oracle.gemm(a1, b1, nthreads=1)
        dt = time.perf_counter() - t0
        single[name] = {"seconds": dt, "tflops": 2.0 * w["M"] * w["N"] * w["K"] / dt / 1e12,
                        "shape": f"{w['M']}x{w['N']}x{w['K']}, full"}
    return {
        "value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "single_thread": single,
        "seconds": t, "cpu_model": cpu_model,
        "sample": f"rows 0..{rows - 1} of C ({rows} x {N} outputs, full K={K}) of the same "
                  f"{res['M']}x{N}x{K} GEMM; fp64 triple loop, OpenMP over rows",
        "parity_rows_checked": rows, "parity_max_err_over_bound": par["max_err_over_bound"],
        "parity_ok": par["ok"],
    }


def copy_leg(args, torch):
    """A plain device copy of known size (the calibration kernel for the byte counters)."""
    n = args.copy_mb * 2 ** 20
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"leg": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": args.steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--chunk", type=int, default=0,
                    help="also report the us per step of every run of this many timed steps")
    ap.add_argument("--workload", default="square_4096",
                    choices=sorted(synth.WORKLOADS) + sorted(synth.MX_WORKLOADS)
                    + sorted(synth.ATTN_WORKLOADS))
    ap.add_argument("--variant", default="auto", choices=sorted(tm.VARIANTS))
    ap.add_argument("--a-layout", default="k", choices=["k", "mn"],
                    help="A stored M x K (k) or K x M (mn)")
    ap.add_argument("--b-layout", default="k", choices=["k", "mn"],
                    help="B stored N x K (k) or K x N (mn: C = A B)")
    ap.add_argument("--splits", type=int, default=None,
                    help="run the GEMM through gemm_bf16_splitk with this many K ranges "
                         "(0: the library's choice)")
    ap.add_argument("--streamk", type=int, default=None, choices=[0, 1, 2],
                    help="run the GEMM through gemm_bf16_streamk with this mode (0 auto, 1 whole "
                         "tiles only, 2 every tile cut when there are fewer tiles than CUs)")
    ap.add_argument("--pad-pitch", action="store_true",
                    help="store A and B rows with a pitch rounded up to 64 elements (128-byte "
                         "aligned rows) instead of K")
    ap.add_argument("--rotate-mb", type=int, default=512,
                    help="total size of the rotating input/output sets")
    ap.add_argument("--gemv-workload", default="gemv_m1", choices=["gemv_m1", "gemv_m16"],
                    help="workload of the GEMV leg")
    ap.add_argument("--gemv-launches", type=int, default=340)
    ap.add_argument("--gemv-replays", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target length of the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read and launch-floor ceilings of the GEMV leg")
    ap.add_argument("--leg", default="all", choices=["all", "gemm", "gemv", "copy", "ceiling"])
    ap.add_argument("--copy-mb", type=int, default=1024)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (each GPU would "
              "take its own columns of B and C, with no communication between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    tm.library()

    if args.leg == "copy":
        copy_leg(args, torch)
        return
    if args.leg == "ceiling":
        _, sets = make_sets("gemv_m1", torch, 2 * MALL_BYTES + 32 * 2 ** 20)
        print(json.dumps({"leg": "ceiling", **ceiling_leg(args, torch, [b for _, b, _ in sets])}))
        return
    if args.leg == "gemv":
        g = gemv_leg(args, torch, args.gemv_workload)
        print(json.dumps({"gemv": g, "kernel_source_sha": kernel_source_sha(g["kernel"])}))
        return

    if args.workload in synth.ATTN_WORKLOADS:
        print(json.dumps(attention_leg(args, torch)))
        return
    if args.workload in synth.MX_WORKLOADS:
        print(json.dumps(mx_leg(args, torch)))
        return
    res = gemm_leg(args, torch)
    result = {
        "metric": "bf16 GEMM TFLOP/s + % MFMA peak at 4096^3; GB/s % HBM peak at M=1",
        "value": res["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{res['name']}: C = A B^T, "
                               + (f"batch={res['batch']} " if res["batch"] > 1 else "")
                               + f"M={res['M']} N={res['N']} K={res['K']}, bf16 in, "
                               f"fp32 accumulate, {res['out']} out",
                   "layouts": res["layouts"], "variant": args.variant, "kernel": res["kernel"],
                   "grid": res["grid"], "block": res["block"], "splits": res["splits"],
                   "rotating_buffer_sets": len(res["sets"])},
        "pct_mfma_peak": 100.0 * res["tflops"] / MFMA_TFLOPS,
        "roofline": gemm_roofline(res),
        "sclk_mhz": res["sclk"],
        **({"us_per_step_by_chunk": {"chunk": args.chunk, "us": res["per_chunk"]}} if args.chunk > 0 else {}),
        "kernel_source_sha": {k: kernel_source_sha(k.split()[0]) for k in res["kernel"].split("+")},
    }
    if args.leg == "all" and not args.no_gemv:
        result["gemv"] = gemv_leg(args, torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_leg(res, args, torch)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
