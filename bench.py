#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 + double-quant linear layer on one MI355X.

One step = one pass of the whole hot path over one batch of seeded synthetic
input, with every input already resident in HBM:
  blockwise NF4 + double quantization of the fp32 weight,
  forward  Y = X·Ŵ + s·(X·A)·B   (T = X·A kept for the backward),
  backward dX = dY·Ŵᵀ + s·(dY·Bᵀ)·Aᵀ, dA, dB.
Default workload: one 4096×4096 linear, 4096 tokens (2 × 2048), rank 64,
s = 2, W ~ N(0, 0.02), X, dY ~ N(0, 1), A, B ~ N(0, 0.02).

`value` is algorithmic fwd+bwd TFLOP/s, 4·M·d·o + 6·M·r·(d+o) FLOP per step
(quantize and dequant count no FLOPs; their time is included).  The JSON line
also carries the dominant kernel's roofline, the few-token dequant-GEMV
bandwidth on the 7B-style MLP weights, the quantization error of each 4-bit
table (NF4, int4, FP4 E2M1, FP4 E3M0) and of the second-level variants on the
workload's weight, the merge/re-quantize study, the (paged) AdamW step of a
65B-style block's adapters, and the CPU oracle timed on the host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_hbm_bytes.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "pmc_mfma_busy_k_qgemm_linear_4096.json")
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE",
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16"]
# Kernels whose HBM bytes per dispatch the counter passes record: name in the
# trace, the sources that define its code, the workload it ran on, and the
# grid size that selects its dispatches of that workload (None: all).
PMC_KERNELS = {
    "k_qgemm": ("k_qgemm", ["qgemm.hip", "common.h"], "linear_4096", None),
    "k_quantize": ("k_quantize", ["quant.hip", "common.h"], "linear_4096", 1024 * 512),   # 1024 groups × 512 threads
    "k_rank_down": ("k_rank_down", ["rank.hip", "common.h"], "linear_4096", None),
    "k_rank_grad": ("k_rank_grad", ["rank.hip", "common.h"], "linear_4096", None),
    "k_reduce_planes": ("k_reduce_planes", ["gemm.hip", "common.h"], "linear_4096", None),
    "k_gemv<1>": ("k_gemv<1>", ["gemv.hip", "common.h"], "decode_mlp_7b", None),
    "k_lora_down_small": ("k_lora_down_small", ["gemv.hip", "common.h"], "decode_mlp_7b", None),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="linear_4096")
    ap.add_argument("--decode-sets", type=int, default=16,
                    help="independent weight sets cycled by the decode measurement")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-blocks", action="store_true",
                    help="skip the 7B / 65B-style block measurements")
    ap.add_argument("--no-tiny", action="store_true",
                    help="skip the 128x128 latency measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pmc", action="store_true",
                    help="short run for hardware-counter passes: a 256 MiB device copy "
                         "(calibration of FETCH_SIZE/WRITE_SIZE) and --steps steps, no timing")
    ap.add_argument("--mfma-summary", metavar="CSV",
                    help="turn the counter_collection.csv of an MFMA-busy pass of --pmc into "
                         + os.path.relpath(MFMA_FILE, ROOT))
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter_collection.csv files of a FETCH_SIZE pass and a "
                         "WRITE_SIZE pass of --pmc into " + os.path.relpath(PMC_FILE, ROOT))
    return ap.parse_args()


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "nf4_double_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_entry(kernel: str, workload: str):
    """The kept counter figures of one kernel, or None when they are missing
    or were taken on other sources or another workload."""
    if not os.path.exists(PMC_FILE):
        return None
    with open(PMC_FILE) as f:
        kept = json.load(f)
    e = kept.get("kernels", {}).get(kernel)
    if e is None or e.get("workload") != workload:
        return None
    if e.get("source_hash") != source_hash(PMC_KERNELS[kernel][1]):
        return None
    return e


def pmc_summary(fetch_csv: str, write_csv: str) -> dict:
    """HBM bytes per dispatch of each kernel in PMC_KERNELS from a FETCH_SIZE
    pass and a WRITE_SIZE pass of `bench.py --pmc`.

    Each counter (KiB per dispatch) is scaled by the ratio of the known bytes
    of the calibration kernel (256 MiB read, 256 MiB written) to what the same
    counter reports for it in the same pass.
    """
    import csv

    def rows(path, counter):
        with open(path) as f:
            return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]

    factors, per = {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rs = rows(path, counter)
        cal = [float(r["Counter_Value"]) for r in rs if "MulFunctor" in r["Kernel_Name"]]
        if not cal:
            raise SystemExit(f"{path}: no calibration dispatches for {counter}")
        cal_kib = statistics.median(cal)
        factors[counter] = {"calibration_kib": cal_kib, "factor": (256 << 20) / (cal_kib * 1024.0)}
        for name, (pat, _, _, grid) in PMC_KERNELS.items():
            vals = [float(r["Counter_Value"]) for r in rs if pat in r["Kernel_Name"]
                    and (grid is None or int(r["Grid_Size"]) == grid)]
            if vals:
                per.setdefault(name, {})[counter] = (statistics.mean(vals), len(vals))
    kernels = {}
    for name, c in per.items():
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        fetch = c["FETCH_SIZE"][0] * 1024 * factors["FETCH_SIZE"]["factor"]
        write = c["WRITE_SIZE"][0] * 1024 * factors["WRITE_SIZE"]["factor"]
        kernels[name] = {"workload": PMC_KERNELS[name][2], "source_hash": source_hash(PMC_KERNELS[name][1]),
                         "dispatches": c["FETCH_SIZE"][1],
                         "hbm_fetch_bytes_per_dispatch": round(fetch),
                         "hbm_write_bytes_per_dispatch": round(write),
                         "hbm_bytes_per_dispatch": round(fetch + write)}
    fetch_rel, write_rel = os.path.relpath(fetch_csv, ROOT), os.path.relpath(write_csv, ROOT)
    commands = [
        f"rocprofv3 --pmc FETCH_SIZE -f csv -d {os.path.dirname(fetch_rel)} -o fetch -- "
        "python3 bench.py --pmc --steps 3",
        f"rocprofv3 --pmc WRITE_SIZE -f csv -d {os.path.dirname(write_rel)} -o write -- "
        "python3 bench.py --pmc --steps 3",
        f"python3 bench.py --pmc-summary {fetch_rel} {write_rel}",
    ]
    return {"commands": commands, "calibration": factors, "kernels": kernels}


def mfma_summary(csv_path: str) -> dict:
    """MFMA-busy figures of k_qgemm (forward and backward averaged) from one
    counter pass of `bench.py --pmc` collecting MFMA_COUNTERS."""
    import csv
    with open(csv_path) as f:
        rs = [r for r in csv.DictReader(f) if "k_qgemm" in r["Kernel_Name"]]
    vals = {}
    for c in MFMA_COUNTERS:
        v = [float(r["Counter_Value"]) for r in rs if r["Counter_Name"] == c]
        if v:
            vals[c] = statistics.mean(v)
    rel = os.path.relpath(csv_path, ROOT)
    out = {"kernel": "k_qgemm (forward and backward launches averaged)", "workload": "linear_4096",
           "source_hash": source_hash(PMC_KERNELS["k_qgemm"][1]), "counters_per_dispatch": vals,
           "command": f"rocprofv3 --pmc {' '.join(MFMA_COUNTERS)} -f csv -d {os.path.dirname(rel)} "
                      "-o mfma -- python3 bench.py --pmc --steps 3"}
    # share of the CUs' busy cycles in which their matrix pipes were busy: the
    # MFMA counter sums over the 4 SIMDs of each CU, the busy counter over CUs
    if vals.get("SQ_BUSY_CU_CYCLES"):
        out["mfma_busy_frac"] = round(vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * vals["SQ_BUSY_CU_CYCLES"]), 4)
    if vals.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
        # bf16 MFMA work in units of 512 flop: checks the algorithmic count
        out["mfma_flop_per_dispatch"] = vals["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    return out


def step_flops(M, d, o, r):
    return 4 * M * d * o + 6 * M * r * (d + o)


def main():
    args = parse()
    if args.mfma_summary:
        res = mfma_summary(args.mfma_summary)
        with open(MFMA_FILE, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
        print(json.dumps(res))
        return
    if args.pmc_summary:
        res = pmc_summary(*args.pmc_summary)
        with open(PMC_FILE, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
        print(json.dumps(res))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer would shard by tokens with an all-reduce of dA, dB; not built).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nf4_double_quant_amd as qb
    import synth

    qb.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]
    p = wl.projs[0]
    M, d, o, r, s = wl.M, p.d, p.o, wl.r, wl.s

    W_h, X_h, A_h, B_h, dY_h = synth.layer_inputs(wl, p)
    bf = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    W = torch.from_numpy(W_h).to(dev)
    X, A, B, dY = bf(X_h), bf(A_h), bf(B_h), bf(dY_h)
    q = qb.qlora_quantize_nf4_dq(W)
    Y = torch.empty((M, o), dtype=torch.bfloat16, device=dev)
    ws_f, ws_b = qb.Workspace(), qb.Workspace()

    def step():
        qb.qlora_quantize_nf4_dq(W, check_finite=False, out=q)
        _, T = qb.qlora_linear_fwd(X, q, A, B, s, ws=ws_f, out=Y)
        qb.qlora_linear_bwd(dY, X, T, q, A, B, s, ws=ws_b)

    if args.pmc:
        # calibration: an elementwise kernel that reads exactly 256 MiB and
        # writes exactly 256 MiB (torch's MulFunctor kernel)
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        # one pass of the 1-token decode over every weight set
        dwl, sets, adapters, _ = decode_setup(args, qb, torch, np, synth, dev)
        xs, ys = decode_inputs(qb, torch, np, synth, dev, dwl, 1)
        dws = qb.Workspace()
        for layer in sets:
            for p_, qw in layer:
                A_, B_ = adapters[p_.name]
                qb.qlora_linear_fwd(xs[p_.name], qw, A_, B_, dwl.s, want_T=False, ws=dws, out=ys[p_.name])
        torch.cuda.synchronize()
        print(json.dumps({"pmc_run": True, "copy_bytes": 256 << 20, "steps": args.steps}))
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step_eager = e0.elapsed_time(e1) / args.steps
    wall_ms_step = (t1 - t0) * 1e3 / args.steps

    # The same step captured once as a HIP graph and replayed: identical
    # kernels, no host launch gaps.  Its outputs are checked bitwise against
    # an eager step before its time is used.
    ms_step, graph_ok = ms_step_eager, None
    try:
        outs = {}

        def step_out():
            qb.qlora_quantize_nf4_dq(W, check_finite=False, out=q)
            _, T = qb.qlora_linear_fwd(X, q, A, B, s, ws=ws_f, out=Y)
            outs["g"] = qb.qlora_linear_bwd(dY, X, T, q, A, B, s, ws=ws_b)

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_out()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_graph = e0.elapsed_time(e1) / args.steps
        got = [Y.clone()] + [t.clone() for t in outs["g"]]
        step_out()
        torch.cuda.synchronize()
        want = [Y] + list(outs["g"])
        graph_ok = all(torch.equal(a, b) for a, b in zip(got, want))
        if graph_ok:
            ms_step = ms_graph
    except Exception as e:  # capture unsupported: the eager figure stands
        print(f"step graph capture failed: {e}", file=sys.stderr)

    # Kernel time per class from one instrumented eager pass of `steps` steps
    # (start/stop events recorded at the dispatches' own begin and end), after
    # a warm-up pass that fills the library's event pool: the breakdown and
    # the dominant kernel's launch time below both come from this pass.
    per_class = instrumented_pass(qb, torch, step, args.steps)
    gemm_ms, gemm_n = per_class["main_gemm"]
    nb = args.steps

    flops = step_flops(M, d, o, r)
    value = flops / (ms_step * 1e-3) / 1e12

    # dominant kernel: the fused main product (forward Y and backward dX)
    gemm_flop_per_launch = (2 * M * d * o + 2 * M * r * o + 2 * M * o * d + 2 * M * r * d) / 2
    gemm_avg_ms = gemm_ms / max(gemm_n, 1)
    achieved = gemm_flop_per_launch / (gemm_avg_ms * 1e-3) / 1e12
    kept = pmc_entry("k_qgemm", wl.name)
    traffic = None if kept is None else kept["hbm_bytes_per_dispatch"]
    roofline = {"bound": "mfma", "kernel": "k_qgemm fused NF4 dequant-GEMM 512x128 (Y = X·Ŵ + sT·B, dX = dY·Ŵᵀ + sU·Aᵀ)",
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "flop_per_launch": gemm_flop_per_launch, "avg_launch_us": round(gemm_avg_ms * 1e3, 2),
                "launches": gemm_n, "timing": "kernel begin/end events of the instrumented pass"}
    if os.path.exists(MFMA_FILE):
        with open(MFMA_FILE) as f:
            mf = json.load(f)
        if mf.get("source_hash") == source_hash(PMC_KERNELS["k_qgemm"][1]):
            roofline["mfma_busy_frac"] = mf.get("mfma_busy_frac")

    roofline["context_plain_bf16_gemm"] = plain_gemm_reference(torch, X, W, args.steps)

    breakdown = {name: {"ms_per_step": round(ms / nb, 4), "launches_per_step": n / nb}
                 for name, (ms, n) in per_class.items() if n}

    decode = None if args.no_decode else bench_decode(args, qb, torch, np, synth, dev)
    blocks = None if args.no_blocks else bench_blocks(qb, torch, synth, dev)
    tiny = None if args.no_tiny else tiny_latency(qb, torch, np, synth, dev)
    formats = format_errors(qb, torch, W)
    merge_res = merge_study(qb, torch, W, q, X, A, B, s)
    optim = optimizer_study(qb, torch, synth, dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, wl, p)

    out = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s (4096 tok) and dequant-GEMV GB/s vs HBM peak",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "timing": "hip_graph" if ms_step is not ms_step_eager else "eager",
        "ms_per_step_eager": round(ms_step_eager, 4), "wall_ms_per_step_eager": round(wall_ms_step, 4),
        "graph_replay_matches_eager": graph_ok,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian, random-init; no datasets or trained weights)",
        "config": {"workload": wl.name, "M": M, "d": d, "o": o, "r": r, "s": s, "w_std": wl.w_std,
                   "step": "quantize NF4+DQ + fwd + bwd (dX, dA, dB)", "flop_per_step": flops,
                   "parallelism": "single GPU"},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "breakdown": breakdown, "decode": decode, "blocks": blocks,
        "tiny_latency": tiny,
        "formats": formats,
        "merge": merge_res, "optimizer": optim,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def instrumented_pass(qb, torch, fn, reps):
    """{class name: (summed kernel ms, calls)} over `reps` calls of fn, every
    kernel class timed at its dispatches (a warm-up pass fills the pool of
    launch events first, so the measured pass creates none)."""
    qb.qlora_timing_begin()
    fn()
    torch.cuda.synchronize()
    qb.qlora_timing_begin()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    qb.qlora_timing_end()
    return {name: qb.qlora_timing_read(k) for name, k in qb.KERNEL_CLASSES.items()}


def _time_decode(qb, torch, sets, one, ys, byts, K_GEMV):
    """Time one MLP pass over every weight set: eager, then as a HIP-graph replay."""
    for layer in sets:
        one(layer)
    torch.cuda.synchronize()
    reps = max(2, 96 // len(sets))
    # kernel time per launch of the dequant-GEMV and of the T planes before it
    cls = instrumented_pass(qb, torch, lambda: [one(layer) for layer in sets], 1)
    gemv_ms, gemv_n = cls["gemv"]
    tdown_ms, tdown_n = cls["adapter"]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # eager: one Python call per projection (host launch cost included)
    e0.record()
    for _ in range(reps):
        for layer in sets:
            one(layer)
    e1.record()
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) * 1e3 / (reps * len(sets))
    # the same launches captured once in a HIP graph and replayed: the GPU time
    us, graph_ok = None, None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for layer in sets:
                one(layer)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * len(sets))
        # every replay leaves the last set's outputs: compare with eager calls
        got = {k: v.clone() for k, v in ys.items()}
        one(sets[-1])
        torch.cuda.synchronize()
        graph_ok = all(torch.equal(got[k], ys[k]) for k in ys)
    except Exception as e:  # capture unsupported: report the eager figure only
        print(f"decode graph capture failed: {e}", file=sys.stderr)
    t = us if (us is not None and graph_ok) else us_eager
    return {"us_per_mlp": round(t, 2), "timing": "hip_graph" if t is us else "eager",
            "us_per_mlp_eager": round(us_eager, 2), "graph_replay_matches_eager": graph_ok,
            "bytes_per_mlp": byts,
            "GBps": round(byts / (t * 1e-6) / 1e9, 1),
            "frac_of_hbm": round(byts / (t * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "gemv_kernel_us": round(gemv_ms * 1e3 / max(gemv_n, 1), 2) if gemv_n else None,
            "gemv_launches_per_mlp": gemv_n / len(sets),
            "t_planes_kernel_us": round(tdown_ms * 1e3 / max(tdown_n, 1), 2) if tdown_n else None}


def decode_setup(args, qb, torch, np, synth, dev):
    """(workload, weight sets, adapters, bf16 upload helper) of the decode
    measurement: args.decode_sets independent sets of quantized gate, up and
    down weights."""
    wl = synth.WORKLOADS["decode_mlp_7b"]
    # weight set 0 is the seeded host recipe; the other sets (only there to
    # defeat caching) come from a seeded device generator
    gen = torch.Generator(device=dev)
    gen.manual_seed(20251203)
    sets = []
    for k in range(args.decode_sets):
        layer = []
        for p in wl.projs:
            if k == 0:
                Wd = torch.from_numpy(synth.normal_f32((p.o, p.d), wl.w_std,
                                                       [wl.wid, synth.PROJ_IDS[p.name], synth.T_W])).to(dev)
            else:
                Wd = torch.empty((p.o, p.d), dtype=torch.float32, device=dev)
                Wd.normal_(0.0, wl.w_std, generator=gen)
            layer.append((p, qb.qlora_quantize_nf4_dq(Wd, check_finite=False)))
            del Wd
        sets.append(layer)
    def bfd(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    adapters = {p.name: (bfd(synth.normal_bf16((p.d, wl.r), 0.02, [wl.wid, synth.PROJ_IDS[p.name], synth.T_A])),
                         bfd(synth.normal_bf16((wl.r, p.o), 0.02, [wl.wid, synth.PROJ_IDS[p.name], synth.T_B])))
                for p in wl.projs}
    return wl, sets, adapters, bfd


def decode_inputs(qb, torch, np, synth, dev, wl, M):
    xs = {p.name: torch.from_numpy(synth.normal_bf16((M, p.d), 1.0, [wl.wid, synth.PROJ_IDS[p.name],
                                                                     synth.T_X]).view(np.int16))
          .view(torch.bfloat16).to(dev) for p in wl.projs}
    ys = {p.name: torch.empty((M, p.o), dtype=torch.bfloat16, device=dev) for p in wl.projs}
    return xs, ys


def gemv_launch_bytes(qb, p, M, r):
    """Algorithmic bytes one few-token dequant-GEMV launch moves: the 4-bit
    codes, 8-bit scales and fp32 steps of the weight, X, B and Y (the T
    planes it sums are a few KB and not counted)."""
    c, s8, s2 = qb.qlora_quant_sizes(p.o * p.d)
    return c + s8 + s2 + 2 * (M * p.d + r * p.o + M * p.o)


def bench_decode(args, qb, torch, np, synth, dev):
    """Few-token forward on 7B-style gate/up/down NF4 weights, rank 16, cycling
    independent weight sets so the 256 MB MALL cannot hold them."""
    wl, sets, adapters, bfd = decode_setup(args, qb, torch, np, synth, dev)
    res = {}
    ws = qb.Workspace()
    for M in (1, 4, 16):
        xs, ys = decode_inputs(qb, torch, np, synth, dev, wl, M)
        byts = 0
        for p in wl.projs:
            c, s8, s2 = qb.qlora_quant_sizes(p.o * p.d)
            byts += c + s8 + s2 + 2 * (p.d * wl.r + wl.r * p.o + M * p.d + M * p.o)

        def one(layer):
            for p, qw in layer:
                A, B = adapters[p.name]
                qb.qlora_linear_fwd(xs[p.name], qw, A, B, wl.s, want_T=False, ws=ws, out=ys[p.name])

        res[f"M{M}"] = _time_decode(qb, torch, sets, one, ys, byts, K_GEMV=qb.K_GEMV)
        if M == 1:
            roofline = decode_roofline(qb, wl, res["M1"])

    # gate and up read the same input in an MLP: run them as one projection of
    # 22016 rows with the two adapters side by side (A = [A_gate | A_up], B
    # block-diagonal), which gives the same outputs with two launches fewer
    P = {p.name: p for p in wl.projs}
    g_, u_, dn_ = P["gate"], P["up"], P["down"]
    fused_sets = []
    for layer in sets:
        qs = {p.name: qw for p, qw in layer}
        fused_sets.append((qb.qlora_stack_rows([qs["gate"], qs["up"]]), qs["down"]))
    Ag, Bg = adapters["gate"]
    Au, Bu = adapters["up"]
    A_gu = torch.cat([Ag, Au], 1).contiguous()
    B_gu = torch.zeros((2 * wl.r, g_.o + u_.o), dtype=torch.bfloat16, device=dev)
    B_gu[:wl.r, :g_.o] = Bg
    B_gu[wl.r:, g_.o:] = Bu
    for M in (1, 4, 16):
        x = torch.from_numpy(synth.normal_bf16((M, g_.d), 1.0, [wl.wid, synth.PROJ_IDS["gate"], synth.T_X])
                             .view(np.int16)).view(torch.bfloat16).to(dev)
        h = torch.from_numpy(synth.normal_bf16((M, dn_.d), 1.0, [wl.wid, synth.PROJ_IDS["down"], synth.T_X])
                             .view(np.int16)).view(torch.bfloat16).to(dev)
        ys = {"gate_up": torch.empty((M, g_.o + u_.o), dtype=torch.bfloat16, device=dev),
              "down": torch.empty((M, dn_.o), dtype=torch.bfloat16, device=dev)}
        byts = 0
        for p in wl.projs:
            c, s8, s2 = qb.qlora_quant_sizes(p.o * p.d)
            byts += c + s8 + s2 + 2 * (p.d * wl.r + wl.r * p.o + M * p.o)
        byts += 2 * M * (g_.d + dn_.d)               # x once for gate and up, h for down
        Ad, Bd = adapters["down"]

        def one_fused(layer):
            qgu, qd = layer
            qb.qlora_linear_fwd(x, qgu, A_gu, B_gu, wl.s, want_T=False, ws=ws, out=ys["gate_up"])
            qb.qlora_linear_fwd(h, qd, Ad, Bd, wl.s, want_T=False, ws=ws, out=ys["down"])

        res[f"M{M}_gate_up_fused"] = _time_decode(qb, torch, fused_sets, one_fused, ys, byts, K_GEMV=qb.K_GEMV)

    # one adapter per token: 16 tokens on 16 different rank-16 adapters per projection
    M, n_ad = 16, 16
    multi_ad = {p.name: (bfd(synth.normal_bf16((n_ad, p.d, wl.r), 0.02, [wl.wid, synth.PROJ_IDS[p.name], synth.T_A_STACK])),
                         bfd(synth.normal_bf16((n_ad, wl.r, p.o), 0.02, [wl.wid, synth.PROJ_IDS[p.name], synth.T_B_STACK])))
                for p in wl.projs}
    s_list = [wl.s] * n_ad
    idx = torch.arange(M, dtype=torch.int32, device=dev)
    xs = {p.name: torch.from_numpy(synth.normal_bf16((M, p.d), 1.0, [wl.wid, synth.PROJ_IDS[p.name],
                                                                     synth.T_X]).view(np.int16))
          .view(torch.bfloat16).to(dev) for p in wl.projs}
    ys = {p.name: torch.empty((M, p.o), dtype=torch.bfloat16, device=dev) for p in wl.projs}
    byts = 0
    for p in wl.projs:
        c, s8, s2 = qb.qlora_quant_sizes(p.o * p.d)
        byts += c + s8 + s2 + 2 * (n_ad * (p.d * wl.r + wl.r * p.o) + M * p.d + M * p.o)

    def one_multi(layer):
        for p, qw in layer:
            A, B = multi_ad[p.name]
            qb.qlora_linear_fwd_multi(xs[p.name], qw, A, B, s_list, idx, ws=ws, out=ys[p.name])

    res["M16_16_adapters"] = _time_decode(qb, torch, sets, one_multi, ys, byts, K_GEMV=qb.K_GEMV)
    return {"workload": "decode_mlp_7b: gate/up 4096->11008, down 11008->4096, r=16, fwd only; "
                        "M*_gate_up_fused: gate and up share their input and run as one 22016-row "
                        "projection (adapters side by side, B block-diagonal); "
                        "M16_16_adapters: one adapter per token (16 adapters per projection)",
            "weight_sets_cycled": len(sets), "peak_GBps": PEAK_HBM_GBPS, "roofline": roofline, **res}


def plain_gemm_reference(torch, X, W, reps):
    """Context for the roofline, not a target: the same-shape product X·Wᵀ as a
    plain bf16 GEMM through torch (hipBLASLt on this system), no dequantization
    and no adapter, timed with events around `reps` back-to-back launches."""
    Wb = W.to(torch.bfloat16)
    y = torch.nn.functional.linear(X, Wb)
    for _ in range(3):
        torch.nn.functional.linear(X, Wb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.nn.functional.linear(X, Wb)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    M, d = X.shape
    o = Wb.shape[0]
    tf = 2 * M * d * o / (us * 1e-6) / 1e12
    del Wb, y
    return {"op": "torch.nn.functional.linear, bf16 (hipBLASLt)", "shape_MNK": [M, o, d],
            "us": round(us, 2), "TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def decode_roofline(qb, wl, m1):
    """HBM roofline of the few-token dequant-GEMV at 1 token: algorithmic
    bytes per launch (averaged over gate, up and down) over its average
    kernel time from the instrumented pass; traffic from the kept counters."""
    per_launch = sum(gemv_launch_bytes(qb, p, 1, wl.r) for p in wl.projs) / len(wl.projs)
    us = m1["gemv_kernel_us"]
    achieved = per_launch / (us * 1e-6) / 1e9
    traffic = pmc_entry("k_gemv<1>", wl.name)
    tplanes = pmc_entry("k_lora_down_small", wl.name)
    return {"bound": "hbm", "kernel": "k_gemv<1> fused NF4 dequant-GEMV, 1 token (gate, up, down)",
            "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": None if traffic is None else traffic["hbm_bytes_per_dispatch"],
            "bytes_per_launch": round(per_launch), "avg_launch_us": us,
            "t_planes_traffic": None if tplanes is None else tplanes["hbm_bytes_per_dispatch"]}


def bench_blocks(qb, torch, synth, dev, steps=5, warmup=2):
    """Forward + backward over every projection of a 7B-style block (4096
    tokens) and a 65B-style block (2048 tokens), rank 64, s = 2, and the
    blockwise NF4 + double-quant of all seven 65B-style tensors.  Weights come
    from a seeded device generator with the workload's standard deviation;
    activations and adapters likewise.  Eager launches timed with events (a
    step is milliseconds, so launch cost is small)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name in ("block_7b", "block_65b"):
        wl = synth.WORKLOADS[name]
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + wl.wid)
        M, r, s = wl.M, wl.r, wl.s
        layers, flops, quant_bytes, n_total = [], 0, 0, 0
        Ws = []
        for p in wl.projs:
            W = torch.empty((p.o, p.d), dtype=torch.float32, device=dev).normal_(0.0, wl.w_std, generator=gen)
            Ws.append(W)
            n_total += W.numel()
            c, s8, s2 = qb.qlora_quant_sizes(W.numel())
            quant_bytes += 4 * W.numel() + c + s8 + s2
        qs = [qb.qlora_quantize_nf4_dq(W, check_finite=False) for W in Ws]
        torch.cuda.synchronize()
        res = {"M": M, "r": r, "s": s, "projections": [f"{p.name} {p.o}x{p.d}" for p in wl.projs]}
        if name == "block_65b":
            # quantize of all seven tensors: fp32 read once, codes and scales written
            for _ in range(2):
                for W, q in zip(Ws, qs):
                    qb.qlora_quantize_nf4_dq(W, check_finite=False, out=q)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                for W, q in zip(Ws, qs):
                    qb.qlora_quantize_nf4_dq(W, check_finite=False, out=q)
            e1.record()
            torch.cuda.synchronize()
            us_sep = e0.elapsed_time(e1) * 1e3 / steps
            # the same seven tensors in one grouped launch
            for _ in range(2):
                qb.qlora_quantize_nf4_dq_grouped(Ws, check_finite=False, outs=qs)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                qb.qlora_quantize_nf4_dq_grouped(Ws, check_finite=False, outs=qs)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            res["quantize_all"] = {"us": round(us, 1), "launch": "one grouped launch",
                                   "us_one_launch_per_tensor": round(us_sep, 1),
                                   "weights": n_total, "bytes": quant_bytes,
                                   "GBps": round(quant_bytes / (us * 1e-6) / 1e9, 1),
                                   "frac_of_hbm": round(quant_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        del Ws
        ws_f, ws_b = qb.Workspace(), qb.Workspace()
        for p, q in zip(wl.projs, qs):
            X = torch.empty((M, p.d), device=dev).normal_(0.0, 1.0, generator=gen).to(torch.bfloat16)
            dY = torch.empty((M, p.o), device=dev).normal_(0.0, 1.0, generator=gen).to(torch.bfloat16)
            A = torch.empty((p.d, r), device=dev).normal_(0.0, 0.02, generator=gen).to(torch.bfloat16)
            B = torch.empty((r, p.o), device=dev).normal_(0.0, 0.02, generator=gen).to(torch.bfloat16)
            Y = torch.empty((M, p.o), dtype=torch.bfloat16, device=dev)
            layers.append((q, X, dY, A, B, Y))
            flops += step_flops(M, p.d, p.o, r)

        def step():
            for q, X, dY, A, B, Y in layers:
                _, T = qb.qlora_linear_fwd(X, q, A, B, s, ws=ws_f, out=Y)
                qb.qlora_linear_bwd(dY, X, T, q, A, B, s, ws=ws_b)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        # the fused GEMM's share, from a separate step with per-launch events
        qb.qlora_timing_begin([qb.K_MAIN_GEMM])
        step()
        torch.cuda.synchronize()
        qb.qlora_timing_end()
        gms, gn = qb.qlora_timing_read(qb.K_MAIN_GEMM)
        res.update({"step": "fwd + bwd (dX, dA, dB) of every projection", "flop_per_step": flops,
                    "ms_per_step": round(ms, 4), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
                    "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "main_gemm_ms_per_step": round(gms, 4), "main_gemm_launches_per_step": gn})
        out[name] = res
        del layers, qs
        torch.cuda.empty_cache()
    return out


def optimizer_study(qb, torch, synth, dev):
    """AdamW over the rank-64 adapters of one 65B-style block (7 projections),
    states in HBM, then paged from pinned host memory through a 64 MiB pool."""
    wl = synth.WORKLOADS["block_65b"]
    n = sum(wl.r * (p.d + p.o) for p in wl.projs)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    p = torch.empty(n, device=dev).normal_(0.0, 0.02, generator=gen)
    g = torch.empty(n, device=dev).normal_(0.0, 1e-3, generator=gen).to(torch.bfloat16)
    p16 = torch.empty(n, dtype=torch.bfloat16, device=dev)
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn(1)
        torch.cuda.synchronize()
        e0.record()
        for t in range(reps):
            fn(t + 2)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    us_dev = timed(lambda t: qb.qlora_adamw_step(p, p16, g, m, v, t), 20)
    mh, vh = qb.pinned_state(n), qb.pinned_state(n)
    pool = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    us_paged = timed(lambda t: qb.qlora_paged_adamw_step(p, p16, g, mh, vh, t, pool), 5)
    # host-link reference: plain pinned copies of the same state bytes, each way
    hbuf = torch.empty(2 * n, dtype=torch.float32, pin_memory=True)
    dbuf = torch.empty(2 * n, dtype=torch.float32, device=dev)
    us_h2d = timed(lambda t: dbuf.copy_(hbuf, non_blocking=True), 5)
    us_d2h = timed(lambda t: hbuf.copy_(dbuf, non_blocking=True), 5)
    st_bytes = 8 * n                                   # m and v, fp32, one way
    return {
        "workload": f"AdamW on the rank-{wl.r} adapters of one 65B-style block: {n} fp32 parameters",
        "device_states": {"us_per_step": round(us_dev, 2), "bytes_per_param": 28,
                          "GBps": round(28 * n / (us_dev * 1e-6) / 1e9, 1),
                          "frac_of_hbm": round(28 * n / (us_dev * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)},
        "paged_states": {"us_per_step": round(us_paged, 2), "pool_MiB": 64,
                         "host_link_GBps_each_way": round(st_bytes / (us_paged * 1e-6) / 1e9, 1),
                         "copy_reference_us": {"h2d": round(us_h2d, 1), "d2h": round(us_d2h, 1)},
                         "frac_of_sequential_copies": round((us_h2d + us_d2h) / us_paged, 3)},
        "device_state_bytes_saved": 8 * n,
    }


def tiny_latency(qb, torch, np, synth, dev, reps=200):
    """Latency of one step (quantize + fwd + bwd) of the single 128×128
    linear (8 tokens, rank 8): eager, and as a HIP-graph replay."""
    wl = synth.WORKLOADS["tiny_128"]
    p = wl.projs[0]
    W_h, X_h, A_h, B_h, dY_h = synth.layer_inputs(wl, p)
    bf = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    W = torch.from_numpy(W_h).to(dev)
    X, A, B, dY = bf(X_h), bf(A_h), bf(B_h), bf(dY_h)
    q = qb.qlora_quantize_nf4_dq(W)
    Y = torch.empty((wl.M, p.o), dtype=torch.bfloat16, device=dev)
    ws_f, ws_b = qb.Workspace(), qb.Workspace()

    def step():
        qb.qlora_quantize_nf4_dq(W, check_finite=False, out=q)
        _, T = qb.qlora_linear_fwd(X, q, A, B, wl.s, ws=ws_f, out=Y)
        qb.qlora_linear_bwd(dY, X, T, q, A, B, wl.s, ws=ws_b)

    for _ in range(10):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        step()
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) * 1e3 / reps
    res = {"workload": "tiny_128: 128x128 linear, 8 tokens, r = 8, quantize + fwd + bwd",
           "us_per_step_eager": round(eager, 2)}
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res["us_per_step_graph"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    except Exception as e:  # capture unsupported: the eager figure stands
        print(f"tiny graph capture failed: {e}", file=sys.stderr)
    return res


def merge_study(qb, torch, W, q, X, A, B, s):
    """Merge the adapter into the base, quantize again, and measure how far the
    merged 4-bit layer's output moves from the unmerged layer's output."""
    o, d = q.shape
    r = A.shape[1]
    for _ in range(3):
        Wm = qb.qlora_merge_adapter(q, A, B, s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        qb.qlora_merge_adapter(q, A, B, s, out=Wm)
    e1.record()
    torch.cuda.synchronize()
    us_merge = e0.elapsed_time(e1) * 1e3 / reps
    q2 = qb.qlora_quantize_nf4_dq(Wm, check_finite=False)
    e0.record()
    for _ in range(reps):
        qb.qlora_quantize_nf4_dq(Wm, check_finite=False, out=q2)
    e1.record()
    torch.cuda.synchronize()
    us_requant = e0.elapsed_time(e1) * 1e3 / reps
    Y_unmerged, _ = qb.qlora_linear_fwd(X, q, A, B, s, want_T=False)
    Y_merged, _ = qb.qlora_linear_fwd(X, q2, None, None, 0.0, want_T=False)
    Y_base, _ = qb.qlora_linear_fwd(X, q, None, None, 0.0, want_T=False)
    Y_fp = X.double() @ W.double().T                       # unquantized base, fp64 reference
    nrm = lambda t: float(torch.linalg.vector_norm(t.double()))   # noqa: E731
    yu = Y_unmerged.double()
    codes_changed = float((q2.codes != q.codes).double().mean())
    flop = 2.0 * o * d * r
    return {
        "workload": f"merge rank-{r} adapter into the {o}x{d} base, then NF4 + DQ again",
        "us_merge": round(us_merge, 2), "us_requantize": round(us_requant, 2),
        "merge_roofline": {"bound": "alu", "achieved": round(flop / (us_merge * 1e-6) / 1e12, 2),
                           "peak": 157.3, "unit": "TFLOP/s (fp32 FMA)",
                           "frac": round(flop / (us_merge * 1e-6) / 1e12 / 157.3, 4),
                           "hbm_GBps": round(o * d * (0.515869 + 4) / (us_merge * 1e-6) / 1e9, 1)},
        "code_bytes_changed": round(codes_changed, 4),
        "rel_change_merged_vs_unmerged": nrm(Y_merged.double() - yu) / nrm(yu),
        "rel_adapter_term": nrm(yu - Y_base.double()) / nrm(yu),
        "rel_base_quantization_error": nrm(Y_base.double() - Y_fp) / nrm(Y_fp),
    }


def format_errors(qb, torch, W):
    """Quantization error of each 4-bit table on the workload's weight, all
    on the GPU: blockwise 4-bit + double quantization, dequant to fp32, mean
    squared error against W (and over W's variance)."""
    var = float(W.double().var())
    out = {}
    for fmt in qb.FORMATS:
        q = qb.qlora_quantize_nf4_dq(W, check_finite=False, fmt=fmt)
        mse = float(((qb.qlora_dequant(q).double() - W.double()) ** 2).mean())
        out[fmt] = {"mse": mse, "mse_over_var": round(mse / var, 6)}
    # the second-level variants centred on the tensor mean, with NF4 codes
    for v in ("int8_mean", "fp8_mean"):
        q = qb.qlora_quantize_nf4_dq(W, check_finite=False, dq=v)
        mse = float(((qb.qlora_dequant(q).double() - W.double()) ** 2).mean())
        out["nf4+" + v] = {"mse": mse, "mse_over_var": round(mse / var, 6)}
    return out


def cpu_baseline(args, wl, p):
    """The oracle as it stands (fp64 NumPy), on the host, on the same workload."""
    import numpy as np

    import synth
    from oracle import linear, nf4
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info())
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    W, X, A, B, dY = synth.layer_inputs(wl, p)
    f = nf4.bf16_bits_to_f64
    Xf, Af, Bf, dYf = f(X), f(A), f(B), f(dY)
    times = []
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < args.cpu_seconds or len(times) < 2:
        t = time.perf_counter()
        c, s8, s2 = nf4.quantize_chunked(W.ravel())
        Wh = f(nf4.dequant_bf16_bits(c, s8, s2, W.size)).reshape(W.shape)
        linear.forward(Xf, Wh, Af, Bf, wl.s)
        linear.backward(dYf, Xf, Wh, Af, Bf, wl.s)
        times.append(time.perf_counter() - t)
        if len(times) >= 20:
            break
    med = statistics.median(times)
    M, d, o, r = wl.M, p.d, p.o, wl.r
    return {"value": round(step_flops(M, d, o, r) / med / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "s_per_step": round(med, 3), "steps_timed": len(times),
            "sample": f"full {wl.name} step (quantize+dequant+fwd+bwd, fp64 NumPy/OpenBLAS), "
                      f"median of {len(times)}"}


if __name__ == "__main__":
    main()
