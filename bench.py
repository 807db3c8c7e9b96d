#!/usr/bin/env python3
"""Sparse-BitLinear 6:8 forward + Dual-STE backward throughput on one MI355X.

Workload (default): the 3B-like decoder-layer linears q/o 2048->2048, k/v
2048->256, gate/up 2048->11008, down 11008->2048, 16 x 2048 = 32768 tokens,
bf16 master weights ~ N(0, 0.02), Student-t(4) activations, dY ~ N(0, 1),
all seeded synthetic data already resident in HBM.

One step = sbl_quant_mask_pack_batch (gamma, 6:8 mask and codes of all 7 linears in one call,
recomputed every step), then for each of the 7 linears, in order:
  sbl_act_quant       (per-token absmax int8)
  sbl_forward         (int8 MFMA, y bf16)
  sbl_backward        (dX and dW in one call: bf16 MFMA, dX bf16, dW float32 dense;
                       the dX product leaves dY^T behind for dW)
Metric: tokens per second of whole steps.  Prints one JSON line; after the timed steps the default
workload also counts the backward call's HBM bytes with two rocprofv3 --pmc passes run as child
processes (--no-live-traffic skips them).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
       python bench.py --workload 0     (one 256x256 linear, 64 tokens, fwd+bwd: launch-bound, timed as
                                         replays of the step captured in a HIP graph; --timing eager for launches)
       python bench.py --workload 1     (0.5B-like up-projection 896->4864, 512 tokens, forward, 8/6/4/2:8;
                                         graph replays as for workload 0)
       python bench.py --workload 2     (1.5B-like linears, 8192 tokens, fwd+bwd)
       python bench.py --workload 4     (decode: per-layer latency at 1/8/64 tokens, 6/4/2:8)
       python bench.py --peaks          (measured ceilings only: matrix instructions on registers, HBM read)
       python bench.py --variants       (every N of N:8, 2:4, the ablations, AdamW + repack, norm + act quant,
                                         2:8 forward dense vs sparse matrix instruction)
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

HBM_PEAK_GBS = 8000.0

# HBM bytes per sbl_backward(dX + dW) call on the default workload (FETCH_SIZE x 2.000 +
# WRITE_SIZE, scale factors from a plain 1 GiB copy), averaged over the 7 linears; measured with
# rocprofv3 --pmc for the backward kernel sources whose hash (code without comments) is given
# (profiles/traffic_backward_3b_32768tok.md).
BWD_TRAFFIC_BYTES = 1.937e9
BWD_TRAFFIC_SRC_SHA = "723f0d7b93da5309"
INT8_PEAK_TOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="index into sbl_inputs.WORKLOADS (2, 3, or 4 = decode)")
    ap.add_argument("--n-keep", type=int, default=6)
    ap.add_argument("--pack", choices=("batch", "single"), default="batch",
                    help="pack all linears in one batched call (default) or one call per linear")
    ap.add_argument("--cpu-tokens", type=int, default=12288,
                    help="token sample for the oracle baseline (about 10 s of host work on the default workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-fuse-max", type=int, default=None,
                    help="decode: largest T * d_in of a group that takes the fused launch (default: wherever supported)")
    ap.add_argument("--breakdown", action="store_true", help="print the per-linear breakdown to stderr")
    ap.add_argument("--variants", action="store_true",
                    help="N:M patterns and ablations: quant/mask/pack per pattern and mask-without-grad on the "
                         "3B-like matrices (one JSON line)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the ceilings (int8 and bf16 matrix instructions on register operands, "
                         "HBM read and copy) and print them as one JSON line")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured ceilings in the other modes")
    ap.add_argument("--launch-floor", action="store_true",
                    help="only time one launch of the library's streaming-read kernel per size (1 KB to 128 MB, "
                         "in a captured graph over distinct buffers) and print one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (scale reference for HBM byte counters)")
    ap.add_argument("--no-live-traffic", action="store_true",
                    help="default workload: skip the live HBM byte count of the backward call (two rocprofv3 "
                         "--pmc passes and their copy calibration, run as child processes after the timed "
                         "steps) and report the figure of the committed profile instead")
    ap.add_argument("--timing", choices=("auto", "eager", "graph"), default="auto",
                    help="how steps are timed: eager launches, or replays of the step captured in one HIP graph "
                         "(auto: graph for the launch-bound workloads 0 and 1, whose kernels run for a few "
                         "microseconds each, eager otherwise)")
    return ap.parse_args()


# Workloads whose step is a handful of launches of a few microseconds each: eager timing would
# measure the host's enqueue rate, so their steps are timed as replays of a captured graph (how a
# training or serving loop at these sizes would run them), the eager figure reported beside it.
# GRAPH_COPIES steps (or calls, for the per-call figures) go into one graph, back to back, so that
# the fixed cost of a graph launch is spread over them.
LAUNCH_BOUND_WORKLOADS = (0, 1)
GRAPH_COPIES = 10


def use_graph(args) -> bool:
    return args.timing == "graph" or (args.timing == "auto" and args.workload in LAUNCH_BOUND_WORKLOADS)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the operator has no multi-GPU path here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparsity_sparse_bitlinear_amd as sbl
    from sbl_inputs import WORKLOADS, activation, grad_out, weight

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        # 1 GiB read + 1 GiB written per copy, float32
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print("copy calibration done", flush=True)
        return
    if args.peaks:
        print(json.dumps({"metric": "measured ceilings", "n_gpus": 1, **measured_peaks()}), flush=True)
        return
    if args.launch_floor:
        sizes = [1 << 14, 1 << 20, 2 << 20, 4 << 20, 8 << 20, 11272192, 16 << 20, 32 << 20, 64 << 20, 128 << 20]
        rows = [{"bytes": n, "us_per_launch": round(read_floor_us(n), 3)} for n in sizes]
        for r in rows:
            r["GBps"] = round(r["bytes"] / r["us_per_launch"] / 1e3, 1)
        print(json.dumps({"metric": "time of one dependent launch of the streaming-read kernel (captured graph)",
                          "unit": "us", "n_gpus": 1, "results": rows}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.variants:
        run_variants(args, wl)
        return
    if not wl.backward and len(wl.T) > 1:
        run_decode(args, wl)
        return
    if not wl.backward:
        run_forward_sweep(args, wl)
        return
    if not wl.backward or len(wl.T) != 1:
        print(f"workload {args.workload} is not a single-T fwd+bwd training workload", file=sys.stderr)
        sys.exit(2)
    T = wl.T[0]
    n_keep = args.n_keep
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    t_gen = time.time()
    layers = []
    for mi, L in enumerate(wl.linears):
        d_out, d_in = L.d_out, L.d_in
        W = up(weight(wl.cfg, mi, d_out, d_in))
        x = up(activation(wl.cfg, mi, T, d_in, dist=wl.act_dist, outlier_frac=wl.outlier_frac))
        dY = up(grad_out(wl.cfg, mi, T, d_out))
        layers.append(dict(
            name=L.name, d_out=d_out, d_in=d_in, W=W, x=x, dY=dY,
            codes=torch.empty((d_out, d_in // 8), dtype=torch.int16, device=dev),
            mask=torch.empty((d_out, d_in // 8), dtype=torch.uint8, device=dev),
            gamma=torch.empty((1,), dtype=torch.float32, device=dev),
            x_q=torch.empty((T, d_in), dtype=torch.int8, device=dev),
            absmax=torch.empty((T,), dtype=torch.float32, device=dev),
            y=torch.empty((T, d_out), dtype=torch.bfloat16, device=dev),
            dX=torch.empty((T, d_in), dtype=torch.bfloat16, device=dev),
            dW=torch.empty((d_out, d_in), dtype=torch.float32, device=dev),
            bws=torch.empty((max(16, sbl.backward_workspace_size(T, d_in, d_out, sbl.BWD_DX | sbl.BWD_DW)),),
                            dtype=torch.uint8, device=dev),
        ))
    qws = torch.empty((max(16, sbl.quant_batch_workspace_size([(L["d_out"], L["d_in"]) for L in layers])),),
                      dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    parts = ("quant", "act", "fwd", "bwd")

    def step(events=None):
        # the packing of every linear in one batched call (three launches), then each linear
        if args.pack == "batch":
            if events is not None:
                events[0][0].record()
            sbl.quant_mask_pack_batch([Lr["W"] for Lr in layers], n_keep, codes=[Lr["codes"] for Lr in layers],
                                      masks=[Lr["mask"] for Lr in layers], gammas=[Lr["gamma"] for Lr in layers],
                                      workspace=qws)
        for li, Lr in enumerate(layers):
            def mark(k):
                if events is not None:
                    events[li][k].record()
            if args.pack == "single":
                mark(0)
                sbl.quant_mask_pack(Lr["W"], n_keep, codes=Lr["codes"], mask=Lr["mask"], gamma=Lr["gamma"],
                                    workspace=qws)
            elif li > 0:
                mark(0)                 # the batch's time is counted once, on the first linear
            mark(1)
            sbl.act_quant(Lr["x"], x_q=Lr["x_q"], absmax=Lr["absmax"])
            mark(2)
            sbl.forward(Lr["codes"], Lr["gamma"], Lr["x_q"], Lr["absmax"], out_dtype=sbl.BF16, y=Lr["y"])
            mark(3)
            sbl.backward(Lr["codes"], Lr["gamma"], Lr["x_q"], Lr["absmax"], Lr["dY"], dx_dtype=sbl.BF16,
                         dX=Lr["dX"], dW=Lr["dW"], workspace=Lr["bws"])
            mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region 1: plain steps, bracketed by synchronize (one process: no barrier needed).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed
    eager_ms_per_step = ms_per_step
    graph = use_graph(args)
    if graph:
        # GRAPH_COPIES whole steps captured back to back and replayed (every kernel of every call
        # runs in each copy)
        ms_per_step = graph_us(step, reps=max(args.steps, 20), warmup=args.warmup, copies=GRAPH_COPIES) / 1e3
        tokens_per_s = T / (ms_per_step * 1e-3)

    # Timed region 2: the same steps with HIP events between the calls (same stream), for the
    # per-kernel durations behind the roofline figures.
    # All steps are enqueued before the one synchronization, so no step starts on an idle GPU
    # waiting for the host (which would count the host's enqueue time in the first call).
    sums = np.zeros((len(layers), len(parts)))
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in layers]
           for _ in range(args.steps)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    for ev in evs:
        for li in range(len(layers)):
            for k in range(len(parts)):
                sums[li, k] += ev[li][k].elapsed_time(ev[li][k + 1])
    per_launch_ms = sums / args.steps          # [layer, part]
    if graph:
        # per call: GRAPH_COPIES copies of the call alone captured in a graph and replayed (events
        # between eager launches would time the host's enqueue gaps)
        for li, Lr in enumerate(layers):
            if args.pack == "single":
                quant = lambda Lr=Lr: sbl.quant_mask_pack(Lr["W"], n_keep, codes=Lr["codes"], mask=Lr["mask"],
                                                          gamma=Lr["gamma"], workspace=qws)
            elif li == 0:
                quant = lambda: sbl.quant_mask_pack_batch([Lq["W"] for Lq in layers], n_keep,
                                                          codes=[Lq["codes"] for Lq in layers],
                                                          masks=[Lq["mask"] for Lq in layers],
                                                          gammas=[Lq["gamma"] for Lq in layers], workspace=qws)
            else:
                quant = None  # the batch's time is counted once, on the first linear
            calls = [
                quant,
                lambda Lr=Lr: sbl.act_quant(Lr["x"], x_q=Lr["x_q"], absmax=Lr["absmax"]),
                lambda Lr=Lr: sbl.forward(Lr["codes"], Lr["gamma"], Lr["x_q"], Lr["absmax"], out_dtype=sbl.BF16,
                                          y=Lr["y"]),
                lambda Lr=Lr: sbl.backward(Lr["codes"], Lr["gamma"], Lr["x_q"], Lr["absmax"], Lr["dY"],
                                           dx_dtype=sbl.BF16, dX=Lr["dX"], dW=Lr["dW"], workspace=Lr["bws"]),
            ]
            for k, c in enumerate(calls):
                per_launch_ms[li, k] = 0.0 if c is None else graph_us(c, reps=max(args.steps, 20), warmup=args.warmup,
                                                                       copies=GRAPH_COPIES) / 1e3

    # Algorithmic work per launch (units x per-unit figure).
    work = []
    for Lr in layers:
        d_out, d_in = Lr["d_out"], Lr["d_in"]
        nw = d_out * d_in
        work.append(dict(
            quant=2.375 * nw,                                   # bytes: read W (2) + codes (0.25) + mask (0.125)
            act=3.0 * T * d_in + 4.0 * T,                       # bytes: read x (2), write x_q (1), absmax (4/token)
            fwd=2.0 * T * d_out * d_in * n_keep / 8.0,          # int8 ops on kept weights
            bwd=2.0 * T * d_out * d_in * n_keep / 8.0 + 2.0 * T * d_out * d_in,  # dX on kept weights + dense dW
            fwd_issued=2.0 * T * d_out * d_in,
            bwd_issued=4.0 * T * d_out * d_in,
        ))
    tot_ms = per_launch_ms.sum(axis=0)
    def rate(part):
        return sum(w[part] for w in work) / (tot_ms[parts.index(part)] * 1e-3)
    kernels = {
        "quant_mask_pack": dict(ms=tot_ms[0], GBps=rate("quant") / 1e9, frac_hbm=rate("quant") / 1e9 / HBM_PEAK_GBS),
        "act_quant": dict(ms=tot_ms[1], GBps=rate("act") / 1e9, frac_hbm=rate("act") / 1e9 / HBM_PEAK_GBS),
        "forward_int8": dict(ms=tot_ms[2], TOPs=rate("fwd") / 1e12, frac_int8=rate("fwd") / 1e12 / INT8_PEAK_TOPS,
                             frac_int8_issued=sum(w["fwd_issued"] for w in work) / (tot_ms[2] * 1e-3) / 1e12 / INT8_PEAK_TOPS),
        "backward_bf16": dict(ms=tot_ms[3], TFLOPs=rate("bwd") / 1e12, frac_bf16=rate("bwd") / 1e12 / BF16_PEAK_TFLOPS,
                              frac_bf16_issued=sum(w["bwd_issued"] for w in work) / (tot_ms[3] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS),
    }
    # HIP kernels behind each timed call (the events bracket the whole call)
    gemm_parts = {
        "fwd": ("forward_int8", "TOP/s", INT8_PEAK_TOPS, ["k_fwd_i8_direct<bf16>"]),
        "bwd": ("backward_bf16 (dX + dW)", "TFLOP/s", BF16_PEAK_TFLOPS,
                ["k_codes_t", "k_gemm_nt_bf16<bf16, codes B, writes dY a/127 run-major>",
                 "k_gemm_nt_bf16<f32, run-major A, int8 B>", "k_splitk_reduce (split-K shapes)"]),
    }
    dom = max(gemm_parts, key=lambda p: tot_ms[parts.index(p)])
    dname, dunit, dpeak, dkernels = gemm_parts[dom]
    n_launch = len(layers)
    achieved = sum(w[dom] for w in work) / n_launch / (tot_ms[parts.index(dom)] / n_launch * 1e-3) / 1e12
    traffic, traffic_src = None, None
    if dom == "bwd" and args.workload == 3 and n_keep == 6 and not args.no_live_traffic:
        live = live_traffic(2 * len(layers))  # the child runs one timed and one event-timed step
        if live is not None:
            traffic, traffic_src = live["bytes"], ("rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE over this "
                                                   "workload in this run, copy-calibrated")
    if (traffic is None and dom == "bwd" and args.workload == 3 and n_keep == 6 and BWD_TRAFFIC_BYTES is not None
            and _bwd_sources_sha() == BWD_TRAFFIC_SRC_SHA):
        traffic, traffic_src = BWD_TRAFFIC_BYTES, "committed counter profile of these backward sources"
    if traffic is not None:
        traffic = float(round(traffic, -6))
    roofline = {"bound": "mfma", "kernel": dname, "achieved": round(achieved, 1), "peak": dpeak,
                "unit": dunit, "frac": round(achieved / dpeak, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "traffic_source": traffic_src,
                "launches_per_step": n_launch, "hip_kernels": dkernels,
                "avg_launch_ms": round(tot_ms[parts.index(dom)] / n_launch, 4)}

    # Measured ceilings of this GPU (matrix instructions on register operands, HBM read), beside the
    # datasheet peaks.
    peaks = None if args.no_peaks else measured_peaks()
    if peaks:
        mp = peaks["bf16_TFLOPs"] if dom == "bwd" else peaks["int8_TOPs"]
        roofline["peak_measured"] = mp
        roofline["frac_measured"] = round(achieved / mp, 4)
        kernels["forward_int8"]["frac_int8_measured"] = rate("fwd") / 1e12 / peaks["int8_TOPs"]
        kernels["backward_bf16"]["frac_bf16_measured"] = rate("bwd") / 1e12 / peaks["bf16_TFLOPs"]
        for k, part in (("quant_mask_pack", "quant"), ("act_quant", "act")):
            kernels[k]["frac_hbm_measured"] = rate(part) / 1e9 / peaks["read_GBps"]

    # CPU baseline: the oracle on a bounded sample, on this host's cores.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, T, n_keep, args.cpu_tokens)

    line = {
        "metric": ("Sparse-BitLinear 6:8 fwd+bwd tokens/s at 3B shapes; % int8 MFMA / HBM peak" if args.workload == 3
                   else f"Sparse-BitLinear {n_keep}:8 fwd+bwd tokens/s ({wl.name})"),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 fwd / bf16 bwd (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "n_keep": n_keep, "m": 8,
                   "linears": [f"{Lr['name']} {Lr['d_in']}->{Lr['d_out']}" for Lr in layers],
                   "y_dtype": "bf16", "dx_dtype": "bf16", "dw_dtype": "f32"},
        "roofline": roofline,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": cpu,
        "measured_peaks": peaks,
        "input_gen_s": round(t_gen, 1),
    }
    if graph:
        line["timing"] = (f"graph replay: {GRAPH_COPIES} steps captured back to back in one HIP graph, replayed, "
                          f"time / {GRAPH_COPIES}; per-call figures likewise from {GRAPH_COPIES} copies of each call")
        line["eager_ms_per_step"] = round(eager_ms_per_step, 4)
    if args.breakdown:
        for li, Lr in enumerate(layers):
            print(Lr["name"], " ".join(f"{p}={per_launch_ms[li, k]:.4f}ms" for k, p in enumerate(parts)),
                  file=sys.stderr)
    print(json.dumps(line), flush=True)


def _counter_kib(csv_path: str, pick) -> tuple:
    """Sum of Counter_Value (KiB) over the dispatches whose kernel name `pick` accepts, and their
    count, from a rocprofv3 counter_collection.csv."""
    import csv
    total, n = 0.0, 0
    with open(csv_path, newline="") as fh:
        for row in csv.DictReader(fh):
            if pick(row["Kernel_Name"]):
                total += float(row["Counter_Value"])
                n += 1
    return total, n


def live_traffic(n_calls: int, timeout_s: float = 90.0):
    """HBM bytes per sbl_backward call of the default workload, counted in this run: rocprofv3
    --pmc FETCH_SIZE, then WRITE_SIZE, each over a child `bench.py --steps 1 --warmup 0` (two steps:
    n_calls backward calls) and over a plain 1 GiB copy whose known size scales the counter.  The
    backward call's kernels are the code-plane transpose, the two bf16 products and the split-K
    sums.  None if rocprofv3 is missing or any pass fails or runs out of time (a pass takes 5-10 s;
    the first failure ends the count, so a stuck profiler costs at most one time limit)."""
    import glob
    import shutil
    import subprocess
    import tempfile

    prof = shutil.which("rocprofv3")
    if prof is None:
        return None
    me = os.path.abspath(__file__)
    env = dict(os.environ, TMPDIR="/tmp")
    bwd = ("k_codes_t", "k_gemm_nt_bf16", "k_splitk_reduce", "k_splitk_add_tail")
    out = {}
    try:
        with tempfile.TemporaryDirectory(prefix="sbl_pmc_", dir="/tmp") as tmp:
            for counter in ("FETCH_SIZE", "WRITE_SIZE"):
                got = {}
                for kind, extra in (("copy", ["--copy-calibration"]),
                                    ("train", ["--steps", "1", "--warmup", "0", "--no-cpu-baseline", "--no-peaks",
                                               "--no-live-traffic"])):
                    d = os.path.join(tmp, f"{kind}_{counter}")
                    cmd = [prof, "--pmc", counter, "--output-format", "csv", "-d", d, "-o", "run", "--",
                           sys.executable, me, *extra]
                    # rocprofv3 may end with a fault of its own after the program has finished: the
                    # result file decides, not the exit status.  The pass runs in a process group of its
                    # own, so that a time-out ends the profiled program too, not only the profiler
                    proc = subprocess.Popen(cmd, cwd="/tmp", env=env, stdout=subprocess.DEVNULL,
                                            stderr=subprocess.DEVNULL, start_new_session=True)
                    try:
                        proc.wait(timeout=timeout_s)
                    except subprocess.TimeoutExpired:
                        import signal
                        os.killpg(proc.pid, signal.SIGKILL)
                        proc.wait()
                        return None
                    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
                    if not files:
                        return None
                    got[kind] = files[0]
                copy_kib, n_copy = _counter_kib(got["copy"], lambda k: "copyBuffer" in k)
                kib, n_k = _counter_kib(got["train"], lambda k: any(b in k for b in bwd))
                if n_copy == 0 or copy_kib <= 0 or n_k == 0:
                    return None
                scale = (1 << 30) / 1024.0 / (copy_kib / n_copy)  # counter KiB -> true KiB (1 GiB per copy)
                out[counter] = kib * scale * 1024.0 / n_calls
    except (subprocess.SubprocessError, OSError, ValueError, KeyError):
        return None
    return {"bytes": out["FETCH_SIZE"] + out["WRITE_SIZE"], "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"]}


def _code_text(src: str) -> str:
    """Source text without comments and blank runs (the code that the counters measured)."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(" ".join(line.split()) for line in src.splitlines() if line.strip())


def _bwd_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_common.h", "gemm_nt.hip", "gemm_bwd.hip"):
        with open(os.path.join(ROOT, "sparsity_sparse_bitlinear_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def run_variants(args, wl):
    """The variant rows on the workload's matrices: quant/mask/pack for every N of N:8, 2:4 and the
    mask-from-quantized-weight ablation (algorithmic 2.375 B per weight), the mask-without-grad
    ablation on float32 dW buffers of the same shapes (8.125 B per weight: dW read and written, mask),
    the AdamW step + repack (24.5 B per weight: W, dW, m, v and the previous mask read; W, m, v,
    the new mask and the codes written), and Q_a(Norm(x)) fused against the act quant alone on the
    workload's activations (3 B per element + 4 B per token: the norm adds arithmetic, no bytes)."""
    import numpy as np
    import torch

    import sparsity_sparse_bitlinear_amd as sbl
    from sbl_inputs import weight

    dev = torch.device("cuda:0")
    Ws = [torch.from_numpy(weight(wl.cfg, mi, L.d_out, L.d_in).view(np.int16)).view(torch.bfloat16).to(dev)
          for mi, L in enumerate(wl.linears)]
    outs = [(torch.empty((L.d_out, L.d_in // 8), dtype=torch.int16, device=dev),
             torch.empty((L.d_out, L.d_in // 8), dtype=torch.uint8, device=dev),
             torch.empty((1,), dtype=torch.float32, device=dev),
             torch.empty((max(16, sbl.quant_workspace_size(L.d_out, L.d_in)),), dtype=torch.uint8, device=dev))
            for L in wl.linears]
    n_w = sum(L.d_out * L.d_in for L in wl.linears)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    patterns = [(n, 8, False) for n in (8, 7, 6, 5, 4, 3, 2)] + [(2, 4, False), (6, 8, True), (2, 4, True)]
    rows = []
    for n, m, fq in patterns:
        def pack():
            for W, (c, mk, g, ws) in zip(Ws, outs):
                sbl.quant_mask_pack(W, n, m=m, from_quantized=fq, codes=c, mask=mk, gamma=g, workspace=ws)
        ms = timed(pack)
        gbs = 2.375 * n_w / (ms * 1e-3) / 1e9
        rows.append({"pattern": f"{n}:{m}" + (" from W_q" if fq else ""), "ms": round(ms, 4),
                     "GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
    dWs = [torch.randn((L.d_out, L.d_in), device=dev) for L in wl.linears]
    for W, (c, mk, g, ws) in zip(Ws, outs):
        sbl.quant_mask_pack(W, 6, codes=c, mask=mk, gamma=g, workspace=ws)

    def mg():
        for dW, (_, mk, _, _) in zip(dWs, outs):
            sbl.mask_grad(dW, mk)
    ms = timed(mg)
    gbs = 8.125 * n_w / (ms * 1e-3) / 1e9
    # optimizer step + repack: reads W, dW, m, v, the previous mask; writes W, m, v, mask, codes
    ms_moments = [(torch.zeros_like(dW), torch.zeros_like(dW)) for dW in dWs]
    new_masks = [torch.empty_like(mk) for (_, mk, _, _) in outs]
    flips = [torch.zeros((1,), dtype=torch.int64, device=dev) for _ in outs]

    def opt():
        for W, dW, (mm, vv), (c, mk, g, ws), mk2, fl in zip(Ws, dWs, ms_moments, outs, new_masks, flips):
            sbl.adamw_repack(W, dW, mm, vv, step=2, lr=1e-5, n_keep=6, mask_prev=mk, mask=mk2, codes=c, gamma=g,
                             flips=fl, workspace=ws)
    ms_opt = timed(opt)
    gbs_opt = 24.5 * n_w / (ms_opt * 1e-3) / 1e9
    # Q_a(Norm(x)) fused against the act quant alone, on the workload's activations
    from sbl_inputs import activation
    T = max(wl.T)
    xs = [torch.from_numpy(activation(wl.cfg, mi, T, L.d_in, dist=wl.act_dist).view(np.int16)).view(torch.bfloat16)
          .to(dev) for mi, L in enumerate(wl.linears)]
    gs = [torch.ones((L.d_in,), dtype=torch.bfloat16, device=dev) for L in wl.linears]
    qs = [(torch.empty((T, L.d_in), dtype=torch.int8, device=dev), torch.empty((T,), device=dev))
          for L in wl.linears]
    n_x = sum(T * L.d_in for L in wl.linears)

    def norm_q():
        for x, g, (q, a) in zip(xs, gs, qs):
            sbl.rmsnorm_act_quant(x, g, 1e-6, x_q=q, absmax=a)

    def plain_q():
        for x, (q, a) in zip(xs, qs):
            sbl.act_quant(x, x_q=q, absmax=a)
    ms_norm, ms_act = timed(norm_q), timed(plain_q)
    bytes_x = 3 * n_x + 4 * T * len(xs)
    # 2:8 forward: the dense path (codes expanded to int8, dense matrix instruction) against the
    # kept-only 2:4 plane on the sparse matrix instruction; the same int32 sums
    sp = []
    for W, (x, (q, a)) in zip(Ws, zip(xs, qs)):
        c28, _, g28 = sbl.quant_mask_pack(W, 2, want_mask=False)
        plane, _ = sbl.pack_sparse24(c28)
        sbl.act_quant(x, x_q=q, absmax=a)
        sp.append((c28, g28, plane, q, a, torch.empty((T, W.shape[0]), dtype=torch.bfloat16, device=dev)))

    def fwd_dense():
        for c28, g28, _, q, a, y in sp:
            sbl.forward(c28, g28, q, a, out_dtype=sbl.BF16, y=y)

    def fwd_sparse():
        for _, g28, plane, q, a, y in sp:
            sbl.forward_sparse24(plane, g28, q, a, out_dtype=sbl.BF16, y=y)
    ms_fd, ms_fs = timed(fwd_dense), timed(fwd_sparse)
    ops_28 = sum(2.0 * T * L.d_out * L.d_in * 2 / 8 for L in wl.linears)
    del xs, qs, sp
    line = {"metric": "Sparse-BitLinear variants: quant/mask/pack per N:M pattern and mask-without-grad, "
                      "7 linears of a 3B-like layer",
            "value": rows[2]["ms"], "unit": "ms per layer (6:8 quant/mask/pack)", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None,
            "dtype": "bf16 in, 2-bit codes + mask plane out", "data": "synthetic",
            "config": {"workload": wl.name, "weights": n_w},
            "quant_mask_pack": rows,
            "mask_grad": {"ms": round(ms, 4), "GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)},
            "adamw_repack": {"ms": round(ms_opt, 4), "GBps": round(gbs_opt, 1),
                             "frac_hbm": round(gbs_opt / HBM_PEAK_GBS, 4), "bytes_per_weight": 24.5},
            "rmsnorm_act_quant": {"tokens": T, "ms": round(ms_norm, 4),
                                  "GBps": round(bytes_x / (ms_norm * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(bytes_x / (ms_norm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "act_quant_alone_ms": round(ms_act, 4)},
            "forward_2of8": {"tokens": T, "dense_ms": round(ms_fd, 4), "sparse24_ms": round(ms_fs, 4),
                             "sparse24_TOPs_algorithmic": round(ops_28 / (ms_fs * 1e-3) / 1e12, 1),
                             "speedup": round(ms_fd / ms_fs, 3)}}
    print(json.dumps(line), flush=True)


DECODE_FUSE_MAX = 1 << 62  # T * d_in up to which a group takes the fused launch (where it is supported)


# Linears of a decoder layer that read the same activations: q, k, v the normed hidden
# state, gate and up the normed residual; o and down read their own inputs.
DECODE_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def decode_groups(wl):
    """Index groups of wl.linears that share one input (DECODE_GROUPS; anything else alone)."""
    names = [L.name for L in wl.linears]
    groups, seen = [], set()
    for g in DECODE_GROUPS:
        idx = [names.index(n) for n in g if n in names]
        if idx:
            groups.append(idx)
            seen.update(idx)
    groups += [[i] for i in range(len(names)) if i not in seen]
    return groups


def _decode_case(args, wl, sbl, torch, up, activation, groups, layers, plane_name, plane_fmt, code_bytes, n_keep, T,
                 copies, fuse_max, peaks):
    """One (plane, mask, T) case of the decode workload: the layer's input groups in one captured graph
    over `copies` packed copies; returns the result record."""
    dev = torch.device("cuda:0")
    gbufs = []
    for g in groups:
        L0 = wl.linears[g[0]]
        x = up(activation(wl.cfg, g[0], T, L0.d_in, dist=wl.act_dist))
        # the activation quantization inside the product's launch wherever it is supported
        fused = sbl.decode_plane_supported(plane_fmt, T, L0.d_in) and T * L0.d_in <= fuse_max
        gbufs.append(dict(x=x, fused=fused,
                          x_q=torch.empty((T, L0.d_in), dtype=torch.int8, device=dev),
                          a=torch.empty((T,), dtype=torch.float32, device=dev),
                          ys=[torch.empty((T, wl.linears[i].d_out), dtype=torch.bfloat16, device=dev) for i in g]))

    def run_group(g, b, mats):
        gm = [mats[i] for i in g]
        if b["fused"]:
            sbl.forward_plane_multi(plane_fmt, gm, x=b["x"], out_dtype=sbl.BF16, ys=b["ys"])
        else:
            sbl.act_quant(b["x"], x_q=b["x_q"], absmax=b["a"])
            sbl.forward_plane_multi(plane_fmt, gm, x_q=b["x_q"], absmax=b["a"], out_dtype=sbl.BF16, ys=b["ys"])

    def layer(mats):
        for g, b in zip(groups, gbufs):
            run_group(g, b, mats)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for mats in layers:         # warm up outside the capture
            layer(mats)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for mats in layers:
            layer(mats)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps / copies
    io_bytes = (sum(2 * T * wl.linears[grp[0]].d_in for grp in groups) + sum(2 * T * L.d_out for L in wl.linears))
    launches = sum(1 if b["fused"] else 2 for b in gbufs)
    r = {"T": T, "n_keep": n_keep, "plane": plane_name, "us_per_layer": round(us, 3), "launches_per_layer": launches,
         "tokens_per_s": round(T / (us * 1e-6), 1), "code_bytes_per_layer": code_bytes,
         "GBps": round((code_bytes + io_bytes) / (us * 1e-6) / 1e9, 1),
         "frac_hbm": round((code_bytes + io_bytes) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if peaks:
        r["frac_hbm_measured"] = round((code_bytes + io_bytes) / (us * 1e-6) / 1e9 / peaks["read_GBps"], 4)
    del graph
    # each input group alone (same copies), beside one launch of the streaming-read kernel over
    # the group's plane bytes: the floor of a dependent launch that moves those bytes
    r["groups"] = []
    for g, b in zip(groups, gbufs):
        gus = graph_us(lambda: [run_group(g, b, mats) for mats in layers], reps=args.steps, warmup=args.warmup)
        gbytes = sum(layers[0][i][0].numel() * layers[0][i][0].element_size() for i in g)
        r["groups"].append({"group": "+".join(wl.linears[i].name for i in g), "launches": 1 if b["fused"] else 2,
                            "us": round(gus / copies, 3), "plane_bytes": gbytes,
                            "read_floor_us": round(read_floor_us(gbytes), 3)})
    return r


def graph_us(fn, reps: int = 20, warmup: int = 3, copies: int = 1) -> float:
    """Time of one call of fn, from replays of a HIP graph that holds `copies` calls of fn back to
    back (fn's launches go to the current stream); copies > 1 spreads the fixed cost of one graph
    launch (about 20 us here, more than a small step's kernels) over that many calls."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(copies):
            fn()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1e3 / reps / copies


def read_floor_us(nbytes: int) -> float:
    """Time per launch of the library's streaming-read kernel (sbl_peak_read) over nbytes, each
    launch of a captured graph reading its own slice of a buffer larger than the last-level cache:
    the floor of one dependent launch that moves nbytes from HBM."""
    import math

    import torch

    import sparsity_sparse_bitlinear_amd as sbl

    nbytes = max(16, nbytes // 16 * 16)
    copies = max(4, min(64, math.ceil(600e6 / nbytes)))
    buf = torch.ones((copies * nbytes // 4 + 4,), dtype=torch.float32, device="cuda")
    word = torch.zeros((1,), dtype=torch.int32, device="cuda")
    base = buf.data_ptr()

    def run():
        for c in range(copies):
            sbl._check(sbl.lib.sbl_peak_read(base + c * nbytes, nbytes, sbl._ptr(word), sbl._stream()),
                       "sbl_peak_read")

    us = graph_us(run) / copies
    del buf
    torch.cuda.synchronize()
    return us


def run_decode(args, wl, copies: int = 16):
    """Decode workload: act quant + forward of every linear of a layer on pre-packed codes, for
    each token count and mask.  The linears that read the same activations (q, k, v; gate, up)
    share one input and one call (the activation quantization fused in where supported, else
    sbl_act_quant + the product); masks keeping at most 2 of 8 are also run on the pair plane.
    `copies` distinct packed copies of the layer (more bytes than the 256 MB last-level cache)
    are walked in turn inside one captured HIP graph, so the code planes stream from HBM; the
    figure is graph time / copies per layer."""
    import numpy as np
    import torch

    import sparsity_sparse_bitlinear_amd as sbl
    from sbl_inputs import activation, weight

    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    Ws = [up(weight(wl.cfg, mi, L.d_out, L.d_in)) for mi, L in enumerate(wl.linears)]
    groups = decode_groups(wl)
    peaks = None if args.no_peaks else measured_peaks()
    fuse_max = DECODE_FUSE_MAX if args.decode_fuse_max is None else args.decode_fuse_max
    results = []
    for n_keep in wl.n_keep:
        packed = [sbl.quant_mask_pack(W, n_keep, want_mask=False) for W in Ws]
        planes = [("codes", sbl.PLANE_CODES, [(c, g) for (c, _, g) in packed])]
        if n_keep <= 2:  # the pair plane: one byte per group of 8
            planes.append(("pairs", sbl.PLANE_PAIRS, [(sbl.pack_pairs(c)[0], g) for (c, _, g) in packed]))
        for plane_name, plane_fmt, mats0 in planes:
            # distinct buffers holding the same packed layer: the graph walks all of them
            layers = [[(pl.clone(), g.clone()) for (pl, g) in mats0] for _ in range(copies)]
            torch.cuda.synchronize()
            code_bytes = sum(L.d_out * L.d_in // (4 if plane_fmt == sbl.PLANE_CODES else 8) for L in wl.linears)
            for T in wl.T:
                results.append(_decode_case(args, wl, sbl, torch, up, activation, groups, layers, plane_name, plane_fmt,
                                            code_bytes, n_keep, T, copies, fuse_max, peaks))
    line = {"metric": "Sparse-BitLinear decode: act quant + forward of a 3B-like layer (7 linears) on packed codes",
            "value": results[0]["us_per_layer"], "unit": "us per layer (T=%d, %d:8)" % (results[0]["T"], results[0]["n_keep"]),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
            "vs_baseline": None, "dtype": "int8 x ternary (int32 accumulate), y bf16", "data": "synthetic",
            "config": {"workload": wl.name, "layer_copies_per_graph": copies,
                       "input_groups": ["+".join(wl.linears[i].name for i in grp) for grp in groups],
                       "code_bytes_per_layer": sum(L.d_out * L.d_in // 4 for L in wl.linears)},
            "results": results, "measured_peaks": peaks}
    print(json.dumps(line), flush=True)


def measured_peaks():
    """Ceilings measured on this GPU: the int8 (32x32x32) and bf16 (32x32x16) matrix instructions
    on register operands (1024 blocks of 4 waves, 4 independent chains each), a streaming read of
    2 GiB with the library's read kernel, and a torch copy of 1 GiB (read + write)."""
    import torch

    import sparsity_sparse_bitlinear_amd as sbl

    dev = torch.device("cuda:0")
    blocks, iters = 1024, 20000
    sink = torch.zeros((blocks,), dtype=torch.float32, device=dev)
    out = {}

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    for kind, key, ops in ((0, "int8_TOPs", 65536), (1, "bf16_TFLOPs", 32768)):
        sec = timed(lambda: sbl._check(sbl.lib.sbl_peak_mfma(kind, iters, blocks, sbl._ptr(sink), None),
                                       "sbl_peak_mfma"), 3)
        out[key] = round(blocks * 4 * 4 * iters * ops / sec / 1e12, 1)
    nbytes = 2 << 30
    buf = torch.ones((nbytes // 4,), dtype=torch.float32, device=dev)
    word = torch.zeros((1,), dtype=torch.int32, device=dev)
    sec = timed(lambda: sbl._check(sbl.lib.sbl_peak_read(sbl._ptr(buf), nbytes, sbl._ptr(word), None),
                                   "sbl_peak_read"), 10)
    out["read_GBps"] = round(nbytes / sec / 1e9, 1)
    a = buf[: (1 << 28)]
    b = torch.empty_like(a)
    sec = timed(lambda: b.copy_(a), 10)
    out["copy_GBps"] = round(2 * a.numel() * 4 / sec / 1e9, 1)
    out["datasheet"] = {"int8_TOPs": INT8_PEAK_TOPS, "bf16_TFLOPs": BF16_PEAK_TFLOPS, "hbm_GBps": HBM_PEAK_GBS}
    del buf, a, b
    torch.cuda.synchronize()
    return out


def run_forward_sweep(args, wl):
    """Forward-only workload swept over masks (the 0.5B-like up-projection): per mask, one step is
    the packing of W (quant/mask/pack), the act quant of x and the forward (y bf16); tokens/s =
    T / step time.  The step is timed as replays of one captured graph (and, as eager_step_ms,
    with HIP events between eager launches; --timing eager makes that the figure).  Inputs
    resident in HBM."""
    import numpy as np
    import torch

    import sparsity_sparse_bitlinear_amd as sbl
    from sbl_inputs import activation, weight

    dev = torch.device("cuda:0")
    T = wl.T[0]
    (L,) = wl.linears
    d_out, d_in = L.d_out, L.d_in

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    W = up(weight(wl.cfg, 0, d_out, d_in))
    x = up(activation(wl.cfg, 0, T, d_in, dist=wl.act_dist, outlier_frac=wl.outlier_frac))
    codes = torch.empty((d_out, d_in // 8), dtype=torch.int16, device=dev)
    mask = torch.empty((d_out, d_in // 8), dtype=torch.uint8, device=dev)
    gamma = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = torch.empty((max(16, sbl.quant_workspace_size(d_out, d_in)),), dtype=torch.uint8, device=dev)
    x_q = torch.empty((T, d_in), dtype=torch.int8, device=dev)
    absmax = torch.empty((T,), dtype=torch.float32, device=dev)
    y = torch.empty((T, d_out), dtype=torch.bfloat16, device=dev)
    peaks = None if args.no_peaks else measured_peaks()
    results = []
    for n_keep in wl.n_keep:
        calls = (lambda: sbl.quant_mask_pack(W, n_keep, codes=codes, mask=mask, gamma=gamma, workspace=ws),
                 lambda: sbl.act_quant(x, x_q=x_q, absmax=absmax),
                 lambda: sbl.forward(codes, gamma, x_q, absmax, out_dtype=sbl.BF16, y=y))
        for _ in range(args.warmup):
            for c in calls:
                c()
        torch.cuda.synchronize()
        reps = max(args.steps, 20)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        t0 = time.perf_counter()
        for ev in evs:
            for k, c in enumerate(calls):
                ev[k].record()
                c()
            ev[3].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / reps
        ms = np.array([[ev[k].elapsed_time(ev[k + 1]) for k in range(3)] for ev in evs]).mean(axis=0)
        step_ms = float(ms.sum())
        eager_step_ms = step_ms
        if use_graph(args):
            # GRAPH_COPIES steps of the three calls captured in one graph and replayed; per call,
            # GRAPH_COPIES copies of it alone
            step_ms = graph_us(lambda: [c() for c in calls], reps=reps, warmup=args.warmup, copies=GRAPH_COPIES) / 1e3
            ms = np.array([graph_us(c, reps=reps, warmup=args.warmup, copies=GRAPH_COPIES) / 1e3 for c in calls])
        ops = 2.0 * T * d_out * d_in * n_keep / 8
        q_bytes = 2.375 * d_out * d_in
        a_bytes = 3.0 * T * d_in + 4.0 * T
        f_bytes = T * d_in + d_out * d_in / 4 + 2.0 * T * d_out
        r = {"n_keep": n_keep, "tokens_per_s": round(T / (step_ms * 1e-3), 1), "step_ms": round(step_ms, 5),
             "eager_step_ms": round(eager_step_ms, 5), "wall_ms_per_step": round(wall * 1e3, 5),
             "quant_mask_pack": {"ms": round(ms[0], 5), "frac_hbm": round(q_bytes / (ms[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
             "act_quant": {"ms": round(ms[1], 5), "frac_hbm": round(a_bytes / (ms[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
             "forward_int8": {"ms": round(ms[2], 5), "TOPs": round(ops / (ms[2] * 1e-3) / 1e12, 2),
                              "frac_int8": round(ops / (ms[2] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                              "frac_hbm": round(f_bytes / (ms[2] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        results.append(r)
    main6 = next((r for r in results if r["n_keep"] == 6), results[0])
    # The dominant kernel of the 6:8 step (all three are far below a microsecond of work at roofline:
    # these launches are bound by launch and memory latency, not by a peak).
    parts = {"quant_mask_pack": ("hbm", 2.375 * d_out * d_in, "GB/s", HBM_PEAK_GBS, 1e9),
             "act_quant": ("hbm", 3.0 * T * d_in + 4.0 * T, "GB/s", HBM_PEAK_GBS, 1e9),
             "forward_int8": ("mfma", 2.0 * T * d_out * d_in * 6 / 8, "TOP/s", INT8_PEAK_TOPS, 1e12)}
    dom = max(parts, key=lambda k: main6[k]["ms"])
    bound, work, unit, peak, scale = parts[dom]
    achieved = work / (main6[dom]["ms"] * 1e-3) / scale
    roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": None, "avg_launch_ms": main6[dom]["ms"]}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_forward_sweep(wl)
    line = {"metric": "Sparse-BitLinear forward tokens/s, 0.5B-like up-projection (quant/mask/pack + act quant + "
                      "forward per step), swept over N:8",
            "value": main6["tokens_per_s"], "unit": "tokens/s (6:8)", "n_gpus": 1, "steps": reps,
            "warmup": args.warmup, "ms_per_step": main6["step_ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int8 x ternary (int32 accumulate), y bf16", "data": "synthetic",
            "config": {"workload": wl.name, "tokens": T, "d_out": d_out, "d_in": d_in, "masks": list(wl.n_keep)},
            "roofline": roofline, "results": results, "cpu_baseline": cpu, "measured_peaks": peaks}
    if use_graph(args):
        line["timing"] = (f"graph replay: {GRAPH_COPIES} steps (the three calls each) captured back to back in one HIP "
                          f"graph, replayed, time / {GRAPH_COPIES}; per-call figures likewise from {GRAPH_COPIES} copies "
                          "of each call; eager_step_ms: events between eager launches")
    print(json.dumps(line), flush=True)


def cpu_forward_sweep(wl):
    """The oracle's forward step (packing, act quant, int64 forward, y) at full shape, 6:8."""
    import oracle
    from sbl_inputs import activation, weight

    (L,) = wl.linears
    T = wl.T[0]
    W = weight(wl.cfg, 0, L.d_out, L.d_in)
    x = activation(wl.cfg, 0, T, L.d_in, dist=wl.act_dist, outlier_frac=wl.outlier_frac)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    w_eff, mask, g = oracle.effective_weight(W, 6)
    oracle.pack_codes(w_eff)
    xq, a = oracle.act_quant(x)
    oracle.forward_y(oracle.forward_acc(w_eff, xq), g, a)
    sec = time.perf_counter() - t0
    return {"value": round(T / sec, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the whole 6:8 step at full shape ({T} tokens), {sec:.2f} s"}


def cpu_baseline(wl, T, n_keep, T_s):
    """Oracle time for one step, estimated from a bounded sample: quant/mask/pack of all
    matrices at full size (a per-step cost independent of T) plus act quant, forward and
    backward of every linear on T_s tokens, scaled by T / T_s."""
    import numpy as np

    import oracle
    from sbl_inputs import activation, grad_out, sample_rows, weight

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    T_s = min(T_s, T)
    t_fixed = 0.0
    t_tok = 0.0
    for mi, L in enumerate(wl.linears):
        W = weight(wl.cfg, mi, L.d_out, L.d_in)
        rows = sample_rows(wl.cfg, 100 + mi, T, T_s)
        x = activation(wl.cfg, mi, T, L.d_in, dist=wl.act_dist, outlier_frac=wl.outlier_frac, rows=rows)
        dY = grad_out(wl.cfg, mi, T, L.d_out, rows=rows)
        t0 = time.perf_counter()
        w_eff, mask, g = oracle.effective_weight(W, n_keep)
        oracle.pack_codes(w_eff)
        oracle.pack_mask(mask)
        t1 = time.perf_counter()
        xq, a = oracle.act_quant(x)
        acc = oracle.forward_acc(w_eff, xq)
        oracle.forward_y(acc, g, a)
        oracle.backward(dY, w_eff, g, xq, a)
        t2 = time.perf_counter()
        t_fixed += t1 - t0
        t_tok += t2 - t1
    est = t_fixed + t_tok * (T / T_s)
    return {"value": round(T / est, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"all {len(wl.linears)} linears: quant/mask/pack at full size ({t_fixed:.1f} s) + "
                      f"act quant, forward, backward on {T_s} of {T} sampled tokens ({t_tok:.1f} s), "
                      f"token part scaled by {T / T_s:g}; estimated {est:.1f} s per step"}


if __name__ == "__main__":
    main()
