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
Metric: tokens per second of whole steps.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
       python bench.py --workload 4     (decode: per-layer latency at 1/8/64 tokens, 6/4/2:8)
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
# rocprofv3 --pmc for the backward kernel sources whose hash is given
# (profiles/traffic_backward_3b_32768tok.md).
BWD_TRAFFIC_BYTES = 2.48e9
BWD_TRAFFIC_SRC_SHA = "b6811c550191b403"
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
    ap.add_argument("--cpu-tokens", type=int, default=1024, help="token sample for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-fuse-max", type=int, default=None,
                    help="decode: largest T * d_in * (16-row blocks of a group) that takes the fused launch")
    ap.add_argument("--breakdown", action="store_true", help="print the per-linear breakdown to stderr")
    ap.add_argument("--variants", action="store_true",
                    help="N:M patterns and ablations: quant/mask/pack per pattern and mask-without-grad on the "
                         "3B-like matrices (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (scale reference for HBM byte counters)")
    return ap.parse_args()


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
    wl = WORKLOADS[args.workload]
    if args.variants:
        run_variants(args, wl)
        return
    if not wl.backward and len(wl.T) > 1:
        run_decode(args, wl)
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
    traffic = None
    if (dom == "bwd" and args.workload == 3 and n_keep == 6 and BWD_TRAFFIC_BYTES is not None
            and _bwd_sources_sha() == BWD_TRAFFIC_SRC_SHA):
        traffic = BWD_TRAFFIC_BYTES
    roofline = {"bound": "mfma", "kernel": dname, "achieved": round(achieved, 1), "peak": dpeak,
                "unit": dunit, "frac": round(achieved / dpeak, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "launches_per_step": n_launch, "hip_kernels": dkernels,
                "avg_launch_ms": round(tot_ms[parts.index(dom)] / n_launch, 4)}

    # CPU baseline: the oracle on a bounded sample, on this host's cores.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, T, n_keep, args.cpu_tokens)

    line = {
        "metric": "Sparse-BitLinear 6:8 fwd+bwd tokens/s at 3B shapes; % int8 MFMA / HBM peak",
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
        "input_gen_s": round(t_gen, 1),
    }
    if args.breakdown:
        for li, Lr in enumerate(layers):
            print(Lr["name"], " ".join(f"{p}={per_launch_ms[li, k]:.4f}ms" for k, p in enumerate(parts)),
                  file=sys.stderr)
    print(json.dumps(line), flush=True)


def _bwd_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm_common.h", "gemm_nt.hip", "gemm_bwd.hip"):
        with open(os.path.join(ROOT, "sparsity_sparse_bitlinear_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
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


DECODE_FUSE_MAX = 32_000_000  # T * d_in * (16-row blocks) per launch up to which the fused decode beats
                              # two calls (2048-wide rows: gate+up of a 3B layer at 8 tokens, 22.5e6, wins)


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


def run_decode(args, wl, copies: int = 16):
    """Decode workload: act quant + forward of every linear of a layer on pre-packed codes, for
    each token count and mask.  The linears that read the same activations (q, k, v; gate, up)
    share one input and one call (sbl_decode_multi, or sbl_act_quant + sbl_forward_decode_multi).
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
    fuse_max = DECODE_FUSE_MAX if args.decode_fuse_max is None else args.decode_fuse_max
    results = []
    for n_keep in wl.n_keep:
        packed = [sbl.quant_mask_pack(W, n_keep, want_mask=False) for W in Ws]
        # distinct buffers holding the same packed layer: the graph walks all of them
        layers = [[(codes.clone(), gamma.clone()) for (codes, _, gamma) in packed] for _ in range(copies)]
        torch.cuda.synchronize()
        code_bytes = sum(L.d_out * L.d_in // 4 for L in wl.linears)
        for T in wl.T:
            gbufs = []
            for g in groups:
                L0 = wl.linears[g[0]]
                x = up(activation(wl.cfg, g[0], T, L0.d_in, dist=wl.act_dist))
                # one fused launch (sbl_decode_multi) where it applies and its per-block
                # re-quantization of the T rows stays small (T * d_in * blocks of 16 rows),
                # else act quant + one sbl_forward_decode_multi
                blocks = sum(-(-wl.linears[i].d_out // 16) for i in g)
                gbufs.append(dict(x=x, fused=sbl.decode_supported(T, L0.d_in) and T * L0.d_in * blocks <= fuse_max,
                                  x_q=torch.empty((T, L0.d_in), dtype=torch.int8, device=dev),
                                  a=torch.empty((T,), dtype=torch.float32, device=dev),
                                  ys=[torch.empty((T, wl.linears[i].d_out), dtype=torch.bfloat16, device=dev)
                                      for i in g]))

            def layer(mats):
                for g, b in zip(groups, gbufs):
                    gm = [mats[i] for i in g]
                    if b["fused"]:
                        sbl.decode_multi(gm, b["x"], out_dtype=sbl.BF16, ys=b["ys"])
                    else:
                        sbl.act_quant(b["x"], x_q=b["x_q"], absmax=b["a"])
                        sbl.forward_decode_multi(gm, b["x_q"], b["a"], out_dtype=sbl.BF16, ys=b["ys"])

            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for mats in layers:         # warm up outside the capture
                    layer(mats)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for mats in layers:
                    layer(mats)
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.steps / copies
            io_bytes = (sum(2 * T * wl.linears[grp[0]].d_in for grp in groups)
                        + sum(2 * T * L.d_out for L in wl.linears))
            launches = sum(1 if b["fused"] else 2 for b in gbufs)
            results.append({"T": T, "n_keep": n_keep, "us_per_layer": round(us, 3), "launches_per_layer": launches,
                            "tokens_per_s": round(T / (us * 1e-6), 1),
                            "GBps": round((code_bytes + io_bytes) / (us * 1e-6) / 1e9, 1),
                            "frac_hbm": round((code_bytes + io_bytes) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
            del g
    line = {"metric": "Sparse-BitLinear decode: act quant + forward of a 3B-like layer (7 linears) on packed codes",
            "value": results[0]["us_per_layer"], "unit": "us per layer (T=%d, %d:8)" % (results[0]["T"], results[0]["n_keep"]),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
            "vs_baseline": None, "dtype": "int8 x ternary (int32 accumulate), y bf16", "data": "synthetic",
            "config": {"workload": wl.name, "layer_copies_per_graph": copies,
                       "input_groups": ["+".join(wl.linears[i].name for i in grp) for grp in groups],
                       "code_bytes_per_layer": code_bytes}, "results": results}
    print(json.dumps(line), flush=True)


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
                      f"token part scaled by {T // T_s}; estimated {est:.1f} s per step"}


if __name__ == "__main__":
    main()
