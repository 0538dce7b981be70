"""Benchmark of the small-M NVFP4 W4A4 decode linear on one MI355X.

A step is one pass of the decode hot path over the four projections of a
Qwen3-8B-shaped decoder layer (QKV 6144x4096, O 4096x4096, gate_up
24576x4096, down 4096x12288) at M activation rows: for each projection the
bf16 activation is quantized to NVFP4 on the device and the NVFP4 linear
streams the FP4 weights.  Weights are quantized once, then copied into
enough distinct buffers (>= 1 GiB in total) that every step reads weights
that are not resident in the 256 MB Infinity Cache.  Inputs are seeded
synthetic data with the shapes and distributions of that workload.

Prints one JSON line: the step's whole-path algorithmic HBM bytes per
second (value), the GEMV kernel's roofline fraction (HIP events around each
GEMV launch on the launch stream, over the timed steps), per-projection
microseconds and GB/s, and the CPU oracle timed on a bounded sample.
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

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
WEIGHT_BYTES_PER_ELEM = 0.5 + 1.0 / 16


def gemv_bytes(M, N, K, out_bytes=4):
    """Algorithmic bytes of one linear: FP4 weight codes + E4M3 scales +
    tensor scale, the quantized activation, and the output."""
    return (N * K * WEIGHT_BYTES_PER_ELEM + 4 + M * K * WEIGHT_BYTES_PER_ELEM + 4
            + M * N * out_bytes)


def actq_bytes(M, K):
    """Algorithmic bytes of the activation quantizer: bf16 in, codes and
    scales out (plus the tensor scale)."""
    return M * K * 2 + M * K * WEIGHT_BYTES_PER_ELEM + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--m", type=int, default=1, help="activation rows (1..8)")
    ap.add_argument("--workload", default="8b", choices=["8b", "32b"])
    ap.add_argument("--copies-gib", type=float, default=1.2,
                    help="total bytes of rotated weight copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--sweep", action="store_true",
                    help="also report GEMV-only us and GB/s at M = 1, 2, 4, 8")
    return ap.parse_args()


def cpu_baseline(linears, cfg, M, kind, budget_s):
    """The oracle as it stands, on a bounded sample: every projection keeps
    its first 1/16 of the weight rows (quantized by the oracle with the
    whole-tensor scale and dequantized once, outside the timed region); one
    timed iteration is oracle.quantize(x) + the FP64 dot for all four
    projections.  Iterations repeat until the time budget is spent."""
    import oracle
    from workloads import activations_bf16, bf16_to_f32, weights_bf16
    prep = []
    for li, L in enumerate(linears):
        rows = max(32, L.N // 16)
        wf = bf16_to_f32(weights_bf16(cfg, li, L.N, L.K))
        _, sg = oracle.global_scale(wf)
        c, s = oracle.quantize_blocks(wf[:rows], sg)
        w_hat = oracle.dequantize(oracle.NVFP4Tensor(c, s, np.asarray(sg, np.float32)))
        x = bf16_to_f32(activations_bf16(cfg, li, M, L.K, kind))
        prep.append((x, w_hat, rows, L))
        del wf
    byts = sum(gemv_bytes(M, rows, L.K) + actq_bytes(M, L.K) for _, _, rows, L in prep)
    n = 0
    t0 = time.perf_counter()
    while True:
        for x, w_hat, rows, L in prep:
            xq = oracle.quantize(x)
            y = oracle.dequantize(xq) @ w_hat.T
            assert y.shape == (M, rows)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": round(byts * n / el / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"{n} iterations over the 4 projections with the first 1/16 of each "
                   f"weight's rows (M={M}); oracle act quantization + FP64 dot; "
                   f"{el:.1f} s on host cores"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode linear runs on a single MI355X "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import nvfp4_decode_linear_amd as nv
    from workloads import QWEN3_8B, QWEN3_32B, activations_bf16, weights_bf16

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    M = args.m
    if args.workload == "8b":
        linears, cfg, kind, wl = QWEN3_8B, (2 if M == 1 else 3), "outlier", "qwen3_8b_decode_step"
    else:
        linears, cfg, kind, wl = QWEN3_32B, 4, "student_t", "qwen3_32b_decode_step"

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # weights: quantize once, then copy to defeat the Infinity Cache
    base = []
    for li, L in enumerate(linears):
        wq = nv.quantize_weight(to_dev(weights_bf16(cfg, li, L.N, L.K)))
        base.append(wq)
    set_bytes = sum(w.codes.numel() + w.scales.numel() for w in base)
    copies = max(1, int(np.ceil(args.copies_gib * (1 << 30) / set_bytes)))
    wsets = [base]
    for _ in range(copies - 1):
        wsets.append([nv.QuantWeight(w.codes.clone(), w.scales.clone(), w.gscale.clone(), w.N,
                                     w.K) for w in base])
    xs = [to_dev(activations_bf16(cfg, li, M, L.K, kind)) for li, L in enumerate(linears)]
    xqs = [nv.empty_act(M, L.K) for L in linears]
    ys = [torch.empty((M, L.N), dtype=torch.float32, device=dev) for L in linears]
    ws = nv.workspace(M, max(L.N for L in linears), max(L.K for L in linears))
    for L in linears:
        ws = nv.workspace(M, L.N, L.K)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(i, evs=None):
        wset = wsets[i % copies]
        for li in range(len(linears)):
            nv.quantize_act(xs[li], out=xqs[li])
            if evs is not None:
                evs[li][0].record(stream)
            nv.linear(xqs[li], wset[li], out=ys[li], ws=ws)
            if evs is not None:
                evs[li][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in linears] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    per = []
    tot_b = tot_t = 0.0
    for li, L in enumerate(linears):
        us = np.mean([ev[i][li][0].elapsed_time(ev[i][li][1]) for i in range(args.steps)]) * 1e3
        b = gemv_bytes(M, L.N, L.K)
        tot_b += b
        tot_t += us
        per.append({"name": L.name, "N": L.N, "K": L.K, "us": round(float(us), 3),
                    "GBps": round(b / (us * 1e-6) / 1e9, 1),
                    "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
    step_bytes = sum(gemv_bytes(M, L.N, L.K) + actq_bytes(M, L.K) for L in linears)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = tot_b / (tot_t * 1e-6) / 1e9

    sweep = None
    if args.sweep:
        sweep = {}
        for Ms in (1, 2, 4, 8):
            res = []
            xq_s = [nv.quantize_act(to_dev(activations_bf16(3, li, Ms, L.K, "outlier")))
                    for li, L in enumerate(linears)]
            y_s = [torch.empty((Ms, L.N), dtype=torch.float32, device=dev) for L in linears]
            for L in linears:
                ws = nv.workspace(Ms, L.N, L.K)
            for li, L in enumerate(linears):
                for r in range(10):
                    nv.linear(xq_s[li], wsets[r % copies][li], out=y_s[li], ws=ws)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                R = 100
                e0.record(stream)
                for r in range(R):
                    nv.linear(xq_s[li], wsets[r % copies][li], out=y_s[li], ws=ws)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / R * 1e3
                gbs = gemv_bytes(Ms, L.N, L.K) / (us * 1e-6) / 1e9
                res.append({"name": L.name, "us": round(us, 3), "GBps": round(gbs, 1)})
            sweep[f"M{Ms}"] = res

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(linears, cfg, M, kind, args.cpu_seconds)

    out = {
        "metric": "NVFP4 W4A4 GEMV achieved HBM GB/s (% of peak) + us per linear at M=1,2,4,8",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e2m1, e4m3 block-16 scales, fp32 accumulate)",
        "data": ("synthetic (seeded; bf16 weights 0.02*N(0,1), activations N(0,1) with 1%% x20 "
                 "outlier channels); weights rotated over %d copies (%.2f GiB)"
                 % (copies, copies * set_bytes / (1 << 30))),
        "config": {"workload": f"{wl}_m{M}", "M": M,
                   "linears": [f"{L.name} {L.N}x{L.K}" for L in linears],
                   "path": "per projection: nvfp4_quantize_act + nvfp4_linear (f32 out)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "gemv_valu_kernel",
                     "per_linear": per},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    if sweep is not None:
        out["sweep_gemv_only"] = sweep
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
