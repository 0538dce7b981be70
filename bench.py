"""Benchmark of the small-M NVFP4 W4A4 decode linear on one MI355X.

A step is one pass of the decode hot path over the four projections of a
Qwen3-8B-shaped decoder layer (QKV 6144x4096, O 4096x4096, gate_up
24576x4096, down 4096x12288) at M activation rows: for each projection the
bf16 activation is quantized to NVFP4 and the NVFP4 linear streams the FP4
weights, in one call (nvfp4_quantize_linear, binary32 out: one kernel whose
prologue quantizes the activation).
Weights are quantized once, then copied into enough distinct buffers
(>= 1.2 GiB) that every step reads weights that are not resident in the
256 MB Infinity Cache; step i uses copy i mod copies.  The timed steps run as
replays of HIP graphs that each hold --graph-steps consecutive steps (36 by
default: one graph per token over Qwen3-8B's 36 decoder layers, as a decode
loop replays one graph per token), plus one graph for the remainder, so that
exactly --steps steps are timed; a spin kernel holds the GPU while the host
enqueues the timed replays, so the host's launch cost is not part of the
measurement.  The same steps replayed one graph per step (which adds the
graph launch's own GPU-side cost to every step) are reported too.  Inputs are
seeded synthetic data with the shapes and distributions of that workload.

Prints one JSON line with the step's whole-path algorithmic HBM bytes per
second (value) and:
  roofline      the step's kernel (gemv_mfma_kernel quantizing its own
                activation): algorithmic bytes per launch / its average
                launch time, from HIP events around replays of graphs of
                that launch alone on the launch stream; traffic from the
                committed rocprofv3 counter summary when it was taken on the
                current kernel source
  per_linear    us and GB/s per projection at M = 1, 2, 4, 8 of the fused
                call, of the linear alone on a quantized activation, and of
                the standalone activation quantizer
  linears_32b   the same for the Qwen3-32B-shaped projections at M = 1, 4, 8
  stack         one decode step of a 64-layer stack of the 32B projections
                (graph replayed 1500 times) at M = 1 and 8
  cpu_baseline  the CPU oracle on a bounded sample of the step
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
WEIGHT_BYTES_PER_ELEM = 0.5 + 1.0 / 16
GEMV_KERNEL = "gemv_mfma_kernel"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_mfma_kernel_qwen3_8b_m1_pmc.txt")
GEMV_SOURCES = (["nvfp4_decode_linear_amd/csrc/gemv_stream.hpp",
                 "nvfp4_decode_linear_amd/csrc/gemv_stream.hip",
                 "nvfp4_decode_linear_amd/csrc/gemv_common.hpp",
                 "nvfp4_decode_linear_amd/csrc/nvfp4_device.hpp"]
                + [f"nvfp4_decode_linear_amd/csrc/gemv_stream_m{m}.hip" for m in range(1, 9)])


def gemv_bytes(M, N, K, out_bytes=4):
    """Algorithmic bytes of one linear: FP4 weight codes + E4M3 scales +
    tensor scale, the quantized activation, and the output."""
    return (N * K * WEIGHT_BYTES_PER_ELEM + 4 + M * K * WEIGHT_BYTES_PER_ELEM + 4
            + M * N * out_bytes)


def actq_bytes(M, K, in_bytes=2):
    """Algorithmic bytes of an activation quantizer: the input read once,
    codes and scales out (plus the tensor scale)."""
    return M * K * in_bytes + M * K * WEIGHT_BYTES_PER_ELEM + 4


def step_linear_bytes(M, N, K, out_bytes=4):
    """Algorithmic bytes of one projection of the step (quantize + linear):
    the weight, the bf16 activation read once, its quantized copy written
    once, the output."""
    return (N * K * WEIGHT_BYTES_PER_ELEM + 4 + M * K * 2 + M * K * WEIGHT_BYTES_PER_ELEM + 4
            + M * N * out_bytes)


def gemv_source_sha():
    h = hashlib.sha256()
    for p in GEMV_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--m", type=int, default=1, help="activation rows of the timed step (1..8)")
    ap.add_argument("--graph-steps", type=int, default=36,
                    help="steps per replayed graph in the timed loop (Qwen3-8B: 36 layers)")
    ap.add_argument("--copies-gib", type=float, default=1.2,
                    help="total bytes of rotated weight copies")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed step and its roofline (no M sweep, 32B, stack)")
    ap.add_argument("--stack-layers", type=int, default=64)
    ap.add_argument("--stack-steps", type=int, default=1500)
    ap.add_argument("--stack-only", action="store_true",
                    help="only the layer stack's decode step (no 8B step, no linear tables); "
                         "prints its own JSON line (for kernel-trace runs of the stack)")
    ap.add_argument("--kernel-compare", action="store_true",
                    help="run only the 8B projections' GEMV at M = 1, 2, 3, 8 on the VALU "
                         "kernels (streaming for M <= 3, split-K for every M) and on the FP4 "
                         "MFMA kernel, 20 launches each, for rocprofv3 kernel traces; prints "
                         "the launch order")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run only a 256 MiB device copy and a few GEMV launches of the "
                         "timed workload (for rocprofv3 counter runs), print nothing else")
    return ap.parse_args()


def graph_plan(first, steps, per_graph):
    """Steps first .. first + steps - 1 as graph replays of at most
    per_graph consecutive steps each: a list of (first step, count)."""
    return [(first + i, min(per_graph, steps - i)) for i in range(0, steps, per_graph)]


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
    byts = sum(step_linear_bytes(M, rows, L.K) for _, _, rows, L in prep)
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


def read_traffic(M):
    """HBM bytes per GEMV launch of the timed workload from the committed
    counter summary, if it was taken on the current GEMV source (else
    None): (FETCH_SIZE + WRITE_SIZE) KiB per dispatch, each scaled by the
    factor that maps the same counter onto a device copy of known size."""
    if M != 1 or not os.path.exists(TRAFFIC_SUMMARY):
        return None, "no counter summary for this workload"
    rec = None
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            m = re.match(r"^TRAFFIC_JSON (.*)$", line.strip())
            if m:
                rec = json.loads(m.group(1))
    if rec is None:
        return None, "counter summary has no TRAFFIC_JSON line"
    if rec.get("gemv_source_sha") != gemv_source_sha():
        return None, "GEMV source changed since the counters were taken"
    return rec["bytes_per_launch"], (f"rocprofv3 FETCH_SIZE x {rec['fetch_scale']:.3f} + "
                                     f"WRITE_SIZE x {rec['write_scale']:.3f} per dispatch, mean "
                                     f"of the step's {rec['launches']} GEMV launches "
                                     f"(algorithmic {rec['algorithmic_bytes_per_launch']:.0f})")


class Timer:
    """Graph capture and replay timing on one side stream (events recorded on
    the stream the kernels run on)."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.Stream()
        self.cycles_per_ms = None

    def lead(self, ms):
        """Keep the GPU busy on the timing stream for about `ms` (torch's spin
        kernel, calibrated once), so that the host has enqueued the timed
        replays before the first of them starts: the events then bracket GPU
        work only, with no gaps where the GPU waits for the host's launches."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            if self.cycles_per_ms is None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                probe = 200_000
                e0.record(self.stream)
                torch.cuda._sleep(probe)
                e1.record(self.stream)
                torch.cuda.synchronize()
                self.cycles_per_ms = probe / max(e0.elapsed_time(e1), 1e-3)
            torch.cuda._sleep(int(self.cycles_per_ms * ms))

    def capture(self, fn):
        torch = self.torch
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            fn()                                   # eager once (lazy init, workspaces)
        torch.cuda.current_stream().wait_stream(self.stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            fn()
        torch.cuda.synchronize()
        return g

    def time_replays(self, graphs, n, warm=2):
        """Average ms of one replay, cycling through `graphs`, n replays."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            for i in range(warm * len(graphs)):
                graphs[i % len(graphs)].replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
        self.lead(1.0 + 0.1 * n)
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            for i in range(n):
                graphs[i % len(graphs)].replay()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n


def progress(msg):
    """One line on stderr per finished phase, so a long run shows progress."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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
    linears, kind = QWEN3_8B, "outlier"
    cfg = 2 if M == 1 else 3
    wl = f"qwen3_8b_decode_step_m{M}"

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- weights: quantize once, then copy to defeat the Infinity Cache
    base = [nv.quantize_weight(to_dev(weights_bf16(cfg, li, L.N, L.K)))
            for li, L in enumerate(linears)]
    set_bytes = sum(w.codes.numel() + w.scales.numel() for w in base)
    copies = max(2, int(np.ceil(args.copies_gib * (1 << 30) / set_bytes)))
    wsets = [base] + [[nv.QuantWeight(w.codes.clone(), w.scales.clone(), w.gscale.clone(), w.N,
                                      w.K) for w in base] for _ in range(copies - 1)]
    xs = [to_dev(activations_bf16(cfg, li, 8, L.K, kind)) for li, L in enumerate(linears)]
    ws = None
    for Mx in (1, 2, 4, 8):
        for L in linears:
            ws = nv.workspace(Mx, L.N, L.K, dev)
    torch.cuda.synchronize()

    if args.kernel_compare:
        kernel_compare(nv, torch, dev, linears, wsets, xs)
        return

    if args.pmc_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)                             # the calibration copy: 256 MiB read + write
        xq = [nv.empty_act(M, L.K) for L in linears]
        ys = [torch.empty((M, L.N), dtype=torch.float32, device=dev) for L in linears]
        for c in range(2):
            for li in range(len(linears)):
                nv.quantize_linear(xs[li][:M], wsets[c][li], out=ys[li], xq=xq[li], ws=ws)
        torch.cuda.synchronize()
        return

    timer = Timer(torch)
    if args.stack_only:
        res = bench_32b_and_stack(args, torch, nv, dev, timer, None)
        print(json.dumps({"workload": "qwen3_32b_layer_stack", **res["stack_qwen3_32b"]}),
              flush=True)
        return

    # ---- the timed steps: per projection act quant + linear
    xqs = [nv.empty_act(M, L.K) for L in linears]
    ys = [torch.empty((M, L.N), dtype=torch.float32, device=dev) for L in linears]
    x_m = [x[:M] for x in xs]

    def steps_fn(first, count):
        """Steps first .. first + count - 1 (step i on weight copy i mod copies)."""
        def fn():
            for k in range(count):
                c = (first + k) % copies
                for li in range(len(linears)):
                    nv.quantize_linear(x_m[li], wsets[c][li], out=ys[li], xq=xqs[li], ws=ws)
        return fn

    def time_steps(graph_for, plan, warm_plan):
        """Replays `plan` (a list of (first step, count)) after `warm_plan`;
        returns ms per step and the wall time."""
        with torch.cuda.stream(timer.stream):
            for f, n in warm_plan:
                graph_for(f, n).replay()
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        gl = [graph_for(f, n) for f, n in plan]
        timer.lead(1.0 + 0.1 * len(gl))      # the host enqueues ahead of the GPU
        t0 = time.perf_counter()
        with torch.cuda.stream(timer.stream):
            t_start.record(timer.stream)
            for g in gl:
                g.replay()
            t_end.record(timer.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return t_start.elapsed_time(t_end) / sum(n for _, n in plan), wall

    graphs = {}

    def graph_for(first, count):
        key = (first % copies, count)
        if key not in graphs:
            graphs[key] = timer.capture(steps_fn(*key))
        return graphs[key]

    S = max(1, args.graph_steps)
    K = args.steps
    plan = graph_plan(args.warmup, K, S)
    warm = graph_plan(0, args.warmup, S)
    ms_step, wall = time_steps(graph_for, plan, warm)
    progress(f"timed steps: {K} in graphs of {S}, {ms_step * 1e3:.2f} us per step")
    graphs.clear()
    # the same steps, one graph replay per step
    ms_single, _ = time_steps(graph_for, graph_plan(args.warmup, K, 1),
                              graph_plan(0, args.warmup, 1))
    progress(f"one graph per step: {ms_single * 1e3:.2f} us per step")
    graphs.clear()
    step_bytes = sum(step_linear_bytes(M, L.N, L.K) for L in linears)
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # ---- GEMV-only graphs (the roofline kernel), per projection and M
    def linear_table(lins, sets, Ms, x_src, reps=8):
        table = {}
        for Mx in Ms:
            rows = []
            for li, L in enumerate(lins):
                xq = nv.quantize_act(x_src[li][:Mx])
                y = torch.empty((Mx, L.N), dtype=torch.float32, device=dev)
                w_ = nv.workspace(Mx, L.N, L.K, dev)
                n_sets = len(sets)

                def fn(xq=xq, y=y, w_=w_, li=li):
                    for c in range(n_sets):
                        nv.linear(xq, sets[c][li], out=y, ws=w_)
                g = timer.capture(fn)
                us = timer.time_replays([g], reps) * 1e3 / n_sets
                xin = torch.empty_like(x_src[li][:Mx]).copy_(x_src[li][:Mx])

                def ff(xin=xin, xq=xq, y=y, w_=w_, li=li):
                    for c in range(n_sets):
                        nv.quantize_linear(xin, sets[c][li], out=y, xq=xq, ws=w_)
                gf = timer.capture(ff)
                us_f = timer.time_replays([gf], reps) * 1e3 / n_sets

                def fq(xin=xin, xq=xq):
                    for _ in range(16):
                        nv.quantize_act(xin, out=xq, ws=ws)
                gq = timer.capture(fq)
                us_q = timer.time_replays([gq], reps) * 1e3 / 16
                b = gemv_bytes(Mx, L.N, L.K)
                bf = step_linear_bytes(Mx, L.N, L.K)
                rows.append({"name": L.name, "N": L.N, "K": L.K,
                             "us": round(us_f, 3), "GBps": round(bf / (us_f * 1e-6) / 1e9, 1),
                             "frac": round(bf / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                             "linear_only_us": round(us, 3),
                             "linear_only_GBps": round(b / (us * 1e-6) / 1e9, 1),
                             "act_quant_us": round(us_q, 3)})
                del g, gq, gf
            table[f"M{Mx}"] = rows
            progress(f"per-linear table M={Mx}: " + ", ".join(
                f"{r['name']} {r['us']:.2f}/{r['linear_only_us']:.2f} us" for r in rows))
        return table

    sweep_ms = (M,) if args.no_extras else tuple(sorted({M, 1, 2, 4, 8}))
    per_linear = linear_table(linears, wsets, sweep_ms, xs)
    rows = per_linear[f"M{M}"]
    tot_b = sum(step_linear_bytes(M, r["N"], r["K"]) for r in rows)
    tot_us = sum(r["us"] for r in rows)
    achieved = tot_b / (tot_us * 1e-6) / 1e9
    # the same kernel's roofline at every M of the sweep: mean algorithmic
    # bytes per launch / mean launch time over the four projections, and the
    # weakest projection
    per_m = {}
    for key, rs in per_linear.items():
        mx = int(key[1:])
        b = sum(step_linear_bytes(mx, r["N"], r["K"]) for r in rs)
        us = sum(r["us"] for r in rs)
        worst = min(rs, key=lambda r: r["frac"])
        per_m[key] = {"achieved": round(b / (us * 1e-6) / 1e9, 1),
                      "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "launch_us_mean": round(us / len(rs), 3),
                      "worst": {"linear": worst["name"], "frac": worst["frac"]}}
    traffic, traffic_note = read_traffic(M)
    del wsets, base

    out_extra = {}
    if not args.no_extras:
        out_extra.update(bench_32b_and_stack(args, torch, nv, dev, timer, linear_table))
        out_extra["reset_temperature"] = bench_reset(torch, nv, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(linears, cfg, M, kind, args.cpu_seconds)
        progress(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} threads")

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
        "dtype": "nvfp4 (e2m1 x e2m1 on fp4 mfma, e4m3 block-16 scales, fp32 accumulate)",
        "data": ("synthetic (seeded; bf16 weights 0.02*N(0,1), activations N(0,1) with 1% "
                 f"x20 outlier channels); weights rotated over {copies} copies "
                 f"({copies * set_bytes / (1 << 30):.2f} GiB)"),
        "config": {"workload": wl, "M": M,
                   "linears": [f"{L.name} {L.N}x{L.K}" for L in linears],
                   "path": "per projection: nvfp4_quantize_linear (activation quantized "
                           "inside the GEMV, f32 out); HIP graphs of "
                           f"{args.graph_steps} steps replayed"},
        "one_graph_per_step": {"ms_per_step": round(ms_single, 5),
                               "value": round(step_bytes / (ms_single * 1e-3) / 1e9, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": GEMV_KERNEL,
                     "traffic_note": traffic_note,
                     "launch_us_mean": round(tot_us / len(rows), 3),
                     "algorithmic_bytes_per_launch": round(tot_b / len(rows)),
                     "per_m": per_m},
        "per_linear": per_linear,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    out.update(out_extra)
    print(json.dumps(out), flush=True)


def kernel_compare(nv, torch, dev, linears, wsets, xs):
    """The same GEMVs on each kernel family (NVFP4_OPT_KERNEL: 1 = VALU
    streaming, M <= 3; 2 = VALU split-K; 3 = FP4 MFMA streaming), 20
    launches per (M, projection, kernel) over rotated weight copies, so that
    a rocprofv3 kernel trace gives each kernel's duration per shape."""
    order = []
    for M in (1, 2, 3, 8):
        for li, L in enumerate(linears):
            xq = nv.quantize_act(xs[li][:M])
            y = torch.empty((M, L.N), dtype=torch.float32, device=dev)
            for kern in ((1, 2, 3) if M <= 3 else (2, 3)):
                nv.set_option("kernel", kern)
                try:
                    ws = nv.workspace(M, L.N, L.K, dev)
                    for c in range(20):
                        nv.linear(xq, wsets[c % len(wsets)][li], out=y, ws=ws)
                    torch.cuda.synchronize()
                finally:
                    nv.set_option("kernel", 0)
                order.append(f"M={M} {L.name} kernel={kern}")
    print("\n".join(order), flush=True)


def bench_reset(torch, nv, dev, V=151936, reps=50):
    """ReSET's step-aware temperature on Qwen3-vocabulary logits (float32
    [M][151936], 4 x N(0,1)): entropy + step statistics + temperature, and
    with the scaled logits written to a second buffer; us per call from
    graph replays.  Bytes: the logits read once by the entropy kernel, and
    read + written once more by the scaling kernel."""
    res = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1519)
    p = nv.ResetParams(0.1, 0.5505, 0.6, 1.5)
    for Mx in (1, 8):
        z = torch.randn((Mx, V), generator=gen, device=dev) * 4.0
        zo = torch.empty_like(z)
        st = torch.zeros((Mx, 2), dtype=torch.float32, device=dev)
        row = {}
        for name, out in (("entropy_temperature", None), ("with_scaled_logits", zo)):
            s = torch.cuda.Stream(device=dev)
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                nv.reset_temperature(z, p, st, None, out=out)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(reps):
                    nv.reset_temperature(z, p, st, None, out=out)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (5 * reps)
            nbytes = Mx * V * 4 * (3 if out is not None else 1)
            row[name] = {"us": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        res[f"M{Mx}"] = row
        progress(f"reset temperature M={Mx}: {row}")
    return {"V": V, "logits": "float32 4 x N(0,1), resident (4.9 MB at M = 8)", **res}


def bench_32b_and_stack(args, torch, nv, dev, timer, linear_table):
    """Qwen3-32B-shaped projections: two seeded layers drawn on the device
    (torch's Philox generator, 0.02 * N(0,1) bf16), quantized, and copied by
    device memcpy into args.stack_layers distinct layers; GEMV-only us per
    projection at M = 1, 4, 8 (rotating over the layers), then the layer
    stack's decode step replayed args.stack_steps times at M = 1 and 8."""
    from workloads import QWEN3_32B, activations_bf16
    lins = QWEN3_32B
    gen = torch.Generator(device=dev)
    gen.manual_seed(2606_5)
    seeds = []
    for _ in range(2):
        layer = []
        for L in lins:
            w = (torch.randn((L.N, L.K), generator=gen, device=dev, dtype=torch.float32)
                 * 0.02).to(torch.bfloat16)
            # gate_up in the interleaved row order of the SiLU * mul epilogue
            layer.append(nv.quantize_weight_gate_up(w) if L.name == "gate_up"
                         else nv.quantize_weight(w))
            del w
        seeds.append(layer)
    nl = args.stack_layers
    layers = [seeds[l] if l < 2 else
              [nv.QuantWeight(w.codes.clone(), w.scales.clone(), w.gscale.clone(), w.N, w.K,
                              w.gate_up)
               for w in seeds[l % 2]] for l in range(nl)]
    torch.cuda.synchronize()
    wbytes = sum(w.codes.numel() + w.scales.numel() for w in layers[0])

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    xs = [to_dev(activations_bf16(4, li, 8, L.K, "student_t")) for li, L in enumerate(lins)]
    lin32 = None if args.stack_only else linear_table(
        lins, layers[:max(2, min(nl, int(np.ceil(1.2 * (1 << 30) / wbytes))))], (1, 4, 8), xs)

    hidden, qkv_n, q_cols, ffn = 5120, 10240, 8192, 25600
    stack = {"layers": nl, "weight_bytes_per_step": int(nl * wbytes)}
    for Mx in (1, 8):
        x_in = to_dev(activations_bf16(5, 0, Mx, hidden, "normal"))
        y_out = torch.empty((Mx, hidden), dtype=torch.bfloat16, device=dev)
        st = nv.Stack(Mx, hidden, qkv_n, q_cols, ffn, [tuple(l) for l in layers], x_in, y_out)
        st.run(5)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st.stream)
        st.run(args.stack_steps)
        e1.record(st.stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.stack_steps
        act = (actq_bytes(Mx, hidden) * 2 + actq_bytes(Mx, q_cols) + actq_bytes(Mx, ffn, 4))
        outs = Mx * (qkv_n + hidden + 2 * ffn + hidden) * 2
        lin_act = Mx * (hidden * 2 + q_cols + ffn) * WEIGHT_BYTES_PER_ELEM
        step_b = nl * (wbytes + act + outs + lin_act)
        finite = bool(torch.isfinite(y_out.float()).all().item())
        # the replayed graph against the same step launched call by call
        y_graph = y_out.clone()
        st.run_eager()
        torch.cuda.synchronize()
        same = bool(torch.equal(y_graph.view(torch.int16), y_out.view(torch.int16)))
        stack[f"M{Mx}"] = {"us_per_step": round(ms * 1e3, 1),
                           "GBps": round(step_b / (ms * 1e-3) / 1e9, 1),
                           "frac": round(step_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "replays": args.stack_steps, "output_finite": finite,
                           "graph_matches_eager": same}
        st.close()
        del st
        progress(f"stack M={Mx}: {ms * 1e3:.1f} us per step")
    return {"linears_32b": lin32, "stack_qwen3_32b": stack}


if __name__ == "__main__":
    main()
