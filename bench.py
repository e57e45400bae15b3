#!/usr/bin/env python3
"""Benchmark of the fused GEMM epilogue and the MLP megakernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The primary workload (default: the bf16 FFN
up-projection, M=8192 tokens, K=4096, N=16384, + bias + GELU(erf)) is timed
as K back-to-back steps bracketed by device synchronisation, each step one
coalesce_gemm_bias_act call on inputs already resident in HBM; `value` is its
TFLOP/s.  The same line carries

  * roofline: the dominant kernel's algorithmic FLOPs per launch divided by
    its mean duration from HIP events recorded on the launch stream;
  * mlp: rows/s of the 3-layer (D=128, 2^20 rows) and 5-layer (D=64, 2^22
    rows) softplus megakernels, timed the same way, with their HBM roofline;
  * pages_harness: the "Coalesce" README's timing method for every workload
    -- >= 1 s of warm-up, then 100 runs each preceded by a 512 MiB cache
    flush and bracketed by their own event pair, median / p10 / p90 -- for
    the fused kernel and for the unfused GEMM -> bias -> activation baseline
    (per-layer GEMM -> softplus for the MLPs);
  * mlp_train: the training pair of both MLP workloads -- the training
    forward (which also stores the fp32 hidden activations) and the fused
    backward (weight gradients of every layer and dx) -- each timed the same
    way, with its HBM roofline, and rows/s of one forward + backward step;
  * weight_norm: the fused weight normalisation of both MLPs' weights (all
    layers in one launch) and its backward, against per-layer eager torch
    ops, and the weight-normalised training step (normalise, training
    forward, backward, normalisation backward);
  * variants: four general chains -- two non-square ones and two whose
    weights exceed the LDS (6 x 128, 3 x 256) -- each with the forward, the
    training forward and the backward against their HBM, MFMA and
    transcendental bounds, and one training step; the FFN GEMM with the ReLU / softplus / no epilogue, the
    bf16 GEMM + bias + GELU at five smaller sizes (1024^3 to 4096^3), the
    3 x 128 MLP with ReLU / no hidden activation, and the 3 x 128 MLP on small
    batches, launched eagerly and replayed from a HIP graph;
  * autotune: the ordinary entry points timed before and after per-shape
    autotuning, with the configuration chosen;
  * cpu_baseline: the fp64 oracle timed on this host's cores on a bounded
    sample of the primary workload.
All inputs are synthetic and seeded (datagen).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused GEMM+bias+GELU TFLOP/s & % MFMA peak; MLP megakernel rows/sec"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
# transcendental (v_exp_f32 / v_log_f32) rate: a quarter of the fp32 vector
# lane rate of 78.6e12 per second (256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz)
PEAK_TRANS_PER_S = 78.6e12 / 4
FLUSH_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_ffn_up_gelu")
    ap.add_argument("--no-harness", action="store_true", help="skip the flushed median-of-100 sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mlp", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the MLP training pair")
    ap.add_argument("--no-wn", action="store_true", help="skip the weight-normalisation section")
    ap.add_argument("--no-tune", action="store_true", help="skip the per-shape autotuning section")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the non-square chains and the other epilogues / hidden activations")
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="untimed back-to-back running before the warmup steps of each timed case")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured ceilings (matrix-core rate probe, plain HBM copy)")
    ap.add_argument("--harness-iters", type=int, default=100)
    ap.add_argument("--harness-warmup-ms", type=float, default=1000.0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-traffic", action="store_true",
                    help="also run a known-size read sweep and a known-size read+write kernel "
                         "(for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--fusion-traffic", action="store_true",
                    help="run only the launch sequence whose FETCH_SIZE / WRITE_SIZE counters give the HBM "
                         "traffic of every fused kernel and of its unfused baseline (see fusion_traffic)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the rocprofv3 counter CSVs of two --fusion-traffic runs into profiles/traffic.json "
                         "and print the tables (no GPU needed)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "BENCH_JSON"),
                    help="mean duration of the timed launches of each timed kernel in a rocprofv3 kernel trace "
                         "of a bench.py run, beside that run's JSON line (no GPU needed)")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the workloads shard by rows with no exchange between GPUs, "
              "but runs on more than one GPU are not supported. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import datagen
    import mlp_megakernel_amd as mk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    mk.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush_buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def flush():
        mk.flush_caches(flush_buf, sink)

    # ------------------------------------------------------------------ inputs
    def gemm_case(w):
        A, B, bias = datagen.gemm_inputs(w)
        A, B, bias = A.to(dev), B.to(dev), bias.to(dev)
        odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.out_dtype]
        Y = torch.empty((w.M, w.N), dtype=odt, device=dev)
        Z = torch.empty((w.M, w.N), dtype=A.dtype, device=dev)
        Z2 = torch.empty((w.M, w.N), dtype=A.dtype, device=dev)
        Yu = torch.empty((w.M, w.N), dtype=A.dtype, device=dev)

        def fused():
            mk.gemm_bias_act(A, B, bias, act=w.act, out=Y)

        def unfused():
            mk.gemm_bias_act(A, B, None, act="none", out=Z)
            mk.bias_add(Z, bias, out=Z2)
            mk.activation(Z2, w.act, out=Yu)

        return fused, unfused

    def mlp_case(w):
        x, Ws = datagen.mlp_inputs(w)
        x = x.to(dev)
        Ws = [t.to(dev) for t in Ws]
        out = torch.empty((w.M, w.dims[-1]), dtype=torch.float16, device=dev)
        hs = [torch.empty((w.M, d), dtype=torch.float16, device=dev) for d in w.dims[1:]]
        hs2 = [torch.empty((w.M, d), dtype=torch.float16, device=dev) for d in w.dims[1:]]

        def fused():
            mk.mlp_forward(x, Ws, out=out)

        def unfused():
            h = x
            for l, Wl in enumerate(Ws):
                mk.gemm_bias_act(h, Wl, None, act="none", out=hs[l])
                h = hs[l]
                if l < w.L - 1:
                    mk.activation(h, "softplus", out=hs2[l])
                    h = hs2[l]

        return fused, unfused

    def train_case(w):
        x, Ws = datagen.mlp_inputs(w)
        g = datagen.mlp_grad_output(w)
        x, g = x.to(dev), g.to(dev)
        Ws = [t.to(dev) for t in Ws]
        out = torch.empty((w.M, w.dims[-1]), dtype=torch.float16, device=dev)
        acts = [torch.empty((w.M, d), dtype=torch.float32, device=dev) for d in w.dims[1:-1]]
        dW = [torch.empty((w.dims[l], w.dims[l + 1]), dtype=torch.float32, device=dev) for l in range(w.L)]
        dx = torch.empty_like(x)
        ws = torch.empty(mk.mlp_backward_workspace_size(w.dims, w.M), dtype=torch.uint8, device=dev)

        def fwd():
            mk.mlp_forward_train(x, Ws, out=out, acts=acts)

        def bwd():
            mk.mlp_backward(x, Ws, acts, g, dW=dW, dx=dx, workspace=ws)

        def step():
            fwd()
            bwd()

        fwd()
        torch.cuda.synchronize()
        return fwd, bwd, step, ws.numel()

    # ----------------------------------------------------------------- timing
    def prewarm(fn):
        """Untimed: run fn back to back for --prewarm-ms so that the clocks
        have settled under this load before the warmup steps."""
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < args.prewarm_ms:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()

    def timed_steps(fn, steps, warmup):
        """K back-to-back steps: wall time per step, and the average launch
        duration from one pair of HIP events around the K launches on the
        launch stream (no per-launch event records between the kernels)."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # A full collection of the Python heap inside the timed region would
        # stall the launching thread while the GPU runs dry; one taken between
        # the warm-up and the region leaves the GPU idle for tens of ms, long
        # enough for its clocks to drop and ramp up again during the first
        # timed launches (measured: +25 % on the 0.14 ms MLP launch).  So
        # collect first, then warm up, then time, with the collector off.
        gc.collect()
        gc.disable()
        try:
            prewarm(fn)
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        finally:
            gc.enable()
        return wall * 1e3 / steps, a.elapsed_time(b) / steps

    def pages_harness(fn):
        """>= warmup_ms of continuous GPU work, then N x {flush, event, fn, event}; median."""
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.harness_iters)]
        # the collection before the warm-up, not between it and the runs (see timed_steps)
        gc.collect()
        gc.disable()
        try:
            spent, reps = 0.0, 1
            while spent < args.harness_warmup_ms:
                s.record(stream)
                for _ in range(reps):
                    fn()
                e.record(stream)
                e.synchronize()
                spent += s.elapsed_time(e)
                reps = min(reps * 2, 256)
            for a, b in ev:
                flush()
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
        finally:
            gc.enable()
        t = np.array([a.elapsed_time(b) for a, b in ev])
        return {"median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
                "p90_ms": float(np.percentile(t, 90)), "iters": int(args.harness_iters)}

    def roofline_gemm(w, mean_ms):
        flops = w.flops()
        kern = "gemm32_kernel" if w.in_dtype == "f32" else "gemm16_kernel"
        ach = flops / (mean_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[w.in_dtype]
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": measured_traffic(kern + "/" + w.name), "kernel": kern,
                "algorithmic_flop_per_launch": flops,
                "algorithmic_bytes_per_launch": w.bytes(), "mean_launch_ms": round(mean_ms, 5)}

    def roofline_mlp(w, mean_ms):
        by = w.bytes()
        trans = 2.0 * w.M * sum(w.dims[1:-1])
        ach = by / (mean_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic("mlp_kernel/" + w.name),
                "kernel": "mlp_kernel",
                "algorithmic_bytes_per_launch": by, "algorithmic_flop_per_launch": w.flops(),
                "mfma_tflops": round(w.flops() / (mean_ms * 1e-3) / 1e12, 2), "mean_launch_ms": round(mean_ms, 5),
                # the co-bound: two transcendentals (exp2, log2) per hidden unit and row
                "valu": {"bound": "alu", "achieved": round(trans / (mean_ms * 1e-3) / 1e12, 3),
                         "peak": round(PEAK_TRANS_PER_S / 1e12, 3), "unit": "T transcendentals/s",
                         "frac": round(trans / (mean_ms * 1e-3) / PEAK_TRANS_PER_S, 4)}}

    def matrix_ceiling():
        """What the matrix cores sustain on this board with nothing else
        sharing the time: the library's rate probe (one 8-wave workgroup per
        CU, the 256 x 256 GEMM wave's 4 x 8 block of bf16 16x16x32 MFMAs on
        register operands) with the FFN's operand distribution (A ~ N(0, 1),
        B ~ N(0, 1/64), 64 distinct sets) and with all-zero operands, each
        timed like the workloads (pre-warm, 20 back-to-back launches), with
        the engine clock from the kernel's own counters."""
        nsets, iters = 64, 1024
        gen = torch.Generator().manual_seed(20)
        ops = torch.randn((nsets, 24, 64, 8), generator=gen)
        ops[:, list(range(4, 12)) + list(range(16, 24))] *= 0.125
        ops = ops.to(torch.bfloat16).to(dev)
        waves = mk.matrix_rate_waves()
        sink = torch.empty(waves * 64, dtype=torch.float32, device=dev)
        clocks = torch.zeros(waves * 2, dtype=torch.int64, device=dev)
        out = {"probe": "one 8-wave workgroup per CU, %d rounds of 64 bf16 16x16x32 MFMAs per wave on register "
                        "operands (2^20 FLOP per round and wave)" % iters}
        for name, o in (("ffn_operands", ops), ("zero_operands", torch.zeros_like(ops))):
            khz = [0]

            def run():
                khz[0] = mk.matrix_rate(o, iters, sink, clocks)[1]

            _, ev = timed_steps(run, 20, 5)
            c = clocks.view(-1, 2).double().sum(0).cpu()
            flop = float(waves) * iters * 2 ** 20
            out[name] = {"tflops": round(flop / (ev * 1e-3) / 1e12, 1), "launch_ms": round(ev, 5),
                         "engine_clock_ghz": round(float(c[0] / c[1]) * khz[0] / 1e6, 3),
                         "frac_of_peak": round(flop / (ev * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4)}
        return out

    def copy_ceiling(w):
        """A plain device-to-device copy (torch's) of the MLP's input bytes:
        the same read and write volume as the megakernel, with no compute."""
        src = torch.empty(w.M * w.dims[0], dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        _, ev = timed_steps(lambda: dst.copy_(src), 20, 5)
        by = 2.0 * src.numel() * 2
        return {"bytes": by, "launch_ms": round(ev, 5), "achieved": round(by / (ev * 1e-3) / 1e9, 1), "unit": "GB/s"}

    def bounds(ms, by, flop, trans):
        """Lower-bound times of one launch (HBM bytes, MFMA flops at the fp16
        dense peak, transcendentals at PEAK_TRANS_PER_S) against the measured
        mean: each as achieved / peak, and the largest as the roofline."""
        kinds = {"hbm": (by / (PEAK_HBM_GBS * 1e9), by / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"),
                 "mfma": (flop / (PEAK_TFLOPS["f16"] * 1e12), flop / (ms * 1e-3) / 1e12, PEAK_TFLOPS["f16"], "TFLOP/s"),
                 "alu": (trans / PEAK_TRANS_PER_S, trans / (ms * 1e-3) / 1e12, round(PEAK_TRANS_PER_S / 1e12, 3),
                         "T transcendentals/s")}
        out = {k: {"achieved": round(v[1], 2), "peak": v[2], "unit": v[3], "frac": round(v[1] / v[2], 4)}
               for k, v in kinds.items()}
        top = max(kinds, key=lambda k: kinds[k][0])
        out["bound"] = top
        out["frac"] = out[top]["frac"]
        out["mean_launch_ms"] = round(ms, 5)
        out["algorithmic_bytes_per_launch"] = by
        out["algorithmic_flop_per_launch"] = flop
        return out

    def chain_case(w):
        """Forward, training forward, backward and one training step of a
        general chain, each with its bounds (bytes: x, out, the fp32
        activations and dx at their true widths; flops at the true widths)."""
        x, Ws = datagen.mlp_inputs(w)
        x, Ws = x.to(dev), [t.to(dev) for t in Ws]
        g_out = datagen.mlp_grad_output(w).to(dev)
        out = torch.empty((w.M, w.dims[-1]), dtype=torch.float16, device=dev)
        H = max(w.dims[1:-1])  # the activations share one pitch
        acts = [torch.empty((w.M, H), dtype=torch.float32, device=dev)[:, :d] for d in w.dims[1:-1]]
        dW = [torch.empty(t.shape, dtype=torch.float32, device=dev) for t in Ws]
        dx = torch.empty_like(x)
        wsp = torch.empty(mk.mlp_backward_workspace_size(w.dims, w.M), dtype=torch.uint8, device=dev)
        mx = max(w.dims)
        P = 64 if mx <= 64 else 128 if mx <= 128 else 256
        resident = (P == 64 and w.L <= 8) or (P == 128 and w.L <= 4)
        hidden = sum(w.dims[1:-1])
        trans = 2.0 * w.M * hidden  # exp2 and log2 per hidden unit and row

        def fwd():
            mk.mlp_forward(x, Ws, out=out)

        def fwd_train():
            mk.mlp_forward_train(x, Ws, out=out, acts=acts)

        def bwd():
            mk.mlp_backward(x, Ws, acts, g_out, dW=dW, dx=dx, workspace=wsp)

        def step():
            fwd_train()
            bwd()

        res = {"dims": list(w.dims), "rows": w.M, "kernel_width": P,
               "forward_kernel": "mlp_kernel" if resident else "mlp_stream_kernel",
               "backward_kernels": ("mlp_bwd_kernel + mlp_bwd_reduce" if resident else
                                    " + ".join(stream_backward_kernels(w.dims)))}
        if resident:
            res["padded_flop_factor"] = round(2.0 * w.M * w.L * P * P / w.flops(), 3)
        f_ms, f_ev = timed_steps(fwd, max(20, args.steps), 10)
        res["forward_ms"] = round(f_ms, 5)
        res["forward_rows_per_s"] = round(w.M / (f_ms * 1e-3), 1)
        res["forward_roofline"] = bounds(f_ev, w.bytes(), w.flops(), trans)
        res["forward_roofline"]["traffic"] = None if resident else measured_traffic("stream_forward/" + w.name)
        t_ms, t_ev = timed_steps(fwd_train, max(20, args.steps), 10)
        res["forward_train_ms"] = round(t_ms, 5)
        res["forward_train_roofline"] = bounds(t_ev, w.bytes() + 4.0 * w.M * hidden, w.flops(), trans)
        res["forward_train_roofline"]["traffic"] = (None if resident else
                                                    measured_traffic("stream_forward_train/" + w.name))
        b_ms, b_ev = timed_steps(bwd, max(20, args.steps), 10)
        bb = w.M * (2.0 * w.dims[0] + 2.0 * w.dims[-1] + 4.0 * hidden + 2.0 * w.dims[0])
        res["backward_ms"] = round(b_ms, 5)
        res["backward_roofline"] = bounds(b_ev, bb, 2.0 * w.flops(), 0.0)
        if not resident:
            # the fp16 dz_l each layer writes and the next one reads back
            res["backward_roofline"]["dz_roundtrip_bytes"] = 4.0 * w.M * hidden
        res["backward_roofline"]["traffic"] = None if resident else measured_traffic("stream_backward/" + w.name)
        res["backward_workspace_bytes"] = wsp.numel()
        s_ms, _ = timed_steps(step, max(20, args.steps), 10)
        res["train_step_ms"] = round(s_ms, 5)
        res["train_step_rows_per_s"] = round(w.M / (s_ms * 1e-3), 1)
        return res

    if args.fusion_traffic:
        fusion_traffic(gemm_case, mlp_case, train_case, flush)
        return

    result = {}
    prim = datagen.WORKLOADS[args.workload]
    is_mlp = isinstance(prim, datagen.MlpWorkload)

    # -------------------------------------------------------- primary workload
    print("bench: generating %s" % prim.name, file=sys.stderr, flush=True)
    fused, unfused = (mlp_case if is_mlp else gemm_case)(prim)
    ms_step, mean_kernel_ms = timed_steps(fused, args.steps, args.warmup)
    if is_mlp:
        value = prim.M / (ms_step * 1e-3)
        unit, dtype = "rows/s", "f16"
        roof = roofline_mlp(prim, mean_kernel_ms)
        cfg = {"workload": prim.name, "rows": prim.M, "dims": list(prim.dims), "hidden_act": "softplus"}
    else:
        value = prim.flops() / (ms_step * 1e-3) / 1e12
        unit, dtype = "TFLOP/s", prim.in_dtype
        roof = roofline_gemm(prim, mean_kernel_ms)
        cfg = {"workload": prim.name, "M": prim.M, "N": prim.N, "K": prim.K, "act": "gelu_erf",
               "in_dtype": prim.in_dtype, "out_dtype": prim.out_dtype, "accumulate": "f32"}
    cfg["description"] = prim.description
    result.update({"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
                   "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
                   "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": cfg})
    if not is_mlp:
        result["pct_mfma_peak"] = round(100.0 * value / PEAK_TFLOPS[prim.in_dtype], 2)
    result["roofline"] = roof
    if not is_mlp and prim.in_dtype == "bf16" and not args.no_ceiling:
        print("bench: matrix-core ceiling", file=sys.stderr, flush=True)
        ceil = matrix_ceiling()
        ceil["frac_of_sustained"] = round(roof["achieved"] / ceil["ffn_operands"]["tflops"], 4)
        roof["measured_ceiling"] = ceil
    if is_mlp and prim.dims[0] == prim.dims[-1] and not args.no_ceiling:
        cc = copy_ceiling(prim)
        cc["frac_of_copy"] = round(roof["achieved"] / cc["achieved"], 4)
        roof["measured_ceiling"] = cc
    harness = {}
    if not args.no_harness:
        print("bench: pages harness %s" % prim.name, file=sys.stderr, flush=True)
        hf, hu = pages_harness(fused), pages_harness(unfused)
        harness[prim.name] = {"fused": hf, "unfused": hu, "fused_speedup": round(hu["median_ms"] / hf["median_ms"], 4)}
        if not is_mlp:
            harness[prim.name]["fused_tflops"] = round(prim.flops() / (hf["median_ms"] * 1e-3) / 1e12, 2)
    del fused, unfused
    torch.cuda.empty_cache()

    # ------------------------------------------------------------- MLP metrics
    if not args.no_mlp:
        mlp_res = {}
        for w in (datagen.MLP3, datagen.MLP5):
            if w.name == prim.name:
                continue
            print("bench: %s" % w.name, file=sys.stderr, flush=True)
            f, u = mlp_case(w)
            ms, mk_ms = timed_steps(f, max(20, args.steps), 10)
            mlp_res[w.name] = {"rows_per_s": round(w.M / (ms * 1e-3), 1), "ms_per_call": round(ms, 5),
                               "roofline": roofline_mlp(w, mk_ms)}
            if not args.no_ceiling and w.dims[0] == w.dims[-1]:
                cc = copy_ceiling(w)
                cc["frac_of_copy"] = round(mlp_res[w.name]["roofline"]["achieved"] / cc["achieved"], 4)
                mlp_res[w.name]["roofline"]["measured_ceiling"] = cc
            if not args.no_harness:
                hf, hu = pages_harness(f), pages_harness(u)
                harness[w.name] = {"fused": hf, "unfused": hu, "rows_per_s": round(w.M / (hf["median_ms"] * 1e-3), 1),
                                   "fused_speedup": round(hu["median_ms"] / hf["median_ms"], 4)}
            del f, u
            torch.cuda.empty_cache()
        result["mlp"] = mlp_res
        if datagen.MLP3.name in mlp_res:
            result["mlp_rows_per_sec"] = mlp_res[datagen.MLP3.name]["rows_per_s"]

    # ------------------------------------------------------- MLP training pair
    if not args.no_train:
        train_res = {}
        for w in (datagen.MLP3, datagen.MLP5):
            print("bench: training pair %s" % w.name, file=sys.stderr, flush=True)
            fwd, bwd, step, ws_bytes = train_case(w)
            hidden = sum(w.dims[1:-1])
            # algorithmic bytes per row: the training forward reads x and
            # writes out and the fp32 activations; the backward reads x, dout
            # and the activations and writes dx (the weights and dW are a few
            # KB; the per-workgroup partial sums are reported separately)
            fb = w.M * (2.0 * w.dims[0] + 2.0 * w.dims[-1] + 4.0 * hidden)
            bb = w.M * (2.0 * w.dims[0] + 2.0 * w.dims[-1] + 4.0 * hidden + 2.0 * w.dims[0])
            res = {}
            for name, fn, by, kern in (("forward_train", fwd, fb, "mlp_kernel"),
                                       ("backward", bwd, bb, "mlp_bwd_kernel + mlp_bwd_reduce")):
                ms, ev_ms = timed_steps(fn, max(20, args.steps), 10)
                ach = by / (ev_ms * 1e-3) / 1e9
                res[name] = {"ms_per_call": round(ms, 5), "rows_per_s": round(w.M / (ms * 1e-3), 1),
                             "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                                          "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                                          "traffic": measured_traffic(name + "/" + w.name), "kernel": kern,
                                          "algorithmic_bytes_per_launch": by, "mean_launch_ms": round(ev_ms, 5)}}
            res["backward"]["workspace_bytes"] = ws_bytes
            ms, _ = timed_steps(step, max(20, args.steps), 10)
            res["step_ms"] = round(ms, 5)
            res["step_rows_per_s"] = round(w.M / (ms * 1e-3), 1)
            train_res[w.name] = res
            del fwd, bwd, step
            torch.cuda.empty_cache()
        result["mlp_train"] = train_res

    # ------------------------------------------------ weight normalisation
    if not args.no_wn:
        wn_res = {}
        for w in (datagen.MLP3, datagen.MLP5):
            print("bench: weight normalisation %s" % w.name, file=sys.stderr, flush=True)
            vs, gs = datagen.wn_inputs(w)
            vs = [t.to(dev).contiguous() for t in vs]
            gs = [t.to(dev).contiguous() for t in gs]
            Ws = [torch.empty_like(v) for v in vs]
            dWs = [torch.randn(v.shape, device=dev, dtype=torch.float32) for v in vs]

            def fused_wn():
                mk.weight_norm(vs, gs, Ws)

            def fused_wn_bwd():
                mk.weight_norm_backward(vs, gs, dWs)

            def eager_wn():  # per layer: norm, divide, multiply, cast (several launches each)
                for v, g, W in zip(vs, gs, Ws):
                    W.copy_((g.float() * v.float() / v.float().norm(dim=0)).to(v.dtype))

            by = sum(4.0 * v.numel() + 2.0 * g.numel() for v, g in zip(vs, gs))
            f_ms, f_ev = timed_steps(fused_wn, max(50, args.steps), 10)
            b_ms, _ = timed_steps(fused_wn_bwd, max(50, args.steps), 10)
            e_ms, _ = timed_steps(eager_wn, max(50, args.steps), 10)
            # the weight-normalised training step of the page's quick start
            x = datagen.mlp_inputs(w)[0].to(dev)
            g_out = datagen.mlp_grad_output(w).to(dev)
            acts = [torch.empty((w.M, d), dtype=torch.float32, device=dev) for d in w.dims[1:-1]]
            out = torch.empty((w.M, w.dims[-1]), dtype=torch.float16, device=dev)
            dW = [torch.empty(v.shape, dtype=torch.float32, device=dev) for v in vs]
            dx = torch.empty_like(x)
            wsp = torch.empty(mk.mlp_backward_workspace_size(w.dims, w.M), dtype=torch.uint8, device=dev)

            def wn_step():
                mk.weight_norm(vs, gs, Ws)
                mk.mlp_forward_train(x, Ws, out=out, acts=acts)
                mk.mlp_backward(x, Ws, acts, g_out, dW=dW, dx=dx, workspace=wsp)
                mk.weight_norm_backward(vs, gs, dW)

            s_ms, _ = timed_steps(wn_step, max(20, args.steps), 10)
            wn_res[w.name] = {"layers": w.L, "fused_us": round(f_ms * 1e3, 2), "fused_launches": 1,
                              "eager_us": round(e_ms * 1e3, 2), "eager_launches": "several per layer",
                              "fused_speedup": round(e_ms / f_ms, 2), "backward_fused_us": round(b_ms * 1e3, 2),
                              "bytes_per_call": by, "achieved_GBps": round(by / (f_ev * 1e-3) / 1e9, 1),
                              "bound": "launch latency (the matrices are a few KB)",
                              "training_step_ms": round(s_ms, 5),
                              "training_step_rows_per_s": round(w.M / (s_ms * 1e-3), 1)}
            del x, g_out, acts, out, dW, dx, wsp
            torch.cuda.empty_cache()
        result["weight_norm"] = wn_res

    # ------------------------------- non-square chains, other epilogues
    if not args.no_variants:
        var = {}
        # the general chains: non-square (narrow input / output) ones that the
        # resident megakernel runs padded, and chains whose weights exceed the
        # LDS (layer-streaming forward, layer-by-layer backward)
        for w in (datagen.MLP_NS1, datagen.MLP_NS2, datagen.MLP6, datagen.MLP3W):
            print("bench: general chain %s" % w.name, file=sys.stderr, flush=True)
            var[w.name] = chain_case(w)
            torch.cuda.empty_cache()
        # the FFN GEMM with the other epilogues (GELU is the primary line)
        g = datagen.BF16_FFN
        A, B, bias = datagen.gemm_inputs(g)
        A, B, bias = A.to(dev), B.to(dev), bias.to(dev)
        Y = torch.empty((g.M, g.N), dtype=torch.bfloat16, device=dev)
        epi = {}
        for act in ("relu", "softplus", "none"):
            print("bench: FFN GEMM epilogue %s" % act, file=sys.stderr, flush=True)
            _, ev = timed_steps(lambda: mk.gemm_bias_act(A, B, bias, act=act, out=Y), max(20, args.steps), 5)
            epi[act] = {"mean_launch_ms": round(ev, 5), "tflops": round(g.flops() / (ev * 1e-3) / 1e12, 1),
                        "frac_of_peak": round(g.flops() / (ev * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4)}
        var["bf16_ffn_up_epilogues"] = epi
        del A, B, bias, Y
        torch.cuda.empty_cache()
        # the 16-bit GEMM (bias + GELU) at smaller sizes, where the launcher
        # takes 128 x 128 tiles while all of them fit on the CUs at once
        sizes = {}
        for (M, N, K) in ((1024, 1024, 1024), (2048, 2048, 2048), (4096, 2048, 4096), (3072, 3072, 4096),
                          (4096, 4096, 4096)):
            print("bench: bf16 GEMM %dx%dx%d" % (M, N, K), file=sys.stderr, flush=True)
            A, B, bias = datagen.gemm_inputs(g, M=M, N=N, K=K)
            A, B, bias = A.to(dev), B.to(dev), bias.to(dev)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            _, ev = timed_steps(lambda: mk.gemm_bias_act(A, B, bias, act="gelu", out=Y), max(20, args.steps), 5)
            fl = 2.0 * M * N * K
            sizes["%dx%dx%d" % (M, N, K)] = {"mean_launch_ms": round(ev, 5), "tflops": round(fl / (ev * 1e-3) / 1e12, 1),
                                             "frac_of_peak": round(fl / (ev * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
                                             "tiles_128": ((M + 127) // 128) * ((N + 127) // 128)}
            del A, B, bias, Y
        var["bf16_gemm_sizes"] = sizes
        torch.cuda.empty_cache()
        # the 3 x 128 MLP with the other hidden activations
        x, Ws = datagen.mlp_inputs(datagen.MLP3)
        x, Ws = x.to(dev), [t.to(dev) for t in Ws]
        out = torch.empty((datagen.MLP3.M, 128), dtype=torch.float16, device=dev)
        hid = {}
        for act in ("relu", "none"):
            print("bench: MLP 3x128 hidden activation %s" % act, file=sys.stderr, flush=True)
            _, ev = timed_steps(lambda: mk.mlp_forward(x, Ws, hidden_act=act, out=out), max(20, args.steps), 10)
            hid[act] = {"mean_launch_ms": round(ev, 5), "rows_per_s": round(datagen.MLP3.M / (ev * 1e-3), 1)}
        var["fp16_mlp3_d128_hidden_acts"] = hid
        # small batches, where the launch dominates: per-call time of eager
        # back-to-back launches and of the same calls replayed from a HIP graph
        small = {}
        for m in (64, 1024, 8192):
            xs = x[:m].contiguous()
            os_ = torch.empty((m, 128), dtype=torch.float16, device=dev)
            _, eager_ms = timed_steps(lambda: mk.mlp_forward(xs, Ws, out=os_), 200, 20)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                mk.mlp_forward(xs, Ws, out=os_)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(20):
                    mk.mlp_forward(xs, Ws, out=os_)
            _, graph_ms = timed_steps(graph.replay, 20, 3)
            small["M%d" % m] = {"eager_us": round(eager_ms * 1e3, 2), "graph_us": round(graph_ms * 1e3 / 20, 2)}
            del graph
        var["fp16_mlp3_d128_small_batch"] = small
        del x, Ws, out
        torch.cuda.empty_cache()
        result["variants"] = var

    # ------------------------------------------------- per-shape autotuning
    if not args.no_tune:
        # The ordinary entry point timed before tuning (the launchers' default
        # configuration) and after it (the recorded winner), both as the
        # device time per call of 20 calls replayed from a HIP graph (eager
        # calls of a few microseconds are bound by the host, which would hide
        # the configurations' difference); the record is cleared afterwards
        # so that nothing else in this run depends on it.
        def graph_call_ms(fn, calls=20, reps=10):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(calls):
                    fn()
            # replays for at least 200 ms first: the case's inputs were just
            # generated on the host, and a GPU left idle that long has lowered
            # its clocks (measured without this: the same configuration 7 %
            # faster after tuning than before it)
            t0 = time.perf_counter()
            while True:
                for _ in range(3):
                    graph.replay()
                torch.cuda.synchronize()
                if time.perf_counter() - t0 > 0.2:
                    break
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                graph.replay()
            b.record(stream)
            torch.cuda.synchronize()
            del graph
            return a.elapsed_time(b) / (reps * calls)

        tune_res = {"search_space": {
            "gemm_bf16_fp16": "compiled tiles 256x256 (8 waves), 128x128, 64x64 x persistent grid (occupancy, 1/2 "
                              "and 3/4 of the tile's workgroup slots, one per tile) x tile-group height 4/8/16",
            "gemm_fp32": "compiled tiles 128x128, 64x64, 32x32, 64x32 x tile-group height 4/8/16",
            "mlp_resident": "the launcher's choice and the three compiled launch configurations (32-row "
                            "wave tiles with width 128: 12 waves / 3 per SIMD or 8 / 2, width 64: 16 / 4 or "
                            "12 / 3; 16-row tiles with 12 / 16 waves) x grid (default, CUs/4, /2, x1, x2, x3)",
            "mlp_streamed": "grid (default, CUs/4, /2, x1, x2, x3)",
            "validation": "bitwise equality with the default configuration's output",
            "timing": "device time per call: 20 calls in a HIP graph, replayed for 200 ms, then 10 timed "
                      "replays; before and after tuning"}}
        cases = [("gemm", datagen.BF16_FFN, None), ("gemm", datagen.FP32_1024, None),
                 ("gemm", datagen.FP32_2048, None)]
        cases += [("mlp", datagen.MLP3, m) for m in (1 << 12, 1 << 14, 1 << 16, 1 << 20)]
        cases += [("mlp", datagen.MLP5, m) for m in (1 << 14, 1 << 22)]
        cases += [("mlp", datagen.MLP_NS1, 1 << 20), ("mlp", datagen.MLP6, 1 << 20)]
        for kind, w, m in cases:
            label = w.name if m is None else "%s_M%d" % (w.name, m)
            print("bench: autotune %s" % label, file=sys.stderr, flush=True)
            mk.autotune_clear()
            if kind == "gemm":
                A, B, bias = datagen.gemm_inputs(w)
                A, B, bias = A.to(dev), B.to(dev), bias.to(dev)
                odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.out_dtype]
                Y = torch.empty((w.M, w.N), dtype=odt, device=dev)

                def run():
                    mk.gemm_bias_act(A, B, bias, act=w.act, out=Y)

                def tune():
                    return mk.autotune_gemm_bias_act(A, B, bias, act=w.act, out=Y, iters=5)[1]
            else:
                x, Ws = datagen.mlp_inputs(w, M=m)
                x, Ws = x.to(dev), [t.to(dev) for t in Ws]
                Y = torch.empty((m, w.dims[-1]), dtype=torch.float16, device=dev)

                def run():
                    mk.mlp_forward(x, Ws, out=Y)

                def tune():
                    return mk.autotune_mlp_forward(x, Ws, out=Y, iters=5)[1]
            d_ev = graph_call_ms(run)
            ref = Y.clone()
            rep = tune()
            t_ev = graph_call_ms(run)
            same = bool(torch.equal(Y, ref))
            tune_res[label] = {"default_us": round(d_ev * 1e3, 2), "tuned_us": round(t_ev * 1e3, 2),
                               "speedup": round(d_ev / t_ev, 4), "bitwise_equal_to_default": same,
                               "chosen": {"grid": rep["grid"], "group_m": rep["group_m"], "variant": rep["variant"]},
                               "candidates": rep["candidates"], "valid": rep["valid"]}
            if kind == "gemm":
                tune_res[label]["tuned_tflops"] = round(w.flops() / (t_ev * 1e-3) / 1e12, 1)
            else:
                tune_res[label]["tuned_rows_per_s"] = round(m / (t_ev * 1e-3), 1)
            mk.autotune_clear()
            del run, tune, Y, ref
            torch.cuda.empty_cache()
        result["autotune"] = tune_res

    # ------------------------------------------- the other GEMM workloads (harness)
    if not args.no_harness:
        for name in ("fp32_gemm_gelu_512", "fp32_gemm_gelu_1024", "fp32_gemm_gelu_2048", "fp32_gemm_gelu_4096",
                     "bf16_ffn_up_gelu"):
            w = datagen.WORKLOADS[name]
            if name == prim.name:
                continue
            print("bench: pages harness %s" % name, file=sys.stderr, flush=True)
            f, u = gemm_case(w)
            hf, hu = pages_harness(f), pages_harness(u)
            harness[name] = {"fused": hf, "unfused": hu, "fused_speedup": round(hu["median_ms"] / hf["median_ms"], 4),
                             "fused_tflops": round(w.flops() / (hf["median_ms"] * 1e-3) / 1e12, 2),
                             "pct_peak": round(100 * w.flops() / (hf["median_ms"] * 1e-3) / 1e12 /
                                               PEAK_TFLOPS[w.in_dtype], 2)}
            del f, u
            torch.cuda.empty_cache()
        result["pages_harness"] = harness

    if args.calibrate_traffic:
        # Known-size kernels for scaling the FETCH_SIZE / WRITE_SIZE counters:
        # the flush sweep reads exactly 512 MiB; the activation kernel on a
        # 256 MiB fp16 tensor reads 256 MiB and writes 256 MiB.
        print("bench: traffic calibration kernels", file=sys.stderr, flush=True)
        flush()
        t = torch.zeros((8192, 16384), dtype=torch.float16, device=dev)
        mk.activation(t, "none", out=torch.empty_like(t))
        torch.cuda.synchronize()
        result["traffic_calibration"] = {"flush_read_bytes": FLUSH_BYTES, "activation_read_bytes": t.numel() * 2,
                                         "activation_write_bytes": t.numel() * 2}

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(prim, args.cpu_seconds)

    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------------
# HBM traffic of the fused kernels and of their unfused baselines
# ----------------------------------------------------------------------------
# The launch sequence of --fusion-traffic, in order, as (section, workload,
# role, kernels launched).  Only the library's own kernels are listed; torch's
# (input fills, copies) are skipped when the counters are matched to it.
TRAFFIC_GEMMS = ("fp32_gemm_gelu_512", "fp32_gemm_gelu_1024", "fp32_gemm_gelu_2048", "fp32_gemm_gelu_4096",
                 "bf16_ffn_up_gelu")
TRAFFIC_MLPS = ("fp16_mlp3_d128", "fp16_mlp5_d64")
TRAFFIC_CHAINS = ("fp16_mlp6_d128", "fp16_mlp3_d256")  # the layer-streaming forward and per-layer backward
WARM_LAUNCHES = 3


def traffic_plan():
    import datagen
    plan = [("calibration", "flush_512MiB", "read", ["flush_kernel"]),
            ("calibration", "activation_256MiB", "read+write", ["activation_kernel"])]
    for name in TRAFFIC_GEMMS:
        w = datagen.WORKLOADS[name]
        g = "gemm32_kernel" if w.in_dtype == "f32" else "gemm16_kernel"
        plan += [("fusion", name, "flush", ["flush_kernel"]), ("fusion", name, "fused_cold", [g]),
                 ("fusion", name, "flush", ["flush_kernel"]),
                 ("fusion", name, "unfused_cold", [g, "bias_add_kernel", "activation_kernel"])]
        plan += [("warm", name, "fused_warm", [g])] * WARM_LAUNCHES
    for name in TRAFFIC_MLPS:
        w = datagen.WORKLOADS[name]
        chain = []
        for l in range(w.L):
            chain.append("gemm16_kernel")
            if l < w.L - 1:
                chain.append("activation_kernel")
        plan += [("fusion", name, "flush", ["flush_kernel"]), ("fusion", name, "fused_cold", ["mlp_kernel"]),
                 ("fusion", name, "flush", ["flush_kernel"]), ("fusion", name, "unfused_cold", chain)]
        plan += [("warm", name, "fused_warm", ["mlp_kernel"])] * WARM_LAUNCHES
    for name in TRAFFIC_MLPS:
        plan += [("warm", name, "forward_train_first", ["mlp_kernel"])]  # train_case's own first call
        plan += [("warm", name, "forward_train_warm", ["mlp_kernel"]),
                 ("warm", name, "backward_warm", ["mlp_bwd_kernel", "mlp_bwd_reduce"])] * WARM_LAUNCHES
    for name in TRAFFIC_CHAINS:
        w = datagen.WORKLOADS[name]
        plan += [("warm", name, "stream_forward_warm", ["mlp_stream_kernel"])] * WARM_LAUNCHES
        plan += [("warm", name, "stream_forward_train_warm", ["mlp_stream_kernel"]),
                 ("warm", name, "stream_backward_warm", stream_backward_kernels(w.dims))] * WARM_LAUNCHES
    return plan


def stream_backward_kernels(dims):
    """Dispatch sequence of the layer-by-layer backward: from the top, two
    layers per launch while every width is at most 128 (then one reduction
    launch for both), else one layer per launch and its reduction."""
    seq, l = [], len(dims) - 2
    pairs = max(dims) <= 128
    while l >= 0:
        if pairs and l >= 1:
            seq += ["mlp_layer2_bwd_kernel", "layer_bwd_reduce"]
            l -= 2
        else:
            seq += ["mlp_layer_bwd_kernel", "layer_bwd_reduce"]
            l -= 1
    return seq


def fusion_traffic(gemm_case, mlp_case, train_case, flush):
    """Launch exactly the sequence of traffic_plan(): the two calibration
    kernels; then for every workload a flushed fused launch, a flushed
    unfused chain (GEMM -> bias-add -> activation; for the MLPs the per-layer
    GEMM -> softplus chain with fp16 intermediates) and WARM_LAUNCHES
    back-to-back fused launches (the regime of the timed steps); then the
    training pair of both MLPs back to back.  Under rocprofv3 --pmc
    FETCH_SIZE (then WRITE_SIZE) every dispatch gets its own counter value;
    summarize_counters matches them to this plan."""
    import torch

    import datagen
    import mlp_megakernel_amd as mk

    dev = torch.device("cuda:0")
    flush()
    t = torch.zeros((8192, 16384), dtype=torch.float16, device=dev)
    mk.activation(t, "none", out=torch.empty_like(t))
    torch.cuda.synchronize()
    del t
    for name in TRAFFIC_GEMMS + TRAFFIC_MLPS:
        w = datagen.WORKLOADS[name]
        print("bench: fusion traffic %s" % name, file=sys.stderr, flush=True)
        fused, unfused = (mlp_case if name in TRAFFIC_MLPS else gemm_case)(w)
        torch.cuda.synchronize()
        flush()
        fused()
        flush()
        unfused()
        for _ in range(WARM_LAUNCHES):
            fused()
        torch.cuda.synchronize()
        del fused, unfused
        torch.cuda.empty_cache()
    for name in TRAFFIC_MLPS:
        w = datagen.WORKLOADS[name]
        print("bench: training-pair traffic %s" % name, file=sys.stderr, flush=True)
        fwd, bwd, step, _ = train_case(w)  # (its first training forward is in the plan)
        torch.cuda.synchronize()
        for _ in range(WARM_LAUNCHES):
            fwd()
            bwd()
        torch.cuda.synchronize()
        del fwd, bwd, step
        torch.cuda.empty_cache()
    for name in TRAFFIC_CHAINS:
        w = datagen.WORKLOADS[name]
        print("bench: streamed-chain traffic %s" % name, file=sys.stderr, flush=True)
        x, Ws = datagen.mlp_inputs(w)
        x, Ws = x.to(dev), [t.to(dev) for t in Ws]
        g = datagen.mlp_grad_output(w).to(dev)
        out = torch.empty((w.M, w.dims[-1]), dtype=torch.float16, device=dev)
        acts = [torch.empty((w.M, d), dtype=torch.float32, device=dev) for d in w.dims[1:-1]]
        dW = [torch.empty(t.shape, dtype=torch.float32, device=dev) for t in Ws]
        dx = torch.empty_like(x)
        ws = torch.empty(mk.mlp_backward_workspace_size(w.dims, w.M), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(WARM_LAUNCHES):
            mk.mlp_forward(x, Ws, out=out)
        for _ in range(WARM_LAUNCHES):
            mk.mlp_forward_train(x, Ws, out=out, acts=acts)
            mk.mlp_backward(x, Ws, acts, g, dW=dW, dx=dx, workspace=ws)
        torch.cuda.synchronize()
        del x, Ws, g, out, acts, dW, dx, ws
        torch.cuda.empty_cache()
    print(json.dumps({"fusion_traffic_plan": traffic_plan()}), flush=True)


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _library_rows(rows):
    """The library's dispatches (kernels in namespace coalesce), in dispatch order."""
    out = [r for r in rows if "coalesce" in r["Kernel_Name"]]
    out.sort(key=lambda r: int(r["Dispatch_Id"]))
    return out


def _match_plan(rows, plan, what):
    """Split the library's dispatches along the plan, checking each kernel name."""
    out, i = [], 0
    for sec, wl, role, kernels in plan:
        vals = []
        for k in kernels:
            if i >= len(rows) or k not in rows[i]["Kernel_Name"]:
                raise SystemExit("%s: dispatch %d is %r, the plan expects %s (%s %s)"
                                 % (what, i, rows[i]["Kernel_Name"] if i < len(rows) else None, k, wl, role))
            vals.append(float(rows[i]["Counter_Value"]))
            i += 1
        out.append((sec, wl, role, kernels, vals))
    return out


def summarize_counters(fetch_csv, write_csv):
    """profiles/traffic.json from the FETCH_SIZE and WRITE_SIZE runs of
    --fusion-traffic: calibration factors, per-workload fused and unfused
    bytes with the model's prediction, and the per-launch traffic of the
    timed kernels (back-to-back, as in the timed steps) that the bench line
    reports while the kernels' sources are unchanged."""
    import hashlib

    import datagen

    plan = traffic_plan()
    fe = _match_plan(_library_rows(_read_csv(fetch_csv)), plan, "FETCH_SIZE")
    wr = _match_plan(_library_rows(_read_csv(write_csv)), plan, "WRITE_SIZE")
    KiB = 1024.0
    f_fac = FLUSH_BYTES / (fe[0][4][0] * KiB)
    w_fac = (8192 * 16384 * 2) / (wr[1][4][0] * KiB)
    C = "mlp_megakernel_amd/csrc/"
    srcs = {"gemm16_kernel": [C + "gemm16.hip", C + "common.hpp"], "gemm32_kernel": [C + "gemm32.hip", C + "common.hpp"],
            "mlp_kernel": [C + "mlp.hip", C + "mlp_small.hip", C + "mlp_alt.hip", C + "mlp_kernel.hpp",
                           C + "mlp_common.hpp", C + "common.hpp"],
            "backward": [C + "mlp_bwd.hip", C + "mlp_common.hpp", C + "common.hpp"],
            "mlp_stream_kernel": [C + "mlp_stream.hip", C + "mlp_common.hpp", C + "common.hpp"],
            "stream_backward": [C + "mlp_bwd_stream.hip", C + "mlp_common.hpp", C + "common.hpp"]}

    def sha(files):
        h = hashlib.sha256()
        for fn in files:
            with open(os.path.join(ROOT, fn), "rb") as f:
                h.update(f.read())
        return h.hexdigest()

    def tot(entries, role, wl, fac):
        vs = [sum(e[4]) for e in entries if e[1] == wl and e[2] == role]
        return fac * KiB * sum(vs) / len(vs)

    out = {"_comment": "HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of "
                       "'bench.py --fusion-traffic', scaled by the calibration factors (FETCH_SIZE x %.4f, "
                       "WRITE_SIZE x %.4f: the 512 MiB read sweep and the 256 MiB read + 256 MiB write activation "
                       "kernel).  Written by 'bench.py --summarize-counters'.  bench.py reports a kernel's traffic "
                       "only while its sources still hash to source_sha256." % (f_fac, w_fac),
           "fetch_factor": f_fac, "write_factor": w_fac, "fusion": {}}
    print("| workload | fused read | fused write | unfused read | unfused write | unfused - fused | model | "
          "measured / model |")
    print("|---|---|---|---|---|---|---|---|")
    for wl in TRAFFIC_GEMMS + TRAFFIC_MLPS:
        w = datagen.WORKLOADS[wl]
        fr, fw = tot(fe, "fused_cold", wl, f_fac), tot(wr, "fused_cold", wl, w_fac)
        ur, uw = tot(fe, "unfused_cold", wl, f_fac), tot(wr, "unfused_cold", wl, w_fac)
        if wl in TRAFFIC_MLPS:
            # each hidden layer's z_l written by its GEMM, read and h_l written
            # by the softplus kernel, h_l read by the next GEMM (fp16)
            s_h = [2.0 * w.M * d for d in w.dims[1:-1]]
            model = 4.0 * sum(s_h)
            model_txt = "4 x sum of S_h (%d hidden layers of %.1f MB)" % (len(s_h), s_h[0] / 1e6)
            kern = "mlp_kernel"
        else:
            # Z written by the GEMM, read by the bias add, Z2 written by it,
            # read by the activation (intermediates in the input dtype,
            # the size of the output here)
            s_out = (4.0 if w.out_dtype == "f32" else 2.0) * w.M * w.N
            model = 4.0 * s_out
            model_txt = "4 x S_out (S_out %.1f MB)" % (s_out / 1e6)
            kern = "gemm32_kernel" if w.in_dtype == "f32" else "gemm16_kernel"
        delta = (ur + uw) - (fr + fw)
        out["fusion"][wl] = {"fused_fetch_bytes": fr, "fused_write_bytes": fw, "unfused_fetch_bytes": ur,
                             "unfused_write_bytes": uw, "delta_bytes": delta, "model_bytes": model,
                             "model": model_txt, "ratio": delta / model,
                             "algorithmic_bytes": w.bytes()}
        print("| %s | %.1f MB | %.1f MB | %.1f MB | %.1f MB | %.1f MB | %.1f MB (%s) | %.3f |"
              % (wl, fr / 1e6, fw / 1e6, ur / 1e6, uw / 1e6, delta / 1e6, model / 1e6, model_txt, delta / model))
        warm_f, warm_w = tot(fe, "fused_warm", wl, f_fac), tot(wr, "fused_warm", wl, w_fac)
        out["%s/%s" % (kern, wl)] = {"kernels": [kern], "sources": srcs[kern], "fetch_bytes": warm_f,
                                     "write_bytes": warm_w, "source_sha256": sha(srcs[kern])}
    print()
    print("| timed kernel (back to back) | FETCH (scaled) | WRITE (scaled) | algorithmic |")
    print("|---|---|---|---|")
    for key, ent in out.items():
        if "/" in key:
            w = datagen.WORKLOADS[key.split("/")[1]]
            print("| %s | %.1f MB | %.1f MB | %.1f MB |" % (key, ent["fetch_bytes"] / 1e6, ent["write_bytes"] / 1e6,
                                                            w.bytes() / 1e6))
    for wl in TRAFFIC_MLPS:
        w = datagen.WORKLOADS[wl]
        hidden = sum(w.dims[1:-1])
        for role, key, kern, by in (("forward_train_warm", "forward_train", "mlp_kernel",
                                     w.M * (2.0 * w.dims[0] + 2.0 * w.dims[-1] + 4.0 * hidden)),
                                    ("backward_warm", "backward", "backward",
                                     w.M * (4.0 * w.dims[0] + 2.0 * w.dims[-1] + 4.0 * hidden))):
            f_, w_ = tot(fe, role, wl, f_fac), tot(wr, role, wl, w_fac)
            out["%s/%s" % (key, wl)] = {"kernels": [kern], "sources": srcs[kern], "fetch_bytes": f_,
                                        "write_bytes": w_, "source_sha256": sha(srcs[kern])}
            print("| %s/%s | %.1f MB | %.1f MB | %.1f MB |" % (key, wl, f_ / 1e6, w_ / 1e6, by / 1e6))
    for wl in TRAFFIC_CHAINS:
        w = datagen.WORKLOADS[wl]
        hidden = sum(w.dims[1:-1])
        for role, key, kern, by in (("stream_forward_warm", "stream_forward", "mlp_stream_kernel", w.bytes()),
                                    ("stream_forward_train_warm", "stream_forward_train", "mlp_stream_kernel",
                                     w.bytes() + 4.0 * w.M * hidden),
                                    ("stream_backward_warm", "stream_backward", "stream_backward",
                                     w.M * (4.0 * w.dims[0] + 2.0 * w.dims[-1] + 4.0 * hidden))):
            f_, w_ = tot(fe, role, wl, f_fac), tot(wr, role, wl, w_fac)
            out["%s/%s" % (key, wl)] = {"kernels": [kern], "sources": srcs[kern], "fetch_bytes": f_,
                                        "write_bytes": w_, "source_sha256": sha(srcs[kern])}
            print("| %s/%s | %.1f MB | %.1f MB | %.1f MB |" % (key, wl, f_ / 1e6, w_ / 1e6, by / 1e6))
    print()
    print("calibration: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (f_fac, w_fac))
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")


def summarize_trace(trace_csv, bench_json):
    """For each kernel a bench.py run timed (its JSON line in bench_json),
    the mean duration of its last K dispatches in the rocprofv3 kernel trace
    of that run -- the timed launches, when the run skipped the sections that
    launch the same kernel later (--no-harness --no-tune --no-variants) --
    beside the mean the run measured with HIP events and the mean over all
    of the kernel's dispatches (what --stats reports)."""
    rows = _read_csv(trace_csv)
    with open(bench_json) as f:
        line = [l for l in f if l.startswith("{")][-1]
    res = json.loads(line)
    by_name = {}
    for r in rows:
        by_name.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    timed = [("primary " + res["config"]["workload"], res["roofline"], res["steps"],
              "mlp_kernel" if res["unit"] == "rows/s" else ("gemm32_kernel" if res["dtype"] == "f32" else "gemm16_kernel"))]
    for wl, ent in (res.get("mlp") or {}).items():
        timed.append((wl, ent["roofline"], max(20, res["steps"]), "mlp_kernel"))
    # the general chains' forward (the last launches of its instantiation in
    # a run without the tuning section)
    for wl, ent in (res.get("variants") or {}).items():
        if isinstance(ent, dict) and "forward_roofline" in ent:
            timed.append((wl + " forward", ent["forward_roofline"], max(20, res["steps"]), ent["forward_kernel"]))
    print("| timed kernel | dispatches | mean of all | mean of the last K (K) | HIP-event mean of the run | "
          "roofline frac from the trace | from the events |")
    print("|---|---|---|---|---|---|---|")
    for label, roof, K, pat in timed:
        want = roof["mean_launch_ms"]
        # the kernel instantiation whose last K dispatches best match the events
        best = None
        for name, ts in by_name.items():
            if pat not in name or "coalesce" not in name or len(ts) < K:
                continue
            ts = sorted(ts)
            last = [(e - s) / 1e6 for s, e in ts[-K:]]
            m = sum(last) / K
            if best is None or abs(m - want) < abs(best[1] - want):
                best = (name, m, sum((e - s) / 1e6 for s, e in ts) / len(ts), len(ts))
        if best is None:
            continue
        name, m, allm, n = best
        if "unit" not in roof:  # a general chain: the fraction of its largest bound scales with 1 / time
            frac = roof["frac"] * want / m
        elif roof["unit"] == "TFLOP/s":
            frac = roof["algorithmic_flop_per_launch"] / (m * 1e-3) / 1e12 / roof["peak"]
        else:
            frac = roof["algorithmic_bytes_per_launch"] / (m * 1e-3) / 1e9 / roof["peak"]
        print("| %s: `%s` | %d | %.4f ms | %.4f ms (%d) | %.4f ms | %.4f | %.4f |"
              % (label, name.replace("void coalesce::(anonymous namespace)::", "").split("(")[0], n, allm, m, K,
                 want, frac, roof["frac"]))


def measured_traffic(key):
    """HBM bytes per launch from the committed counter runs (profiles/traffic.json),
    or None when the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f).get(key)
        if not entry:
            return None
        h = hashlib.sha256()
        for src in entry["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != entry["source_sha256"]:
            return None
        return float(entry["fetch_bytes"]) + float(entry["write_bytes"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(w, target_s):
    """Time the fp64 oracle (as it stands) on a bounded row sample of workload w."""
    import numpy as np

    import datagen
    import oracle

    threads = oracle.max_threads()
    if isinstance(w, datagen.MlpWorkload):
        x, Ws = datagen.mlp_inputs(w)
        x64 = datagen.to_f64(x[: 1 << 16])
        W64 = [datagen.to_f64(t) for t in Ws]
        rows = 4096
        while True:
            t0 = time.perf_counter()
            oracle.mlp_forward(x64[:rows], W64)
            dt = time.perf_counter() - t0
            if dt * 2 >= target_s or rows >= x64.shape[0]:
                break
            rows = min(x64.shape[0], int(rows * max(2.0, target_s / max(dt, 1e-3) * 0.9)))
        return {"value": round(rows / dt, 1), "unit": "rows/s", "cores": threads, "kind": "oracle",
                "sample": "%d of %d rows of %s, fp64 naive loops, %.1f s" % (rows, w.M, w.name, dt)}
    A, B, bias = datagen.gemm_inputs(w)
    A64, B64, b64 = datagen.to_f64(A), datagen.to_f64(B), datagen.to_f64(bias)
    rows = max(1, threads)
    while True:
        t0 = time.perf_counter()
        oracle.gemm_bias_act(A64, B64, b64, act="gelu", rows=np.arange(rows))
        dt = time.perf_counter() - t0
        if dt * 2 >= target_s or rows >= w.M:
            break
        rows = min(w.M, int(rows * max(2.0, target_s / max(dt, 1e-3) * 0.9)))
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d rows of %s (all %d columns), fp64 naive triple loop, %.1f s"
                      % (rows, w.M, w.name, w.N, dt)}


if __name__ == "__main__":
    main()
