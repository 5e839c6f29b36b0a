#!/usr/bin/env python3
"""Throughput of the Averis hot path on one MI355X.

Headline step: one training step of the seven linears of a Qwen3-0.6B-shaped transformer
layer at l = 16384 tokens (q 1024->2048, k and v 1024->1024, o 2048->1024, gate and up
1024->3072, down 3072->1024; bf16 inputs): split + FP4-quantize every distinct input (q, k
and v share theirs, gate and up share theirs) and every output gradient, quantize every
weight, and run each linear's forward (bf16 Y), input-gradient (bf16 dX) and weight-gradient
(fp32 dW) GEMM with the mean terms, in a training step's order: the weights (one batched
launch), the forward input by input (its split, then the forward GEMMs reading it), the
backward in reverse (the batched split of the output gradients of the linears sharing an
input, then their dX and dW); the weights and the dW GEMMs on a second stream that forks from the
timed stream and joins it before the step ends.  Linears that share an input share GEMMs:
q/k/v and gate/up one forward GEMM each (the Y_i are its column blocks), q/k/v one
weight-gradient GEMM (the dW_i are its column blocks); each linear keeps its own dX.  Format MXFP4 (gfx950's native scaled-MFMA format); NVFP4-style
blocks and the vanilla (no split) step are timed beside it.
value = GEMM flops of the step / the step's median cold time.

Timing: each measured call sequence is captured once in a HIP graph.  Cold replays follow a
512 MiB read that evicts the L2s and the 256 MB Infinity Cache (inputs start in HBM); warm
replays run back to back.  HIP events on the launching stream bracket every replay; median and
minimum are reported.  The roofline kernel's launch duration is the mean per launch of a graph
of ten back-to-back launches replayed between events (a replay of a one-launch graph holds
about 10 us of launch latency inside the events, a fifth of this kernel's time).

Other stages (parity configurations and the pages' comparisons): the same layer with
independent inputs per linear, a GEMM output split next (the gate forward GEMM, then the split
of Y, with the statistics pass over Y or with the GEMM taking the column statistics in its
epilogue), the MLP block's forward (RMSNorm, split, gate and up GEMMs, SwiGLU, split, down GEMM)
with and without RMSNorm and SwiGLU writing the splits' column statistics, the up_proj layer
(l = 8192), the down_proj layer in its four
variants ({NVFP4, MXFP4} x {Hadamard off, on}, each also vanilla), the MoE layer, and Averis vs
16x16-Hadamard preprocessing at the explainer's activation shapes (512 x 2048 tokens, 4096 and
8192 channels).

Prints one JSON line.  --gpus N > 1 is refused: everything here runs on one GPU.
"""
import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "split+FP4-quant HBM GB/s; FP4 GEMM fwd+bwd TFLOP/s; Averis overhead % vs vanilla"
PEAK_HBM_GBPS = 8000.0
PEAK_FP4_TFLOPS = 10100.0
PEAK_BF16_TFLOPS = 2500.0
L_LAYER = 16384


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50, help="timed replays per measurement (cold and warm each)")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--one-stream", action="store_true",
                   help="run the layer and MoE steps on one stream (per-launch attribution in a trace)")
    p.add_argument("--stages", default="all",
                   help="comma list of stages to run: layer,independent,chain,mlp,up_proj,down_proj,moe,prep,roofline")
    return p.parse_args()


def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


def gpu_clocks():
    """Current GPU clocks as reported by amd-smi (or rocm-smi), or None."""
    for cmd in (["amd-smi", "metric", "--clock", "--json"], ["rocm-smi", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.TimeoutExpired):
            continue
        if r.returncode != 0 or not r.stdout.strip():
            continue
        try:
            data = json.loads(r.stdout)
        except ValueError:
            return {"tool": cmd[0], "text": r.stdout.strip()[:400]}
        return {"tool": cmd[0], "clocks": _clock_summary(data)}
    return None


def _clock_summary(data):
    """The graphics and memory clocks (current, MHz) from an amd-smi / rocm-smi JSON dump."""
    out = {}

    def walk(o, path):
        if isinstance(o, dict):
            for k, v in o.items():
                walk(v, path + [str(k)])
        elif isinstance(o, list):
            for i, v in enumerate(o):
                walk(v, path + [str(i)])
        else:
            key = "/".join(path).lower()
            if any(t in key for t in ("gfx", "sclk", "mclk", "mem")) and any(
                    t in key for t in ("clk", "clock", "freq")) and len(out) < 16:
                out["/".join(path[-3:])] = o
    walk(data, [])
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is "
              "described in the design notes, not run.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_quantized_amd.averis as av
    from fp4_quantized_amd import workloads
    from fp4_quantized_amd.step import LayerStep, LinearStep, MoEStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    av.lib()
    stages = set(args.stages.split(",")) if args.stages != "all" else \
        {"layer", "independent", "chain", "mlp", "up_proj", "down_proj", "moe", "prep", "roofline"}
    dev = torch.device("cuda:0")
    # Cache eviction before cold replays: read (not write) 512 MiB, so the L2s and the 256 MB
    # Infinity Cache end up holding clean lines of another buffer.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    steps, warmup = args.steps, args.warmup

    def timed(fn, n=None, w=None):
        """Median / min of cold and warm replays of fn captured in a graph (ms)."""
        n = n or steps
        w = warmup if w is None else w
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(w):
            g.replay()
        torch.cuda.synchronize()
        cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in cold:
            flush.sum()
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        warm = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in warm:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        c = [a.elapsed_time(b) for a, b in cold]
        wm = [a.elapsed_time(b) for a, b in warm]
        del g
        return {"cold_med": float(np.median(c)), "cold_min": float(np.min(c)),
                "warm_med": float(np.median(wm)), "warm_min": float(np.min(wm))}

    def timed_launch(fn, n=None, reps=10):
        """One kernel's launch duration (ms): a graph of `reps` back-to-back launches replayed n
        times between events on the launching stream, per launch (mean and median over the
        replays); and, for reference, single eager launches after the cache-evicting read (cold),
        whose events also hold a few microseconds of event and launch latency."""
        n = n or steps
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        back = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in back:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        cold = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            flush.sum()
            a.record()
            fn()
            b.record()
            cold.append((a, b))
        torch.cuda.synchronize()
        bk = [a.elapsed_time(b) / reps for a, b in back]
        c = [a.elapsed_time(b) for a, b in cold]
        del g
        return {"mean": float(np.mean(bk)), "med": float(np.median(bk)), "min": float(np.min(bk)),
                "cold_eager_med": float(np.median(c)), "cold_eager_min": float(np.min(c))}

    def r4(d):
        return {k: round(v, 5) for k, v in d.items()}

    env = {"clocks_before": gpu_clocks(), "host_cores_affinity": len(os.sched_getaffinity(0)),
           "device": torch.cuda.get_device_name(0)}
    # measured copy bandwidth: a second denominator for the memory-bound kernels
    src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    env["copy_GBps"] = round(2 * src.numel() * 4 / (t_copy["cold_med"] * 1e-3) / 1e9, 1)
    del src, dst
    log(f"copy {env['copy_GBps']} GB/s")

    line_extra = {}
    out = {}

    # ---------------- headline: the layer step (shared inputs) ----------------
    headline = None
    if "roofline" in stages and "layer" not in stages:
        # the roofline launch alone: its operands, without timing the step
        headline = LayerStep(workloads.layer_device(3, L_LAYER, dev, shared=True), av.MXFP4, split=True)
        headline.quantize()
        torch.cuda.synchronize()
    if "layer" in stages:
        t0 = time.time()
        layers = workloads.layer_device(3, L_LAYER, dev, shared=True)
        log(f"layer inputs ready in {time.time() - t0:.1f}s")
        res = {}
        for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
            r = {}
            for split in (True, False):
                st = LayerStep(layers, fmt, split=split, overlap=not args.one_stream)
                tag = "averis" if split else "vanilla"
                r[tag] = r4(timed(st.run))
                if fmt == av.MXFP4 or split:
                    r[f"{tag}_quant"] = r4(timed(st.quantize))
                    r[f"{tag}_gemm"] = r4(timed(st.gemms))
                flops = st.flops
                if split:
                    qbytes = st.quant_bytes()
                if fmt == av.MXFP4 and split:
                    res["split_quant_bytes_mxfp4"] = int(qbytes)
                if fmt == av.MXFP4 and split and "roofline" in stages:
                    headline = st  # kept for the roofline launch below
                else:
                    del st
                log(f"layer {name} {tag}: step {r[tag]['cold_med']*1e3:.1f} us cold, {r[tag]['warm_med']*1e3:.1f} warm")
            r["step_tflops"] = round(flops / (r["averis"]["cold_med"] * 1e-3) / 1e12, 1)
            r["overhead_pct"] = round(100.0 * (r["averis"]["cold_med"] - r["vanilla"]["cold_med"])
                                      / r["vanilla"]["cold_med"], 2)
            r["overhead_pct_warm"] = round(100.0 * (r["averis"]["warm_med"] - r["vanilla"]["warm_med"])
                                           / r["vanilla"]["warm_med"], 2)
            r["split_quant_GBps"] = round(qbytes / (r["averis_quant"]["cold_med"] * 1e-3) / 1e9, 1)
            r["gemm_tflops"] = round(flops / (r["averis_gemm"]["cold_med"] * 1e-3) / 1e12, 1)
            res[name] = r
        res["gflop"] = round(flops / 1e9, 1)
        del layers
        # q/k/v and gate/up stored as fused projections (their output gradients and weights
        # column blocks of one tensor each): one split of each group's D and W and one dX GEMM
        # per group, the sum of its linears' dX_i (the same flops)
        layers = workloads.layer_device(3, L_LAYER, dev, shared=True, cat=True)
        r = {}
        for split in (True, False):
            st = LayerStep(layers, av.MXFP4, split=split, overlap=not args.one_stream)
            r["averis" if split else "vanilla"] = r4(timed(st.run))
            del st
        r["overhead_pct"] = round(100.0 * (r["averis"]["cold_med"] - r["vanilla"]["cold_med"])
                                  / r["vanilla"]["cold_med"], 2)
        r["step_tflops"] = round(flops / (r["averis"]["cold_med"] * 1e-3) / 1e12, 1)
        res["mxfp4_fused_projections"] = r
        log(f"layer mxfp4 fused projections: averis {r['averis']['cold_med']*1e3:.1f} us, "
            f"vanilla {r['vanilla']['cold_med']*1e3:.1f} us")
        out["layer"] = res
        del layers

    # ---------------- roofline: the step's longest kernel ----------------
    roofline = None
    if headline is not None:
        # the fused gate/up forward GEMM (X_R [W_gate W_up]^T + the mean row, one launch for both)
        pi = next(i for i, (_, _, lins) in enumerate(headline.x_plan)
                  if [headline.lin[j]["name"] for j in lins] == ["gate", "up"])
        f = headline.fwd_fused[pi]
        c = headline.lin[headline.x_plan[pi][2][0]]
        l, m, n = c["l"], c["m"], f["w"].outer
        t = timed_launch(lambda: av.linear_fwd(f["sx"]["row"], f["sx"]["mean_q"], f["w"], out=f["y"], ws=f["ws"]))
        launch_s = t["mean"] * 1e-3
        op = 0.5 + 1.0 / 32
        flops = 2.0 * l * m * n
        nbytes = (l * m + n * m + m) * op + 2.0 * l * n
        t_mfma, t_hbm = flops / (PEAK_FP4_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9)
        hbm_bound = t_hbm > t_mfma
        roofline = {
            "bound": "hbm" if hbm_bound else "mfma",
            "kernel": f"k_gemm_ws<MXFP4, mean term> forward GEMM of gate and up together, {l} x {n} x {m}, bf16 Y "
                      "(the step's longest launch when its launches run one at a time)",
            "achieved": round(nbytes / launch_s / 1e9, 1) if hbm_bound else round(flops / launch_s / 1e12, 1),
            "peak": PEAK_HBM_GBPS if hbm_bound else PEAK_FP4_TFLOPS,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round((t_hbm if hbm_bound else t_mfma) / launch_s, 4),
            "traffic": gemm_traffic(),
            "algorithmic_bytes": int(nbytes), "flops": flops,
            "launch_us": {k: round(v * 1e3, 2) for k, v in t.items()},
            "mfma_frac": round(t_mfma / launch_s, 4), "hbm_frac": round(t_hbm / launch_s, 4),
            "frac_vs_measured_copy": round(nbytes / launch_s / 1e9 / env["copy_GBps"], 4),
        }
        log(f"roofline launch {t['mean']*1e3:.1f} us: {flops / launch_s / 1e12:.0f} TFLOP/s, "
            f"{nbytes / launch_s / 1e9:.0f} GB/s")
        del headline

    # ---------------- producer-fused column statistics: a GEMM output split next ----------------
    if "chain" in stages:
        # the gate projection's forward GEMM (16384 x 1024 -> 3072, bf16 Y) followed by the split
        # of Y, as when a GEMM output is the next linear's input: the split's statistics pass over
        # Y against the GEMM taking them in its epilogue (and the split starting from them)
        _, x, _, w = next(c for c in workloads.layer_device(3, L_LAYER, dev, shared=True) if c[0] == "gate")
        l, n = x.shape[0], w.shape[1]
        res = {}
        for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
            sx, sw = av.split_quant(x, fmt), av.split_quant(w, fmt, split=False)
            y = torch.empty(l, n, dtype=torch.bfloat16, device=dev)
            wsl = av.linear_workspace(sx["row"], sw["col"])
            cs = av.ColStats(l, n, minmax=fmt == av.NVFP4)
            o_a = av.split_quant_outputs(l, n, fmt, True, device=dev)
            o_v = av.split_quant_outputs(l, n, fmt, False, device=dev)
            wsq = av.split_quant_workspace(l, n, fmt, True, device=dev)

            def gemm():
                av.linear_fwd(sx["row"], sx["mean_q"], sw["col"], out=y, ws=wsl)

            def gemm_stats():
                av.linear_fwd_stats(sx["row"], sx["mean_q"], sw["col"], cs, out=y, ws=wsl)

            r = {
                "gemm": r4(timed(gemm)),
                "gemm_stats": r4(timed(gemm_stats)),
                "vanilla": r4(timed(lambda: (gemm(), av.split_quant(y, fmt, split=False, out=o_v, ws=wsq)))),
                "averis": r4(timed(lambda: (gemm(), av.split_quant(y, fmt, out=o_a, ws=wsq)))),
                "averis_stats": r4(timed(lambda: (gemm_stats(), av.split_quant_stats(y, cs, fmt, out=o_a, ws=wsq)))),
            }
            v = r["vanilla"]["cold_med"]
            r["averis_overhead_pct"] = round(100.0 * (r["averis"]["cold_med"] - v) / v, 2)
            r["averis_stats_overhead_pct"] = round(100.0 * (r["averis_stats"]["cold_med"] - v) / v, 2)
            r["epilogue_stats_us"] = round((r["gemm_stats"]["cold_med"] - r["gemm"]["cold_med"]) * 1e3, 2)
            r["part_rows"] = int(cs.part_rows)
            res[name] = r
            log(f"chain {name}: averis +{r['averis_overhead_pct']} %, with producer statistics "
                f"+{r['averis_stats_overhead_pct']} % over vanilla")
            del sx, sw, y, wsl, cs, o_a, o_v, wsq
        out["chain_gemm_then_split"] = res
        del x, w

    # ---------------- the MLP block's forward with its producers ----------------
    if "mlp" in stages:
        # RMSNorm of the residual stream [16384, 1024] -> split -> gate and up forward GEMMs
        # (1024 -> 3072) -> SwiGLU -> split -> down forward GEMM (3072 -> 1024); weights quantized
        # beforehand (once per optimizer step).  Vanilla FP4, Averis with the splits' own
        # statistics passes, and Averis with RMSNorm and SwiGLU writing the column statistics
        # that the splits start from.
        lay = workloads.layer_device(3, L_LAYER, dev, shared=True)
        h = next(c for c in lay if c[0] == "gate")[1]
        wg, wu, wd = (next(c for c in lay if c[0] == nm)[3] for nm in ("gate", "up", "down"))
        del lay
        hid, ffn = wg.shape
        gam = torch.ones(hid, dtype=torch.float32, device=dev)
        xn = torch.empty(L_LAYER, hid, dtype=torch.bfloat16, device=dev)
        yg, yu, xd = (torch.empty(L_LAYER, ffn, dtype=torch.bfloat16, device=dev) for _ in range(3))
        yd = torch.empty(L_LAYER, hid, dtype=torch.bfloat16, device=dev)
        res = {}
        for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
            sg, su, sd_ = (av.split_quant(w, fmt, split=False)["col"] for w in (wg, wu, wd))
            mm = fmt == av.NVFP4
            cs_n, cs_d = av.ColStats(L_LAYER, hid, minmax=mm), av.ColStats(L_LAYER, ffn, minmax=mm)
            o = {sp: (av.split_quant_outputs(L_LAYER, hid, fmt, sp, device=dev),
                      av.split_quant_outputs(L_LAYER, ffn, fmt, sp, device=dev)) for sp in (True, False)}
            wsn, wsd = av.split_quant_workspace(L_LAYER, hid, fmt, device=dev), \
                av.split_quant_workspace(L_LAYER, ffn, fmt, device=dev)
            wg_ws = av.linear_workspace(o[True][0]["row"], sg)
            wd_ws = av.linear_workspace(o[True][1]["row"], sd_)

            def block(mode):
                split = mode != "vanilla"
                on, od = o[split]
                prod = mode == "averis_producer"
                av.rmsnorm(h, gam, 1e-6, stats=cs_n if prod else None, out=xn)
                if prod:
                    av.split_quant_stats(xn, cs_n, fmt, out=on, ws=wsn)
                else:
                    av.split_quant(xn, fmt, split, out=on, ws=wsn)
                mu = on["mean_q"] if split else None
                av.linear_fwd(on["row"], mu, sg, out=yg, ws=wg_ws)
                av.linear_fwd(on["row"], mu, su, out=yu, ws=wg_ws)
                av.swiglu(yg, yu, stats=cs_d if prod else None, out=xd)
                if prod:
                    av.split_quant_stats(xd, cs_d, fmt, out=od, ws=wsd)
                else:
                    av.split_quant(xd, fmt, split, out=od, ws=wsd)
                av.linear_fwd(od["row"], od["mean_q"] if split else None, sd_, out=yd, ws=wd_ws)

            r = {m: r4(timed(lambda m=m: block(m))) for m in ("vanilla", "averis", "averis_producer")}
            v = r["vanilla"]["cold_med"]
            r["averis_overhead_pct"] = round(100.0 * (r["averis"]["cold_med"] - v) / v, 2)
            r["averis_producer_overhead_pct"] = round(100.0 * (r["averis_producer"]["cold_med"] - v) / v, 2)
            res[name] = r
            log(f"mlp forward {name}: averis +{r['averis_overhead_pct']} %, with producer statistics "
                f"+{r['averis_producer_overhead_pct']} % over vanilla ({v*1e3:.1f} us)")
            del sg, su, sd_, cs_n, cs_d, o, wsn, wsd, wg_ws, wd_ws
        out["mlp_forward_with_producers"] = res
        del h, wg, wu, wd, xn, yg, yu, xd, yd

    # ---------------- the layer with independent inputs per linear ----------------
    if "independent" in stages:
        layers = workloads.layer_device(3, L_LAYER, dev, shared=False)
        res = {}
        for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
            r = {}
            for split in (True, False):
                st = LayerStep(layers, fmt, split=split, overlap=not args.one_stream)
                r["averis" if split else "vanilla"] = r4(timed(st.run, max(5, steps // 2)))
                flops = st.flops
                del st
            r["overhead_pct"] = round(100.0 * (r["averis"]["cold_med"] - r["vanilla"]["cold_med"])
                                      / r["vanilla"]["cold_med"], 2)
            r["step_tflops"] = round(flops / (r["averis"]["cold_med"] * 1e-3) / 1e12, 1)
            res[name] = r
            log(f"layer (independent inputs) {name}: overhead {r['overhead_pct']} %")
        out["layer_independent_inputs"] = res
        del layers

    # ---------------- up_proj (l = 8192) ----------------
    if "up_proj" in stages:
        lin = workloads.up_proj()
        x, d, w = (workloads.to_torch(a, "bf16", dev) for a in (lin.x, lin.d, lin.w))
        l, m = lin.x.shape
        n = lin.d.shape[1]
        res = {}
        for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
            r = {}
            for split in (True, False):
                st = LinearStep(x, d, w, fmt, split=split)
                tag = "averis" if split else "vanilla"
                r[tag] = r4(timed(st.run))
                r[f"{tag}_quant"] = r4(timed(st.quantize))
                r[f"{tag}_gemm"] = r4(timed(st.gemms))
                del st
            g = av.BLOCK[fmt]
            qb = (l * m + l * n + m * n) * (2 + 2 * (0.5 + 1.0 / g)) + (m + n) * (4 + 0.5 + 1.0 / g)
            r["step_tflops"] = round(6.0 * l * m * n / (r["averis"]["cold_med"] * 1e-3) / 1e12, 1)
            r["split_quant_GBps"] = round(qb / (r["averis_quant"]["cold_med"] * 1e-3) / 1e9, 1)
            r["gemm_tflops"] = round(6.0 * l * m * n / (r["averis_gemm"]["cold_med"] * 1e-3) / 1e12, 1)
            r["overhead_pct"] = round(100.0 * (r["averis"]["cold_med"] - r["vanilla"]["cold_med"])
                                      / r["vanilla"]["cold_med"], 2)
            res[name] = r
            log(f"up_proj {name}: step {r['averis']['cold_med']*1e3:.1f} us, split+quant {r['split_quant_GBps']} GB/s")
        out["up_proj"] = res
        del x, d, w, lin

    # ---------------- down_proj (l = 16384) in its four variants ----------------
    if "down_proj" in stages:
        x, d, w = workloads.down_proj_device(2, L_LAYER, 3072, 1024, dev)
        res = {}
        for fmt, name in ((av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")):
            r = {}
            for split, h16, tag in ((False, False, "vanilla"), (True, False, "averis"), (False, True, "hadamard"),
                                    (True, True, "averis_hadamard")):
                st = LinearStep(x, d, w, fmt, split=split, hadamard=h16)
                r[tag] = r4(timed(st.run, max(5, steps // 2)))
                del st
            v = r["vanilla"]["cold_med"]
            for tag in ("averis", "hadamard", "averis_hadamard"):
                r[f"{tag}_overhead_pct"] = round(100.0 * (r[tag]["cold_med"] - v) / v, 2)
            r["step_tflops"] = round(6.0 * L_LAYER * 3072 * 1024 / (r["averis"]["cold_med"] * 1e-3) / 1e12, 1)
            res[name] = r
            log(f"down_proj {name}: averis +{r['averis_overhead_pct']} %, hadamard +{r['hadamard_overhead_pct']} %")
        out["down_proj"] = res
        del x, d, w

    # ---------------- MoE layer ----------------
    if "moe" in stages:
        moe_in = workloads.moe_device(4, device=dev)
        res = {}
        for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
            r = {}
            # gate and up as one projection (hidden -> 2 ffn, the gated MLP's layout), and as two
            for fused, sfx in ((True, ""), (False, "_separate")):
                for split in (True, False):
                    ms = MoEStep(*moe_in[:8], moe_in[8], fmt, split=split, overlap=not args.one_stream,
                                 fuse_gate_up=fused)
                    r[("averis" if split else "vanilla") + sfx] = r4(timed(ms.run, max(5, steps // 2)))
                    flops = ms.flops
                    del ms
                r["overhead_pct" + sfx] = round(100.0 * (r["averis" + sfx]["cold_med"] - r["vanilla" + sfx]["cold_med"])
                                                / r["vanilla" + sfx]["cold_med"], 2)
                r["step_tflops" + sfx] = round(flops / (r["averis" + sfx]["cold_med"] * 1e-3) / 1e12, 1)
                log(f"moe {name}{sfx}: averis {r['averis' + sfx]['cold_med']*1e3:.0f} us, "
                    f"vanilla {r['vanilla' + sfx]['cold_med']*1e3:.0f} us")
            res[name] = r
        res["routed_rows"] = int(moe_in[8][-1])
        res["gflop"] = round(flops / 1e9, 1)
        out["moe"] = res
        del moe_in

    # ---------------- Averis vs 16x16 Hadamard preprocessing, the pages' shapes ----------------
    if "prep" in stages:
        res = {}
        lp = 512 * 2048
        for m_ in (4096, 8192):
            xa = workloads.activations_device_chunked(7, lp, m_, dev)
            for fmt, name in ((av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")):
                r = {}
                for tag, split, h16 in (("vanilla", False, False), ("averis", True, False), ("hadamard", False, True)):
                    o = av.split_quant_outputs(lp, m_, fmt, split, h16, row=True, col=False, device=dev)
                    ws = av.split_quant_workspace(lp, m_, fmt, split, h16, dev)
                    r[tag] = r4(timed(lambda: av.split_quant(xa, fmt, split, h16, row=True, col=False, out=o, ws=ws),
                                      max(5, steps // 4), 2))
                    del o, ws
                van = r["vanilla"]["cold_med"]
                r["averis_prep_ms"] = round(r["averis"]["cold_med"] - van, 4)
                r["hadamard_prep_ms"] = round(r["hadamard"]["cold_med"] - van, 4)
                r["hadamard_over_averis"] = round(r["hadamard_prep_ms"] / max(r["averis_prep_ms"], 1e-9), 2)
                res[f"{name}_m{m_}"] = r
                log(f"prep {name} l={lp} m={m_}: vanilla {van:.3f} ms, averis {r['averis']['cold_med']:.3f} ms, "
                    f"hadamard {r['hadamard']['cold_med']:.3f} ms")
            del xa
        res["pages_blackwell_ms"] = {"averis_m4096": 2.0494, "averis_m8192": 3.9927, "hadamard_m4096": 9.1614,
                                     "hadamard_m8192": 18.8421}
        out["preprocessing"] = res

    env["clocks_after"] = gpu_clocks()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()

    lay = out.get("layer", {})
    mx = lay.get("mxfp4", {})
    line = {
        "metric": METRIC,
        "value": mx.get("step_tflops"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(mx["averis"]["cold_med"], 5) if mx else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "Qwen3-0.6B-shaped transformer layer, 7 linears (q 1024->2048, k/v 1024->1024, "
                               "o 2048->1024, gate/up 1024->3072, down 3072->1024) at l=16384 tokens, fwd+dX+dW "
                               "each, bf16 in, bf16 Y/dX, fp32 dW, MXFP4 with the Averis split; q/k/v and gate/up "
                               "share their split input and their forward GEMM, q/k/v also their "
                               "weight-gradient GEMM",
                   "l": L_LAYER, "format": "mxfp4", "timing": "median of cold (cache-evicted) graph replays",
                   "streams": 1 if args.one_stream else 2},
        "split_quant": {"GBps": mx.get("split_quant_GBps"),
                        "frac_hbm": round(mx["split_quant_GBps"] / PEAK_HBM_GBPS, 4) if mx else None,
                        "frac_measured_copy": round(mx["split_quant_GBps"] / env["copy_GBps"], 4) if mx else None},
        "gemm": {"TFLOPs": mx.get("gemm_tflops"),
                 "frac_fp4_peak": round(mx["gemm_tflops"] / PEAK_FP4_TFLOPS, 4) if mx else None},
        "overhead_pct_vs_vanilla": mx.get("overhead_pct"),
        "overhead_pct_vs_vanilla_nvfp4": lay.get("nvfp4", {}).get("overhead_pct"),
        "pages_overhead_pct_context": {"qwen3_0.6b": 2.01, "qwen3_7b_a1.5b": 2.20,
                                       "note": "end-to-end training step on Blackwell, NVFP4; not this op-level "
                                               "measurement"},
        **out,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "env": env,
        **line_extra,
    }
    print(json.dumps(line), flush=True)


def gemm_traffic():
    """HBM bytes per launch of the roofline kernel from the committed counter summary, or None
    once the GEMM source has changed since those counters were taken."""
    import re
    prof = os.path.join(ROOT, "profiles", "k_gemm_ws_mxfp4_mean_16384x6144x1024_traffic.txt")
    try:
        text = open(prof).read()
    except OSError:
        return None
    m_t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    m_h = re.search(r"^gemm_source_sha1: ([0-9a-f]+)$", text, re.M)
    if not (m_t and m_h):
        return None
    from fp4_quantized_amd.build import gemm_source_digest
    return int(m_t.group(1)) if gemm_source_digest()[:len(m_h.group(1))] == m_h.group(1) else None


def cpu_baseline():
    """The CPU oracle on a bounded sample of the headline layer: the gate linear (1024 -> 3072)
    at all 16384 tokens, MXFP4 with the split (split+quant of X, D and W, then the three GEMMs),
    one of the layer's seven linears.  Throughput = that linear's GEMM flops / its time."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from fp4_quantized_amd import workloads
    from oracle import averis_oracle as O
    lin = workloads.up_proj_like([3, 4], L_LAYER, 1024, 3072, name="gate")
    l, m = lin.x.shape
    n = lin.d.shape[1]
    t0 = time.perf_counter()
    sw = O.split_quant(lin.w, O.MXFP4, split=False)
    sx = O.split_quant(lin.x, O.MXFP4)
    sd = O.split_quant(lin.d, O.MXFP4)
    O.linear_fwd(sx["row"], sx["mean"], sw["col"])
    O.linear_bwd_dx(sd["row"], sd["mean"], sw["row"])
    O.linear_bwd_dw(sx["col"], sd["col"], sx["mean"], sd["mean"], l)
    t = time.perf_counter() - t0
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(6.0 * l * m * n / t / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas),
            "kind": "oracle", "host_cores_affinity": len(os.sched_getaffinity(0)),
            "sample": f"the gate linear (1024 -> 3072) of the layer at all {l} tokens, MXFP4 split+quant of "
                      f"X, D, W and fwd/dX/dW, one of the layer's seven linears: {t:.1f} s; numpy, fp64 GEMMs "
                      f"on {blas} BLAS threads"}


if __name__ == "__main__":
    main()
