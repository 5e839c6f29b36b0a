#!/usr/bin/env python3
"""Throughput of the Averis hot path on one MI355X.

A step is one pass of the whole path for the Qwen3-0.6B-shaped up_proj linear layer
(l = 8192 tokens = 4 x 2048, m = 1024 -> n = 3072, bf16 inputs): split + FP4-quantize X and D
(both layouts and the mean), quantize W, then the forward GEMM (bf16 Y), the input-gradient
GEMM (bf16 dX) and the weight-gradient GEMM (fp32 dW) with the mean terms.  The headline
format is MXFP4 (gfx950's native scaled-MFMA format); NVFP4-style blocks are reported beside it.

Timing: the step is captured once in a HIP graph; each timed replay is bracketed by HIP events
on the launching stream, after a 512 MiB read that evicts the 256 MB Infinity Cache and the
L2, so inputs start in HBM.  value = GEMM flops of the step / step time.

Prints one JSON line.  --gpus N > 1 is refused: everything here runs on one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "split+FP4-quant HBM GB/s; FP4 GEMM fwd+bwd TFLOP/s; Averis overhead % vs vanilla"
PEAK_HBM_GBPS = 8000.0
PEAK_FP4_TFLOPS = 10100.0
PEAK_BF16_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=8192, help="token rows of the oracle's timed sample")
    return p.parse_args()


def quant_bytes(l, m, n, g, in_bytes=2):
    """Algorithmic bytes of split+quant for X [l, m], D [l, n] and W [m, n]: each input read
    once, two packed layouts written (codes 1/2 B + scales 1/g B per element), mean vectors."""
    per = 2 * (0.5 + 1.0 / g)
    elems = l * m + l * n + m * n
    means = (m + n) * (4 + 0.5 + 1.0 / g)
    return elems * (in_bytes + per) + means


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
    from fp4_quantized_amd.step import LinearStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    av.lib()
    dev = torch.device("cuda:0")
    t0 = time.time()
    lin = workloads.up_proj()
    l, m = lin.x.shape
    n = lin.d.shape[1]
    x = workloads.to_torch(lin.x, "bf16", dev)
    d = workloads.to_torch(lin.d, "bf16", dev)
    w = workloads.to_torch(lin.w, "bf16", dev)
    # Cache eviction between timed replays: read (not write) 512 MiB, so the L2 and the 256 MB
    # Infinity Cache end up holding clean lines of another buffer and the step pays no
    # write-back of someone else's dirty data.
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def timed(fn, steps, warmup):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            flush.sum()
            evs[i][0].record()
            g.replay()
            evs[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))  # ms

    results = {}
    for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
        g = av.BLOCK[fmt]
        r = {}
        for split in (True, False):
            st = LinearStep(x, d, w, fmt, split=split)
            tag = "averis" if split else "vanilla"
            r[f"{tag}_step_ms"] = timed(st.run, args.steps, args.warmup)
            r[f"{tag}_quant_ms"] = timed(st.quantize, args.steps, args.warmup)
            r[f"{tag}_gemm_ms"] = timed(st.gemms, args.steps, args.warmup)
            print(f"# {name} {tag}: step {r[f'{tag}_step_ms']*1e3:.1f} us, quant {r[f'{tag}_quant_ms']*1e3:.1f} us, "
                  f"gemm {r[f'{tag}_gemm_ms']*1e3:.1f} us", file=sys.stderr, flush=True)
            del st
        flops = 6.0 * l * m * n
        qb = quant_bytes(l, m, n, g)
        r["step_tflops"] = flops / (r["averis_step_ms"] * 1e-3) / 1e12
        r["quant_GBps"] = qb / (r["averis_quant_ms"] * 1e-3) / 1e9
        r["gemm_tflops"] = flops / (r["averis_gemm_ms"] * 1e-3) / 1e12
        r["overhead_pct"] = 100.0 * (r["averis_step_ms"] - r["vanilla_step_ms"]) / r["vanilla_step_ms"]
        results[name] = r

    # Layer sweep (the overhead target's workload): the seven Qwen3-0.6B-shaped linears at
    # l = 16384, one step = all seven linears' quantize + fwd/dX/dW, Averis vs vanilla.
    sweep = {}
    layers = workloads.sweep_device(3, 16384, dev)
    sweep_flops = sum(6.0 * x_.shape[0] * x_.shape[1] * d_.shape[1] for _, x_, d_, _ in layers)
    for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
        r = {}
        for split in (True, False):
            sts = [LinearStep(x_, d_, w_, fmt, split=split) for _, x_, d_, w_ in layers]

            def run_all():
                for s_ in sts:
                    s_.run()
            tag = "averis" if split else "vanilla"
            r[f"{tag}_step_ms"] = round(timed(run_all, max(3, args.steps // 4), max(1, args.warmup // 2)), 4)
            del sts
        r["overhead_pct"] = round(100.0 * (r["averis_step_ms"] - r["vanilla_step_ms"]) / r["vanilla_step_ms"], 2)
        r["step_tflops"] = round(sweep_flops / (r["averis_step_ms"] * 1e-3) / 1e12, 1)
        print(f"# sweep {name}: averis {r['averis_step_ms']*1e3:.0f} us, vanilla {r['vanilla_step_ms']*1e3:.0f} us, "
              f"overhead {r['overhead_pct']:.1f} %", file=sys.stderr, flush=True)
        sweep[name] = r
    del layers

    # MoE grouped layer (every kernel one grouped launch over the experts): 8192 tokens routed
    # top-8 over 64 experts with Zipf(1.1) skew (65,536 routed rows), hidden 2048, expert FFN 768;
    # one step = the gate, up and down linears' split+quant, fwd, dX and dW.
    from fp4_quantized_amd.step import MoEStep
    moe_in = workloads.moe_device(4, device=dev)
    moe = {}
    for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
        r = {}
        for split in (True, False):
            ms = MoEStep(*moe_in[:7], moe_in[7], fmt, split=split)
            tag = "averis" if split else "vanilla"
            r[f"{tag}_step_ms"] = round(timed(ms.run, max(3, args.steps // 4), max(1, args.warmup // 2)), 4)
            flops = ms.flops
            del ms
        r["overhead_pct"] = round(100.0 * (r["averis_step_ms"] - r["vanilla_step_ms"]) / r["vanilla_step_ms"], 2)
        r["step_tflops"] = round(flops / (r["averis_step_ms"] * 1e-3) / 1e12, 1)
        print(f"# moe {name}: averis {r['averis_step_ms']*1e3:.0f} us, vanilla {r['vanilla_step_ms']*1e3:.0f} us, "
              f"{r['step_tflops']} TFLOP/s", file=sys.stderr, flush=True)
        moe[name] = r
    moe_rows = int(moe_in[7][-1])
    del moe_in

    # Averis vs 16x16-Hadamard preprocessing at the operator level (the explainer's comparison of
    # the two activation transforms): X [l, m] bf16 quantized for the forward GEMM (row layout),
    # vanilla, with the mean-residual split, and with the Hadamard instead; the preprocessing cost
    # of each is its time minus vanilla's.  l = 65536 tokens (the pages' 512 x 2048 scaled down by
    # 16: every operand stays below 2^31 bytes), m = 4096 and 8192.
    prep = {}
    for m_ in (4096, 8192):
        xa = workloads.activations_device(7, 65536, m_, dev)
        for fmt, name in ((av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")):
            r = {}
            for tag, split, h16 in (("vanilla", False, False), ("averis", True, False), ("hadamard", False, True)):
                out = av.split_quant_outputs(65536, m_, fmt, split, h16, row=True, col=False, device=dev)
                ws = av.split_quant_workspace(65536, m_, fmt, split, h16, dev)
                r[f"{tag}_ms"] = round(timed(lambda: av.split_quant(xa, fmt, split, h16, row=True, col=False,
                                                                     out=out, ws=ws), args.steps, args.warmup), 4)
                del out, ws
            van = r["vanilla_ms"]
            r["hadamard_over_averis_prep"] = round((r["hadamard_ms"] - van) / max(r["averis_ms"] - van, 1e-9), 2)
            prep[f"{name}_m{m_}"] = r
            print(f"# prep {name} l=65536 m={m_}: vanilla {van*1e3:.0f} us, averis {r['averis_ms']*1e3:.0f} us, "
                  f"hadamard {r['hadamard_ms']*1e3:.0f} us", file=sys.stderr, flush=True)
        del xa

    # Dominant kernel: the MXFP4 GEMM tile kernel.  The vanilla forward and input-gradient GEMMs
    # are exactly one k_gemm launch each (2 l m n flops per launch).  A graph of REPS back-to-back
    # (forward, input-gradient) pairs is replayed after a cache-evicting read; HIP events on the
    # launching stream bracket each replay, so the per-launch time carries no event or launch
    # gaps (inside a graph our kernels run back to back) and can be compared with the kernel
    # trace of the same launches.  The first pair of a replay reads its operands from HBM, the
    # rest find them in the caches.
    REPS = 10
    st = LinearStep(x, d, w, av.MXFP4, split=False)
    st.quantize()

    def gemm_pairs():
        for _ in range(REPS):
            av.linear_fwd(st.sx["row"], None, st.sw["col"], out=st.y, ws=st.ws_fwd)
            av.linear_bwd_dx(st.sd["row"], None, st.sw["row"], out=st.dx, ws=st.ws_dx)

    launch_s = timed(gemm_pairs, args.steps, args.warmup) * 1e-3 / (2 * REPS)
    achieved = 2.0 * l * m * n / launch_s / 1e12
    # the binding roofline of each launch: max(MFMA time, HBM time of its algorithmic bytes:
    # both packed operands read once, the bf16 output written once), averaged over the pair
    op = 0.5 + 1.0 / 32
    t_mfma = 2.0 * l * m * n / (PEAK_FP4_TFLOPS * 1e12)
    t_hbm = [((l * m + n * m) * op + 2 * l * n) / (PEAK_HBM_GBPS * 1e9),   # Y [l, n]
             ((l * n + m * n) * op + 2 * l * m) / (PEAK_HBM_GBPS * 1e9)]   # dX [l, m]
    t_bind = sum(max(t_mfma, t) for t in t_hbm) / 2
    roofline = {"bound": "mfma", "kernel": "k_gemm_ws<MXFP4> (forward and input-gradient GEMMs)",
                "achieved": round(achieved, 1), "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP4_TFLOPS, 4), "traffic": gemm_traffic(),
                "traffic_unit": "bytes per launch (HBM, counter runs)", "launch_us": round(launch_s * 1e6, 2),
                "binding_roofline_us": round(t_bind * 1e6, 2), "frac_of_binding": round(t_bind / launch_s, 4)}
    del st

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lin, args.cpu_rows)

    mx = results["mxfp4"]
    line = {
        "metric": METRIC,
        "value": round(mx["step_tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mx["averis_step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "Qwen3-0.6B-shaped up_proj fwd+dX+dW: l=8192 (4x2048), m=1024, n=3072, "
                               "bf16 in, bf16 Y/dX, fp32 dW, MXFP4 Averis split",
                   "l": l, "m": m, "n": n, "format": "mxfp4"},
        "split_quant": {"GBps": round(mx["quant_GBps"], 1), "frac_hbm": round(mx["quant_GBps"] / PEAK_HBM_GBPS, 4),
                        "us": round(mx["averis_quant_ms"] * 1e3, 2)},
        "gemm": {"TFLOPs": round(mx["gemm_tflops"], 1), "frac_fp4_peak": round(mx["gemm_tflops"] / PEAK_FP4_TFLOPS, 4),
                 "us": round(mx["averis_gemm_ms"] * 1e3, 2)},
        "overhead_pct_vs_vanilla": round(mx["overhead_pct"], 2),
        "vanilla_ms_per_step": round(mx["vanilla_step_ms"], 5),
        "nvfp4": {k: round(v, 5) for k, v in results["nvfp4"].items()},
        "layer_sweep": dict(workload="Qwen3-0.6B-shaped layer sweep: q, k, v, o, gate, up, down linears at "
                                     "l=16384, fwd+dX+dW each, bf16 in", l=16384, linears=7,
                            gflop=round(sweep_flops / 1e9, 1), **sweep),
        "moe": dict(workload="MoE FFN layer: 8192 tokens top-8 of 64 experts (Zipf 1.1), hidden 2048, expert FFN "
                             "768, gate/up/down fwd+dX+dW, grouped launches", routed_rows=moe_rows,
                    gflop=round(3 * 6 * moe_rows * 2048 * 768 / 1e9, 1), **moe),
        "preprocessing": dict(workload="X [65536, m] bf16, row layout only; Averis split vs 16x16 Hadamard "
                                        "vs vanilla FP4 quantization", **prep),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def gemm_traffic():
    """HBM bytes per k_gemm launch from the committed counter summary, or None once the GEMM
    source has changed since those counters were taken."""
    import re
    prof = os.path.join(ROOT, "profiles", "k_gemm_mxfp4_up_proj_traffic.txt")
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


def cpu_baseline(lin, rows):
    """The CPU oracle on a token sample of the same step: X and D rows [0, rows) with all of W.
    W's quantization is a per-step cost; the rest scales with tokens, so the full-step time is
    extrapolated as t_W + (l / rows) * t_rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import averis_oracle as O
    l, m = lin.x.shape
    n = lin.d.shape[1]
    xs, ds = lin.x[:rows], lin.d[:rows]
    t0 = time.perf_counter()
    sw = O.split_quant(lin.w, O.MXFP4, split=False)
    t_w = time.perf_counter() - t0
    t0 = time.perf_counter()
    sx = O.split_quant(xs, O.MXFP4)
    sd = O.split_quant(ds, O.MXFP4)
    O.linear_fwd(sx["row"], sx["mean"], sw["col"])
    O.linear_bwd_dx(sd["row"], sd["mean"], sw["row"])
    O.linear_bwd_dw(sx["col"], sd["col"], sx["mean"], sd["mean"], rows)
    t_r = time.perf_counter() - t0
    t_full = t_w + (l / rows) * t_r
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(6.0 * l * m * n / t_full / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"MXFP4 step on X/D token rows 0..{rows - 1} of {l} with all of W "
                      f"({t_w + t_r:.1f} s measured); full step extrapolated linearly in tokens: {t_full:.1f} s"}


if __name__ == "__main__":
    main()
