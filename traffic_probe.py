"""Launches whose HBM traffic and MFMA use are read with rocprofv3 counters.

Run under `rocprofv3 --pmc FETCH_SIZE` and again under `--pmc WRITE_SIZE` (or other counters, or
`--kernel-trace` for the same launches' durations).  In order: a plain 64 MiB device copy (known
bytes: it calibrates the counters, whose request-size accounting need not match this GPU's line
size), then, each after a 512 MiB read that evicts the caches so that operands come from HBM:
  default  the up_proj MXFP4 forward and input-gradient GEMMs (vanilla operands, the roofline
           kernel of bench.py);
  quant    the up_proj MXFP4 split+quant of X and D (mean split) and W, then the vanilla
           quantization of X and D (l = 8192, m = 1024, n = 3072, bf16 inputs).
"""
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main(mode="gemm"):
    import torch

    import fp4_quantized_amd.averis as av
    from fp4_quantized_amd import workloads
    from fp4_quantized_amd.step import LinearStep

    dev = torch.device("cuda:0")
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    a = torch.ones(16 << 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    lin = workloads.up_proj()
    x, d, w = (workloads.to_torch(t, "bf16", dev) for t in (lin.x, lin.d, lin.w))
    st = LinearStep(x, d, w, av.MXFP4, split=False)
    st.quantize()
    if mode == "quant":
        sa = LinearStep(x, d, w, av.MXFP4, split=True)
        sa.quantize()
        torch.cuda.synchronize()
        flush.sum()
        b.copy_(a)
        for s_, t, ou, ws_, split in ((sa, x, sa.sx, sa.ws_x, True), (sa, d, sa.sd, sa.ws_d, True),
                                      (sa, w, sa.sw, sa.ws_w, False), (st, x, st.sx, st.ws_x, False),
                                      (st, d, st.sd, st.ws_d, False)):
            flush.sum()
            av.split_quant(t, av.MXFP4, split, out=ou, ws=ws_)
        torch.cuda.synchronize()
        print("traffic probe done", flush=True)
        return
    torch.cuda.synchronize()
    flush.sum()
    b.copy_(a)                      # calibration: 64 MiB read, 64 MiB written
    flush.sum()
    av.linear_fwd(st.sx["row"], None, st.sw["col"], out=st.y, ws=st.ws_fwd)
    flush.sum()
    av.linear_bwd_dx(st.sd["row"], None, st.sw["row"], out=st.dx, ws=st.ws_dx)
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "gemm")
