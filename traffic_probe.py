"""Launches whose HBM traffic and MFMA use are read with rocprofv3 counters.

Run under `rocprofv3 --pmc FETCH_SIZE` and again under `--pmc WRITE_SIZE` (or other counters, or
`--kernel-trace` for the same launches' durations).  In order: a plain 64 MiB device copy (known
bytes: it calibrates the counters, whose request-size accounting need not match this GPU's line
size), then, each after a 512 MiB read that evicts the caches so that operands come from HBM:
  gemm   (default) the forward GEMM with the mean term of the layer's gate and up linears
         together (their shared input times both weights, MXFP4, 16384 x 6144 x 1024, bf16 Y):
         the longest launch of bench.py's layer step and its roofline kernel; then the same GEMM
         without the mean term;
  quant  the split+quant of the gate linear's input X [16384, 1024] and output gradient
         D [16384, 3072] (MXFP4, mean split), then their vanilla quantization.
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
    from fp4_quantized_amd.step import LayerStep

    dev = torch.device("cuda:0")
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    a = torch.ones(16 << 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    gate = [c for c in workloads.layer_device(3, 16384, dev, shared=True) if c[0] in ("gate", "up")]
    st = LayerStep(gate, av.MXFP4, split=True)
    st.quantize()
    f = st.fwd_fused[0]  # gate and up share X: one forward GEMM
    torch.cuda.synchronize()
    flush.sum()
    b.copy_(a)                      # calibration: 64 MiB read, 64 MiB written
    if mode == "quant":
        sv = LayerStep(gate, av.MXFP4, split=False)
        torch.cuda.synchronize()
        for t, sp, out, ws in [st.quants[i] for i in (0, 1)] + [sv.quants[i] for i in (0, 1)]:
            flush.sum()
            av.split_quant(t, av.MXFP4, sp, out=out, ws=ws)
    else:
        flush.sum()
        av.linear_fwd(f["sx"]["row"], f["sx"]["mean_q"], f["w"], out=f["y"], ws=f["ws"])
        flush.sum()
        av.linear_fwd(f["sx"]["row"], None, f["w"], out=f["y"], ws=f["ws"])
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else "gemm")
