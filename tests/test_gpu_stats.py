"""GPU parity of the producer-fused column statistics: a GEMM that writes X also writes the
column partials of what it stored, and the split of X starts from them.

Per case:
  * the GEMM's output equals the plain entry point's bit for bit (the statistics change no
    arithmetic of the product, which test_gpu_gemm.py checks against the oracle);
  * the partial sums are those of the stored output: within fp32 summation error of the fp64
    sums of each part's rows (at most 12 roundings deep: a lane's rows in order, then a 32-lane
    tree; or 8 rows in fp32, then fp64), 12 * 2^-24 of the magnitude sum, and minima and maxima
    exact;
  * the split from the statistics: its mean within the mean tolerance of the oracle's column
    mean of the stored output, and, given that mean, every code, block scale and tensor scale
    bit-exact against the oracle's split of the same output (and equal to the GPU's own split
    with that mean given).
The output of the GEMM is the input of the split under test here, so the oracle is handed the
GPU's stored output, as it is handed the GPU's mean: the step is checked on the input it gets.
"""
import ctypes

import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok

pytestmark = pytest.mark.gpu


def operands(l, m, n, fmt, seed):
    dev = device()
    lin = workloads.up_proj_like(seed, l, m, n)
    x = workloads.to_torch(lin.x, "bf16", dev)
    d = workloads.to_torch(lin.d, "bf16", dev)
    w = workloads.to_torch(lin.w, "bf16", dev)
    return av.split_quant(x, fmt), av.split_quant(d, fmt), av.split_quant(w, fmt, split=False)


def check_partials(st, yh, depth=12):
    rows, cols = yh.shape
    assert st.cs.rows == rows and st.cs.cols == cols
    pr = st.part_rows
    assert st.parts == -(-rows // pr)
    got = st.view("sum").cpu().numpy().astype(np.float64)
    y64 = yh.astype(np.float64)
    for p in range(st.parts):
        blk = y64[p * pr:(p + 1) * pr]
        ref = blk.sum(axis=0)
        tol = depth * 2.0 ** -24 * np.abs(blk).sum(axis=0) + 1e-45
        bad = np.abs(got[p] - ref) > tol
        assert not bad.any(), f"part {p}: {bad.sum()} column sums off"
        if st.min is not None:
            assert np.array_equal(st.view("min").cpu().numpy()[p], blk.min(axis=0).astype(np.float32))
            assert np.array_equal(st.view("max").cpu().numpy()[p], blk.max(axis=0).astype(np.float32))


def check_split(y, st, fmt, hadamard, tag):
    sq = av.split_quant_stats(y, st, fmt, hadamard=hadamard)
    mu = sq["mean"]
    again = av.split_quant(y, fmt, hadamard=hadamard, mean=mu)
    torch.cuda.synchronize()
    yh = y.float().cpu().numpy()
    muh = mu.cpu().numpy()
    assert mean_ok(muh, yh), f"{tag}: mean from the statistics"
    ref = O.split_quant(yh, fmt, hadamard=hadamard, mean=muh)
    for lay in ("row", "col"):
        assert_q_equal(sq[lay], ref[lay], f"{tag}: {lay} layout")
        assert_q_equal(again[lay], ref[lay], f"{tag}: {lay} layout, mean given")
    assert_q_equal(sq["mean_q"], ref["mean"], f"{tag}: quantized mean")


CASES = [
    # (tag, fmt, l, m, n, out dtype, minmax, expected part rows)
    ("mxfp4-ws-bf16", av.MXFP4, 4000, 512, 1024, torch.bfloat16, False, 64),
    ("mxfp4-ws-f32", av.MXFP4, 4000, 512, 1024, torch.float32, False, 64),
    ("mxfp4-wide-bf16", av.MXFP4, 8200, 512, 1024, torch.bfloat16, False, 128),
    ("mxfp4-splitk-bf16", av.MXFP4, 1000, 512, 384, torch.bfloat16, False, 512),
    ("mxfp4-minmax-bf16", av.MXFP4, 4000, 512, 1024, torch.bfloat16, True, 512),
    ("nvfp4-short-bf16", av.NVFP4, 4000, 512, 1024, torch.bfloat16, False, 64),
    ("nvfp4-minmax-bf16", av.NVFP4, 4000, 512, 1024, torch.bfloat16, True, 512),
]


@pytest.mark.parametrize("tag,fmt,l,m,n,odt,minmax,part_rows", CASES, ids=[c[0] for c in CASES])
def test_forward_stats_then_split(tag, fmt, l, m, n, odt, minmax, part_rows):
    print(f"case {tag}", flush=True)
    sx, _, sw = operands(l, m, n, fmt, seed=11)
    st = av.ColStats(l, n, minmax=minmax)
    y = av.linear_fwd_stats(sx["row"], sx["mean_q"], sw["col"], st, odt)
    y0 = av.linear_fwd(sx["row"], sx["mean_q"], sw["col"], odt)
    torch.cuda.synchronize()
    assert st.part_rows == part_rows, f"{tag}: part rows {st.part_rows}"
    assert torch.equal(y, y0), f"{tag}: output differs from the plain forward GEMM"
    check_partials(st, y.float().cpu().numpy())
    if odt == torch.bfloat16:
        hs = [False, True] if (fmt == av.MXFP4 or minmax) else [True]
        for h in hs:
            check_split(y, st, fmt, h, f"{tag}{'-h16' if h else ''}")


@pytest.mark.parametrize("fmt,fname", [(av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")])
def test_input_gradient_stats_then_split(fmt, fname):
    # dX [l, m] of an up projection: the next D of the layer below
    tag = f"dx-{fname}"
    print(f"case {tag}", flush=True)
    l, m, n = 4000, 1024, 512
    _, sd, sw = operands(l, m, n, fmt, seed=12)
    st = av.ColStats(l, m, minmax=fmt == av.NVFP4)
    dx = av.linear_bwd_dx_stats(sd["row"], sd["mean_q"], sw["row"], st, torch.bfloat16)
    dx0 = av.linear_bwd_dx(sd["row"], sd["mean_q"], sw["row"], torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx0), f"{tag}: output differs from the plain input-gradient GEMM"
    check_partials(st, dx.float().cpu().numpy())
    check_split(dx, st, fmt, False, tag)


def test_layer_shape_forward_stats_then_split():
    # the gate projection of the layer workload at full size (16384 tokens, 1024 -> 3072): the
    # 256 x 128 warp-specialized tiles, sums in the epilogue
    dev = device()
    print("case layer-gate-mxfp4", flush=True)
    _, x, _, w = next(c for c in workloads.layer_device(3, 16384, dev, shared=True) if c[0] == "gate")
    sx = av.split_quant(x, av.MXFP4)
    sw = av.split_quant(w, av.MXFP4, split=False)
    st = av.ColStats(x.shape[0], w.shape[1])
    y = av.linear_fwd_stats(sx["row"], sx["mean_q"], sw["col"], st, torch.bfloat16)
    torch.cuda.synchronize()
    assert st.part_rows == 128
    check_partials(st, y.float().cpu().numpy())
    check_split(y, st, av.MXFP4, False, "layer-gate-mxfp4")


def test_empty_output_rows():
    dev = device()
    print("case empty", flush=True)
    _, _, sw = operands(64, 512, 256, av.MXFP4, seed=13)
    xr = av.empty_qtensor(0, 512, av.MXFP4, device=dev)
    mu = av.split_quant(torch.zeros(64, 512, dtype=torch.bfloat16, device=dev), av.MXFP4)["mean_q"]
    st = av.ColStats(0, 256)
    y = av.linear_fwd_stats(xr, mu, sw["col"], st, torch.bfloat16)
    sq = av.split_quant_stats(y, st, av.MXFP4)
    torch.cuda.synchronize()
    assert st.parts == 0 and y.shape == (0, 256)
    assert not sq["mean"].any()


def test_stats_argument_errors():
    dev = device()
    print("case errors", flush=True)
    sx, _, sw = operands(256, 512, 256, av.NVFP4, seed=14)
    small = av.ColStats(64, 256)
    with pytest.raises(av.AverisError, match="sizes"):
        av.linear_fwd_stats(sx["row"], sx["mean_q"], sw["col"], small, torch.bfloat16)
    st = av.ColStats(256, 256)
    y = av.linear_fwd_stats(sx["row"], sx["mean_q"], sw["col"], st, torch.bfloat16)
    # NVFP4 without the Hadamard takes its residual tensor scale from minima and maxima
    with pytest.raises(av.AverisError, match="NULL"):
        av.split_quant_stats(y, st, av.NVFP4)
    # statistics of another shape
    with pytest.raises(av.AverisError, match="sizes"):
        av.split_quant_stats(y[:128], st, av.NVFP4, hadamard=True)
    L = av.lib()
    out = av.split_quant_outputs(256, 256, av.NVFP4, True, True, device=dev)
    ws = av.split_quant_workspace(256, 256, av.NVFP4, True, True, dev)
    st_ = L.averis_split_quant_stats(y.data_ptr(), av.BF16, 256, 256, 256, av.NVFP4,
                                     av.SPLIT | av.HADAMARD16 | av.MEAN_GIVEN, ctypes.byref(st.cs),
                                     out["mean"].data_ptr(), av._ptr(out["row"]), av._ptr(out["col"]),
                                     av._ptr(out["mean_q"]), ws.data_ptr(), ws.numel(), av._stream())
    assert st_ == 6  # AVERIS_E_FLAGS
    torch.cuda.synchronize()
