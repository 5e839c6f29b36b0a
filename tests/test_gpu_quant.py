"""GPU parity of averis_split_quant against the CPU oracle.

The mean must match the oracle's fp64 mean within 1e-6 (relative to |mu| + mean |x|); given
the GPU's fp32 mean, every packed code, block scale and tensor scale must be bit-exact, in
both layouts and for the quantized mean.
"""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok

pytestmark = pytest.mark.gpu

FMTS = [(av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")]


def run_case(x_np, dtype, fmt, split=True, hadamard=False, mean=None, tag=""):
    dev = device()
    print(f"case {tag} shape={x_np.shape} dtype={dtype} fmt={fmt} split={split} h16={hadamard}", flush=True)
    x = workloads.to_torch(x_np, dtype, dev)
    m_t = torch.from_numpy(mean).to(dev) if mean is not None else None
    g = av.split_quant(x, fmt, split=split, hadamard=hadamard, mean=m_t)
    torch.cuda.synchronize()
    mu_gpu = g["mean"].cpu().numpy() if split else None
    if split and mean is None:
        assert mean_ok(mu_gpu, x_np), f"{tag}: mean outside tolerance"
    if mean is not None:
        np.testing.assert_array_equal(mu_gpu, mean)
    o = O.split_quant(x_np, fmt, split=split, hadamard=hadamard, mean=mu_gpu)
    assert_q_equal(g["row"], o["row"], f"{tag} row layout")
    assert_q_equal(g["col"], o["col"], f"{tag} column layout")
    if split:
        assert_q_equal(g["mean_q"], o["mean"], f"{tag} quantized mean")
    return g, o


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("hadamard", [False, True])
def test_tiny_fp32(fmt, fname, split, hadamard):
    lin = workloads.tiny(0)
    run_case(lin.x, "f32", fmt, split, hadamard, tag=f"tiny-{fname}")
    run_case(lin.w, "f32", fmt, False, hadamard, tag=f"tiny-w-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("rows", [1000, 1, 17, 64, 129, 320])
def test_ragged_bf16(fmt, fname, hadamard, rows):
    # 384 columns = 1.5 column tiles of 256 bf16; rows not a multiple of the 64-row tile
    lin = workloads.up_proj_like(11, rows, 384, 128)
    run_case(lin.x, "bf16", fmt, True, hadamard, tag=f"ragged-{fname}-{rows}")
    run_case(lin.d, "bf16", fmt, True, hadamard, tag=f"ragged-d-{fname}-{rows}")


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("cols", [32, 96, 160, 288])
def test_column_counts_multiple_of_32(fmt, fname, hadamard, cols):
    # columns past the last 256-column tile and past the last 64-column statistics strip
    lin = workloads.up_proj_like(14, 333, cols, 128)
    run_case(lin.x, "bf16", fmt, True, hadamard, tag=f"cols-{cols}-{fname}")
    run_case(lin.x, "f32", fmt, True, hadamard, tag=f"cols-{cols}-f32-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_zero_rows(fmt, fname):
    run_case(np.zeros((0, 256), np.float32), "bf16", fmt, True, False, tag=f"empty-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
def test_degenerate_inputs(fmt, fname, hadamard):
    rng = np.random.default_rng(5)
    mu = workloads._round(rng.standard_normal(256) * 8, "bf16")
    const = np.repeat(mu[None, :], 200, axis=0)            # residual exactly 0 everywhere
    g, _ = run_case(const, "bf16", fmt, True, hadamard, tag=f"constant-cols-{fname}")
    assert not g["row"].codes.any().item() and not g["col"].codes.any().item()
    run_case(np.zeros((96, 128), np.float32), "f32", fmt, True, hadamard, tag=f"zeros-{fname}")
    spikes = workloads._round(rng.standard_normal((300, 256)), "bf16")
    spikes[:, 7] *= 1000.0
    spikes[13, 100] = -3e4
    run_case(workloads._round(spikes, "bf16"), "bf16", fmt, True, hadamard, tag=f"spikes-{fname}")
    tiny_vals = workloads._round(rng.standard_normal((128, 128)) * 1e-30, "f32")
    run_case(tiny_vals, "f32", fmt, True, hadamard, tag=f"tiny-magnitudes-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_mean_given(fmt, fname):
    lin = workloads.up_proj_like(12, 300, 256, 128)
    mean = (lin.x.astype(np.float64).mean(axis=0) + 0.25).astype(np.float32)
    run_case(lin.x, "bf16", fmt, True, False, mean=mean, tag=f"mean-given-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_up_proj_full_size(fmt, fname):
    # l = 8192 tokens, m = 1024, n = 3072: X, D and W in both layouts, full comparison
    lin = workloads.up_proj()
    run_case(lin.x, "bf16", fmt, True, False, tag=f"up_proj-X-{fname}")
    run_case(lin.d, "bf16", fmt, True, False, tag=f"up_proj-D-{fname}")
    run_case(lin.w, "bf16", fmt, False, False, tag=f"up_proj-W-{fname}")


def test_down_proj_hadamard_nvfp4_full_size():
    # l = 16384, m = 3072 SwiGLU-like input with the 16x16 Hadamard on the residual
    lin = workloads.down_proj()
    run_case(lin.x, "bf16", av.NVFP4, True, True, tag="down_proj-X-nvfp4-h16")


def test_deterministic():
    dev = device()
    lin = workloads.up_proj_like(13, 2000, 512, 128)
    x = workloads.to_torch(lin.x, "bf16", dev)
    a = av.split_quant(x, av.NVFP4)
    b = av.split_quant(x, av.NVFP4)
    torch.cuda.synchronize()
    assert torch.equal(a["mean"], b["mean"])
    for k in ("row", "col", "mean_q"):
        assert torch.equal(a[k].codes, b[k].codes) and torch.equal(a[k].scales, b[k].scales)


@pytest.mark.parametrize("fmt,fname,hadamard", [(av.MXFP4, "mxfp4", False), (av.NVFP4, "nvfp4", False),
                                                (av.NVFP4, "nvfp4", True)])
def test_many_tiles_per_workgroup(fmt, fname, hadamard):
    # 16001 rows x 1152 columns (4.5 column tiles of 256 bf16): about 2500 tiles of 32 rows, more
    # than four per workgroup of the persistent launch, so the LDS ring wraps; ragged last rows
    lin = workloads.up_proj_like(31, 16001, 1152, 128)
    run_case(lin.x, "bf16", fmt, True, hadamard, tag=f"many-{fname}-{hadamard}")


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_strided_rows(fmt, fname, dtype):
    # x is a column slice of a wider matrix: row stride 640 elements, 384 columns used
    dev = device()
    lin = workloads.up_proj_like(32, 777, 640, 128)
    wide = workloads.to_torch(lin.x, dtype, dev)
    x = wide[:, :384]
    print(f"case strided-{fname}-{dtype} shape={tuple(x.shape)} ldx={x.stride(0)}", flush=True)
    g = av.split_quant(x, fmt, split=True)
    torch.cuda.synchronize()
    x_np = lin.x[:, :384]
    mu = g["mean"].cpu().numpy()
    assert mean_ok(mu, x_np.astype(np.float64)), "mean"
    o = O.split_quant(np.ascontiguousarray(x_np), fmt, split=True, mean=mu)
    assert_q_equal(g["row"], o["row"], "row layout")
    assert_q_equal(g["col"], o["col"], "column layout")
    assert_q_equal(g["mean_q"], o["mean"], "quantized mean")


def test_workspace_reused_across_calls():
    # the split's workspace carries per-strip arrival counters that each call must leave at
    # zero: three calls on one workspace (different data, both formats) must each match the
    # oracle, and the counters must read zero afterwards
    dev = device()
    rows, cols = 1500, 384
    ws = av.split_quant_workspace(rows, cols, av.NVFP4, split=True, device=dev)
    for k, fmt in enumerate((av.MXFP4, av.NVFP4, av.MXFP4)):
        lin = workloads.up_proj_like(40 + k, rows, cols, 128)
        print(f"case reuse-{k} fmt={fmt}", flush=True)
        g = av.split_quant(workloads.to_torch(lin.x, "bf16", dev), fmt, split=True, ws=ws)
        torch.cuda.synchronize()
        mu = g["mean"].cpu().numpy()
        assert mean_ok(mu, lin.x), f"call {k}: mean"
        o = O.split_quant(lin.x, fmt, split=True, mean=mu)
        assert_q_equal(g["row"], o["row"], f"call {k} row layout")
        assert_q_equal(g["col"], o["col"], f"call {k} column layout")
        assert_q_equal(g["mean_q"], o["mean"], f"call {k} quantized mean")
    # header: amax slots (3 + 2 uint32, padded to 256 bytes), then one 128-byte line per
    # 64-column strip holding that strip's counter (the rest of the line stays zero)
    counters = ws[256:256 + 128 * (cols // 64)].cpu().numpy().view(np.uint32)
    assert not counters.any(), f"strip counters left at {counters.reshape(-1, 32)[:, 0]}"


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("split", [True, False])
def test_single_layout_nvfp4_hadamard(layout, split):
    # NVFP4 + Hadamard takes its rotated amax in a separate pass, which covers only the layouts
    # requested: each one alone must still equal the oracle's
    dev = device()
    lin = workloads.up_proj_like(41, 300, 256, 128)
    print(f"case single-layout {layout} split={split}", flush=True)
    x = workloads.to_torch(lin.x, "bf16", dev)
    g = av.split_quant(x, av.NVFP4, split=split, hadamard=True, row=layout == "row", col=layout == "col")
    torch.cuda.synchronize()
    assert g["row" if layout == "col" else "col"] is None
    mu_gpu = g["mean"].cpu().numpy() if split else None
    o = O.split_quant(lin.x, av.NVFP4, split=split, hadamard=True, mean=mu_gpu)
    assert_q_equal(g[layout], o[layout], f"single {layout} layout")
    if split:
        assert_q_equal(g["mean_q"], o["mean"], "quantized mean")


def _golden():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "blocks.json")) as f:
        return json.load(f)


def _golden_rows(values, rows=32, cols=128):
    """fp32 [rows, cols]: row 0 starts with the golden values, everything else is zero."""
    x = np.zeros((rows, cols), np.float32)
    x[0, :len(values)] = np.asarray(values, np.float32)
    return x


def test_golden_mxfp4_subnormal_scale_block():
    # hand-worked block with amax 2^-126: E = -128 clamps to -127 (scale byte 0, a subnormal
    # 2^-127 decode scale) and the elements scale by 2^127 (tests/golden/blocks.json, MXFP4
    # case 5): the GPU's row layout must hold exactly those codes and that scale byte
    c = _golden()["mxfp4"][4]
    g, _ = run_case(_golden_rows(c["values"]), "f32", av.MXFP4, False, False, tag="golden-mx-subnormal")
    codes = O.unpack_nibbles(g["row"].codes[0].cpu().numpy())[:32]
    np.testing.assert_array_equal(codes, c["codes"], err_msg=c["name"])
    from tests.gpu_util import row_scales
    assert int(row_scales(g["row"])[0, 0]) == c["scale"], c["name"]


@pytest.mark.parametrize("case", [0, 1, 2])
def test_golden_nvfp4_blocks_on_gpu(case):
    # the hand-worked NVFP4 rows (tests/golden/blocks.json) as row 0 of an otherwise zero operand,
    # so the tensor amax is the row's: case 2's tensor decode scale is an fp32 subnormal and its
    # second block's decode scale falls below 2^-126 (that block's codes are zero)
    c = _golden()["nvfp4"][case]
    g, _ = run_case(_golden_rows(c["values"]), "f32", av.NVFP4, False, False, tag=f"golden-nv-{case}")
    nv = len(c["values"])
    codes = O.unpack_nibbles(g["row"].codes[0].cpu().numpy())[:nv]
    np.testing.assert_array_equal(codes, c["codes"], err_msg=c["name"])
    from tests.gpu_util import row_scales
    np.testing.assert_array_equal(row_scales(g["row"])[0, :nv // 16], c["scales"], err_msg=c["name"])
    assert np.float32(g["row"].tensor_scale[0].item()) == np.float32(c["s_dec"]), c["name"]


def test_golden_nvfp4_hadamard_block_on_gpu():
    # NVFP4 with the 16x16 rotation: the tensor scale comes from the rotated operand's amax
    c = _golden()["nvfp4_hadamard"][0]
    g, _ = run_case(_golden_rows(c["values"]), "f32", av.NVFP4, False, True, tag="golden-nv-h16")
    codes = O.unpack_nibbles(g["row"].codes[0].cpu().numpy())[:32]
    np.testing.assert_array_equal(codes, c["codes"], err_msg=c["name"])
    from tests.gpu_util import row_scales
    np.testing.assert_array_equal(row_scales(g["row"])[0, :2], c["scales"], err_msg=c["name"])
    assert np.float32(g["row"].tensor_scale[0].item()) == np.float32(c["s_dec"]), c["name"]


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("split", [True, False])
def test_check_finite_status(fmt, fname, dtype, split):
    # AVERIS_CHECK_FINITE: status 0 and unchanged outputs for finite inputs; the non-finite bit for
    # a NaN or an infinity anywhere; the status word cleared by every call (one workspace reused)
    dev = device()
    lin = workloads.up_proj_like(91, 300, 384, 8)
    x_np = workloads._round(lin.x, dtype)
    ws = av.split_quant_workspace(300, 384, fmt, split, device=dev)
    x = workloads.to_torch(x_np, dtype, dev)
    print(f"case check-finite {fname} {dtype} split={split}", flush=True)
    for bad, where in ((np.nan, (0, 0)), (np.inf, (299, 383)), (-np.inf, (150, 200)), (None, None)):
        xb = x.clone()
        if bad is not None:
            xb[where] = bad
        g = av.split_quant(xb, fmt, split, ws=ws, check_finite=True)
        torch.cuda.synchronize()
        st = int(g["status"].item())
        if bad is None:
            assert st == 0, f"status {st} for finite input"
            ref = av.split_quant(x, fmt, split)
            torch.cuda.synchronize()
            for k in ("row", "col"):
                assert torch.equal(g[k].codes, ref[k].codes) and torch.equal(g[k].scales, ref[k].scales)
        else:
            assert st & av.STATUS_NONFINITE, f"status {st} for {bad} at {where}"


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_check_finite_reports_scale_underflow(fmt, fname):
    # a block whose scale underflows: the NVFP4 golden row whose second block is zeroed, and an
    # MXFP4 block of amax 2^-126 (exponent clamped at -127); a normal operand reports nothing
    dev = device()
    c = _golden()["nvfp4"][2] if fmt == av.NVFP4 else _golden()["mxfp4"][4]
    x = workloads.to_torch(_golden_rows(c["values"]), "f32", dev)
    g = av.split_quant(x, fmt, split=False, check_finite=True)
    torch.cuda.synchronize()
    assert int(g["status"].item()) == av.STATUS_UNDERFLOW
    lin = workloads.up_proj_like(92, 256, 256, 8)
    g = av.split_quant(workloads.to_torch(lin.x, "bf16", dev), fmt, split=True, check_finite=True)
    torch.cuda.synchronize()
    assert int(g["status"].item()) == 0


def test_check_finite_grouped():
    dev = device()
    lens = [0, 37, 300, 1]
    x_np = workloads.up_proj_like(93, sum(lens), 256, 8).x
    grp = av.Groups(np.concatenate([[0], np.cumsum(lens)]), dev)
    x = workloads.to_torch(x_np, "bf16", dev)
    ws = av.split_quant_grouped_workspace(sum(lens), 256, len(lens), av.MXFP4, device=dev)
    L = av.lib()
    for bad in (None, np.nan):
        xb = x.clone()
        if bad is not None:
            xb[40, 17] = bad
        out = av.split_quant_grouped_outputs(grp, 256, av.MXFP4, device=dev)
        st = L.averis_split_quant_grouped(xb.data_ptr(), av.BF16, 256, 256, grp.d.data_ptr(), grp.h, grp.E, av.MXFP4,
                                          av.SPLIT | av.CHECK_FINITE, out["mean"].data_ptr(), av._ptr(out["row"]),
                                          av._ptr(out["col"]), av._ptr(out["mean_q"]), ws.data_ptr(), ws.numel(),
                                          av._stream())
        assert st == 0
        torch.cuda.synchronize()
        word = int(ws[:4].view(torch.int32).item())
        assert word == (0 if bad is None else av.STATUS_NONFINITE), word
