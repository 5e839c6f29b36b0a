"""GPU parity at the full sizes of the layer, down_proj and MoE workloads, compared in full.

Every case goes through the entry points the bench times.  Means within the 1e-6 mean
tolerance; given the GPU's mean, every code, block scale and tensor scale of every quantized
operand bit-exact against the oracle's quantization of the same input; fp32 GEMM outputs within
1e-5 relative Frobenius error of the oracle's fp64 products of the dequantized operands
(computed from the oracle's own bytes, which equal the GPU's).
  * layer (l = 16384, the bench's device draws, q/k/v and gate/up sharing their input): per
    linear X, D and W in every layout and the quantized means in full, dW in full, and 256 rows
    of fp32 Y and dX (the full products of the seven linears are checked in the down_proj
    cases below, whose shapes they share);
  * down_proj (l = 16384, 3072 -> 1024, SwiGLU-like input) in its four variants {NVFP4, MXFP4} x
    {Hadamard off, on}: every operand and fp32 Y, dX and dW in full;
  * MoE (8192 tokens, top-8 of 64 experts, Zipf routing): the grouped quantization of the routed
    token states, the down projection's input and its output gradient for every expert, and the
    down projection (768 -> 2048) forward, input and weight gradients for every expert.
"""
import functools

import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from fp4_quantized_amd.step import LinearStep
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok, rel_fro

pytestmark = pytest.mark.gpu

FMTS = [(av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")]
TOL = 1e-5
LAYER = [name for name, _, _ in workloads.SWEEP_LAYERS]


@functools.lru_cache(maxsize=1)
def _layer():
    return workloads.layer_device(3, 16384, device(), shared=True)


def quantized_in_full(st, xh, dh, wh, fmt, hadamard, what):
    """Means and every quantized operand of a LinearStep against the oracle; returns the
    oracle's split outputs for X, D and W."""
    mux, mud = st.sx["mean"].cpu().numpy(), st.sd["mean"].cpu().numpy()
    assert mean_ok(mux, xh), f"{what}: mean of X"
    assert mean_ok(mud, dh), f"{what}: mean of D"
    ox = O.split_quant(xh, fmt, hadamard=hadamard, mean=mux)
    od = O.split_quant(dh, fmt, hadamard=hadamard, mean=mud)
    ow = O.split_quant(wh, fmt, split=False, hadamard=hadamard)
    for lay in ("row", "col"):
        assert_q_equal(st.sx[lay], ox[lay], f"{what}: X {lay} layout")
        assert_q_equal(st.sd[lay], od[lay], f"{what}: D {lay} layout")
        assert_q_equal(st.sw[lay], ow[lay], f"{what}: W {lay} layout")
    assert_q_equal(st.sx["mean_q"], ox["mean"], f"{what}: quantized mean of X")
    assert_q_equal(st.sd["mean_q"], od["mean"], f"{what}: quantized mean of D")
    return ox, od, ow


def sub(q, rows):
    return O.QTensor(q.codes[rows], q.scales[rows], q.s_dec, q.fmt, q.k, q.rotated)


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("name", LAYER)
def test_layer_linear_full(name, fmt, fname):
    _, x, d, w = next(c for c in _layer() if c[0] == name)
    l, m = x.shape
    n = d.shape[1]
    what = f"layer-{name}-{fname}"
    print(f"case {what} l={l} m={m} n={n}", flush=True)
    st = LinearStep(x, d, w, fmt, split=True, out_dtype=torch.float32)
    st.run()
    torch.cuda.synchronize()
    xh, dh, wh = (t.float().cpu().numpy() for t in (x, d, w))
    ox, od, ow = quantized_in_full(st, xh, dh, wh, fmt, False, what)
    del xh, dh
    dw_ref = O.linear_bwd_dw(ox["col"], od["col"], ox["mean"], od["mean"], l)
    err = rel_fro(st.dw.cpu().numpy(), dw_ref)
    assert err <= TOL, f"{what}: dW relative Frobenius error {err:.3e}"
    rng = np.random.default_rng(100 + LAYER.index(name))
    rows = np.unique(np.concatenate([[0, 1, 255, 256, l - 1], rng.choice(l, 251, replace=False)]))
    y_ref = O.linear_fwd(sub(ox["row"], rows), ox["mean"], ow["col"])
    dx_ref = O.linear_bwd_dx(sub(od["row"], rows), od["mean"], ow["row"])
    err_y = rel_fro(st.y.cpu().numpy()[rows], y_ref)
    err_dx = rel_fro(st.dx.cpu().numpy()[rows], dx_ref)
    assert err_y <= TOL, f"{what}: Y rows relative Frobenius error {err_y:.3e}"
    assert err_dx <= TOL, f"{what}: dX rows relative Frobenius error {err_dx:.3e}"


@functools.lru_cache(maxsize=1)
def _down_proj():
    return workloads.down_proj()


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
def test_down_proj_full(fmt, fname, hadamard):
    dev = device()
    lin = _down_proj()
    what = f"down_proj-{fname}{'-h16' if hadamard else ''}"
    print(f"case {what}", flush=True)
    x, d, w = (workloads.to_torch(a, "bf16", dev) for a in (lin.x, lin.d, lin.w))
    l = lin.x.shape[0]
    st = LinearStep(x, d, w, fmt, split=True, hadamard=hadamard, out_dtype=torch.float32)
    st.run()
    torch.cuda.synchronize()
    ox, od, ow = quantized_in_full(st, lin.x, lin.d, lin.w, fmt, hadamard, what)
    for out, ref in ((st.y, O.linear_fwd(ox["row"], ox["mean"], ow["col"])),
                     (st.dx, O.linear_bwd_dx(od["row"], od["mean"], ow["row"])),
                     (st.dw, O.linear_bwd_dw(ox["col"], od["col"], ox["mean"], od["mean"], l))):
        err = rel_fro(out.cpu().numpy(), ref)
        del ref
        assert err <= TOL, f"{what}: relative Frobenius error {err:.3e}"


@functools.lru_cache(maxsize=1)
def _moe():
    return workloads.moe()


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_moe_grouped_quant_full(fmt, fname):
    # every expert's slice of the routed token states [65536, 2048], of the down projection's
    # input [65536, 768] and of its output gradient [65536, 2048]
    from tests.test_gpu_moe import grouped_quant_case
    mo = _moe()
    lens = [int(v) for v in np.diff(mo.offsets)]
    grouped_quant_case(mo.x, lens, fmt, tag=f"moe-x-{fname}")
    grouped_quant_case(mo.x_down, lens, fmt, tag=f"moe-xdown-{fname}")
    grouped_quant_case(mo.d_down, lens, fmt, tag=f"moe-ddown-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_moe_down_projection_full(fmt, fname):
    # the down projection (768 -> 2048) of every expert: grouped forward, input gradient and
    # weight gradient, each expert against the oracle in full
    dev = device()
    mo = _moe()
    lens = [int(v) for v in np.diff(mo.offsets)]
    E, f = len(lens), mo.x_down.shape[1]
    h = mo.d_down.shape[1]
    print(f"case moe-down-{fname} E={E}", flush=True)
    grp = av.Groups(mo.offsets, dev)
    wgrp = av.Groups(np.arange(E + 1) * f, dev)
    w = mo.w_down.reshape(E * f, h)
    gx = av.split_quant_grouped(workloads.to_torch(mo.x_down, "bf16", dev), grp, fmt)
    gd = av.split_quant_grouped(workloads.to_torch(mo.d_down, "bf16", dev), grp, fmt)
    gw = av.split_quant_grouped(workloads.to_torch(w, "bf16", dev), wgrp, fmt, split=False)
    y = av.linear_fwd_grouped(gx["row"], gx["mean_q"], av.stacked_weight_view(gw["col"], E, f), grp)
    dx = av.linear_bwd_dx_grouped(gd["row"], gd["mean_q"], gw["row"], grp)
    dw = av.linear_bwd_dw_grouped(gx["col"], gd["col"], gx["mean_q"], gd["mean_q"], grp)
    torch.cuda.synchronize()
    mx, md = gx["mean"].cpu().numpy(), gd["mean"].cpu().numpy()
    y, dx, dw = y.cpu().numpy(), dx.cpu().numpy(), dw.cpu().numpy()
    for e in range(E):
        a, b = int(mo.offsets[e]), int(mo.offsets[e + 1])
        what = f"moe-down-{fname} expert {e} (l_e={b - a})"
        if b == a:
            assert not dw[e].any(), f"{what}: empty expert dW"
            continue
        ox = O.split_quant(mo.x_down[a:b], fmt, mean=mx[e])
        od = O.split_quant(mo.d_down[a:b], fmt, mean=md[e])
        ow = O.split_quant(w[e * f:(e + 1) * f], fmt, split=False)
        for got, ref, nm in ((y[a:b], O.linear_fwd(ox["row"], ox["mean"], ow["col"]), "forward"),
                             (dx[a:b], O.linear_bwd_dx(od["row"], od["mean"], ow["row"]), "input gradient"),
                             (dw[e], O.linear_bwd_dw(ox["col"], od["col"], ox["mean"], od["mean"], b - a),
                              "weight gradient")):
            err = rel_fro(got, ref)
            assert err <= TOL, f"{what}: {nm} {err:.3g}"
