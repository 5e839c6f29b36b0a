"""GPU parity of the grouped (MoE) entry points against the CPU oracle, expert by expert.

Per expert the grouped path must equal the dense path on the expert's token slice: its mean
within the mean tolerance; given that mean, codes, block scales and tensor scales bit-exact in
every grouped layout (padding rows and tokens zero); GEMM outputs within 1e-5 relative
Frobenius error of the oracle's exact product of the dequantized operands.
"""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok, rel_fro, untile_scales

pytestmark = pytest.mark.gpu

FMTS = [(av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")]
TOL = 1e-5


def ru(a, b):
    return (a + b - 1) // b * b


def row_view(q, grp, e):
    """Group e's block of a grouped row layout as a dense QTensor [l_e, k]."""
    g = av.BLOCK[q.fmt]
    r0, le = grp.row_starts[e], grp.lens[e]
    nb = q.k_pad // g
    sc = q.scales.view(-1)[r0 * nb:(r0 + ru(le, 32)) * nb].view(ru(le, 32), nb)
    ts = q.tensor_scale[e:e + 1] if q.tensor_scale is not None else None
    return av.QTensor(q.codes[r0:r0 + le], sc, ts, le, q.k, q.fmt, q.rotated)


def col_view(q, grp, e):
    """Group e's [cols, round_up(l_e, 256)] operand of a grouped column layout."""
    g = av.BLOCK[q.fmt]
    t0, le, cols = grp.tok_starts[e], grp.lens[e], q.outer
    kp = ru(le, 256)
    codes = q.codes.view(-1)[cols * t0 // 2:cols * (t0 + kp) // 2].view(cols, kp // 2)
    sc = q.scales.view(-1)[cols * t0 // g:cols * (t0 + kp) // g].view(cols, kp // g)
    ts = q.tensor_scale[e:e + 1] if q.tensor_scale is not None else None
    return av.QTensor(codes, sc, ts, cols, le, q.fmt, q.rotated)


def check_mean_row(qm, e, o_mean, what):
    g = av.BLOCK[qm.fmt]
    np.testing.assert_array_equal(qm.codes[e].cpu().numpy(), o_mean.codes[0], err_msg=what)
    full = untile_scales(qm.scales.cpu().numpy(), qm.outer, qm.k_pad, g)
    np.testing.assert_array_equal(full[e], o_mean.scales[0], err_msg=what)
    assert not full[qm.outer:].any(), f"{what}: mean scale rows past E not zero"
    if o_mean.s_dec is not None:
        assert np.float32(qm.tensor_scale[e].item()) == o_mean.s_dec, what


def grouped_quant_case(x_np, lens, fmt, hadamard=False, split=True, tag=""):
    dev = device()
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    print(f"case {tag} lens={list(lens)} cols={x_np.shape[1]} fmt={fmt} h16={hadamard} split={split}", flush=True)
    grp = av.Groups(offs, dev)
    x = workloads.to_torch(x_np, "bf16", dev)
    g = av.split_quant_grouped(x, grp, fmt, split=split, hadamard=hadamard)
    torch.cuda.synchronize()
    means = g["mean"].cpu().numpy() if split else None
    oracle = []
    for e, le in enumerate(lens):
        a, b = int(offs[e]), int(offs[e + 1])
        what = f"{tag} expert {e} (l_e={le})"
        mu = means[e] if split else None
        if split:
            if le == 0:
                assert not means[e].any(), what
            else:
                assert mean_ok(means[e], x_np[a:b]), f"{what}: mean"
        o = O.split_quant(x_np[a:b], fmt, split=split, hadamard=hadamard, mean=mu)
        oracle.append(o)
        rv = row_view(g["row"], grp, e)
        assert_q_equal(rv, o["row"], f"{what} row layout")
        r0 = grp.row_starts[e]
        assert not g["row"].codes[r0 + le:r0 + ru(le, 32)].any().item(), f"{what}: padding rows"
        assert_q_equal(col_view(g["col"], grp, e), o["col"], f"{what} column layout")
        if split:
            check_mean_row(g["mean_q"], e, o["mean"], f"{what} quantized mean")
    return grp, g, oracle


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
def test_grouped_split_quant_ragged(fmt, fname, hadamard):
    lens = [0, 37, 300, 1, 129, 0, 64]
    x = workloads.up_proj_like(21, sum(lens), 256, 8).x
    grouped_quant_case(x, lens, fmt, hadamard, tag=f"ragged-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_grouped_weights_vanilla(fmt, fname):
    # stacked per-expert weights [E * m, n] with groups of m rows: split off, both layouts
    rng = np.random.default_rng(22)
    E, m, n = 3, 96, 128
    w = workloads._round(rng.standard_normal((E * m, n)) * 0.02, "bf16")
    grouped_quant_case(w, [m] * E, fmt, split=False, tag=f"weights-{fname}")


def moe_case(fmt, lens, m, n, seed, hadamard=False, experts=None, tag="", split=True):
    """Grouped forward, input gradient and weight gradient of one MoE linear, expert by expert
    (split=False: the vanilla GEMMs, no mean terms)."""
    dev = device()
    rng = np.random.default_rng(seed)
    E = len(lens)
    L = int(sum(lens))
    x = workloads.up_proj_like(seed, L, m, 8).x
    d = workloads._grad(rng, L, n, "bf16")
    w = workloads._round(rng.standard_normal((E * m, n)) * 0.02, "bf16")
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    print(f"moe case {tag} E={E} L={L} m={m} n={n} fmt={fmt} h16={hadamard} split={split}", flush=True)
    grp = av.Groups(offs, dev)
    wgrp = av.Groups(np.arange(E + 1) * m, dev)
    gx = av.split_quant_grouped(workloads.to_torch(x, "bf16", dev), grp, fmt, split=split, hadamard=hadamard)
    gd = av.split_quant_grouped(workloads.to_torch(d, "bf16", dev), grp, fmt, split=split, hadamard=hadamard)
    gw = av.split_quant_grouped(workloads.to_torch(w, "bf16", dev), wgrp, fmt, split=False, hadamard=hadamard)
    w_fwd = av.stacked_weight_view(gw["col"], E, m)
    y = av.linear_fwd_grouped(gx["row"], gx["mean_q"], w_fwd, grp)
    dx = av.linear_bwd_dx_grouped(gd["row"], gd["mean_q"], gw["row"], grp)
    dw = av.linear_bwd_dw_grouped(gx["col"], gd["col"], gx["mean_q"], gd["mean_q"], grp)
    torch.cuda.synchronize()
    mx = gx["mean"].cpu().numpy() if split else [None] * E
    md = gd["mean"].cpu().numpy() if split else [None] * E
    y, dx, dw = y.cpu().numpy(), dx.cpu().numpy(), dw.cpu().numpy()
    for e in (range(E) if experts is None else experts):
        a, b = int(offs[e]), int(offs[e + 1])
        what = f"{tag} expert {e} (l_e={b - a})"
        if b == a:
            assert not dw[e].any(), f"{what}: empty expert dW"
            continue
        ox = O.split_quant(x[a:b], fmt, split=split, hadamard=hadamard, mean=mx[e])
        od = O.split_quant(d[a:b], fmt, split=split, hadamard=hadamard, mean=md[e])
        ow = O.split_quant(w[e * m:(e + 1) * m], fmt, split=False, hadamard=hadamard)
        ref_y = O.linear_fwd(ox["row"], ox["mean"], ow["col"])
        ref_dx = O.linear_bwd_dx(od["row"], od["mean"], ow["row"])
        ref_dw = O.linear_bwd_dw(ox["col"], od["col"], ox["mean"], od["mean"], b - a)
        assert rel_fro(y[a:b], ref_y) <= TOL, f"{what}: forward {rel_fro(y[a:b], ref_y):.3g}"
        assert rel_fro(dx[a:b], ref_dx) <= TOL, f"{what}: input gradient {rel_fro(dx[a:b], ref_dx):.3g}"
        assert rel_fro(dw[e], ref_dw) <= TOL, f"{what}: weight gradient {rel_fro(dw[e], ref_dw):.3g}"


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
def test_grouped_linear_small(fmt, fname, hadamard):
    moe_case(fmt, [0, 37, 300, 1, 129, 0, 64], 256, 128, 23, hadamard, tag=f"small-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_grouped_linear_small_vanilla(fmt, fname):
    moe_case(fmt, [0, 37, 300, 1, 129, 0, 64], 256, 128, 27, tag=f"small-vanilla-{fname}", split=False)


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("split", [True, False])
def test_grouped_linear_empty_experts_between_full_ones(fmt, fname, split):
    # 48 experts of 8 weight-gradient tiles each (384 units for 256 workgroups): a workgroup's
    # units then belong to different experts, and empty experts (a third of them) sit between
    # non-empty ones in its walk; every expert is checked
    rng = np.random.default_rng(28)
    lens = [0 if e % 3 == 1 else int(rng.integers(1, 400)) for e in range(48)]
    moe_case(fmt, lens, 512, 256, 29, tag=f"gaps-{fname}-{'averis' if split else 'vanilla'}", split=split)


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_grouped_linear_many_experts(fmt, fname):
    # more than 64 groups: the group lookup scans in chunks of 64
    rng = np.random.default_rng(24)
    lens = list(rng.integers(0, 40, size=70))
    moe_case(fmt, lens, 128, 128, 25, tag=f"many-{fname}", experts=[0, 1, 63, 64, 65, 69])


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_moe_full_size_sampled_experts(fmt, fname):
    # the MoE workload's routing: 8192 tokens, top-8 of 64 experts with Zipf(1.1) skew, so the
    # expert slices range from a few hundred to several thousand rows; gate projection
    # 2048 -> 768.  Every GPU output is produced for all experts; the oracle checks the largest,
    # a middle and the smallest expert in full.
    rng = np.random.default_rng(4)
    _, counts = workloads.zipf_topk_counts(rng, 8192, 64, 8)
    order = np.argsort(counts)
    pick = sorted({int(order[-1]), int(order[len(order) // 2]), int(order[0])})
    moe_case(fmt, [int(c) for c in counts], 2048, 768, 26, experts=pick, tag=f"moe-{fname}")


def test_moe_step_matches_grouped_calls():
    # the bench's MoE step (preallocated outputs and workspaces, one grouped launch per kernel)
    # gives exactly what the grouped entry points give when called one by one
    from fp4_quantized_amd.step import MoEStep
    dev = device()
    print("case moe-step", flush=True)
    x, x_down, d_gate, d_up, d_dn, w_gate, w_up, w_down, offs = workloads.moe_device(
        5, tokens=512, hidden=256, ffn=128, experts=8, device=dev)
    st = MoEStep(x, x_down, d_gate, d_up, d_dn, w_gate, w_up, w_down, offs, av.MXFP4)
    st.run()
    torch.cuda.synchronize()
    grp = av.Groups(offs, dev)
    wgrp = av.Groups(np.arange(9) * 256, dev)
    gx = av.split_quant_grouped(x, grp, av.MXFP4)
    gd = av.split_quant_grouped(d_up, grp, av.MXFP4)
    gw = av.split_quant_grouped(w_up, wgrp, av.MXFP4, split=False)
    y = av.linear_fwd_grouped(gx["row"], gx["mean_q"], av.stacked_weight_view(gw["col"], 8, 256), grp, torch.bfloat16)
    dx = av.linear_bwd_dx_grouped(gd["row"], gd["mean_q"], gw["row"], grp, torch.bfloat16)
    dw = av.linear_bwd_dw_grouped(gx["col"], gd["col"], gx["mean_q"], gd["mean_q"], grp)
    torch.cuda.synchronize()
    _, args_y, kw_y = st.gemms[3]
    _, _, kw_dx = st.gemms[4]
    _, _, kw_dw = st.gemms[5]
    assert torch.equal(kw_y["out"], y) and torch.equal(kw_dx["out"], dx) and torch.equal(kw_dw["dw"], dw)


@pytest.mark.parametrize("fused", [False, True])
def test_moe_step_overlap_matches_one_stream(fused):
    # the two-stream MoE step (weights and weight gradients on a second stream), eager and
    # replayed from a graph three times (outputs cleared between replays), equals the one-stream
    # step
    from fp4_quantized_amd.step import MoEStep
    dev = device()
    print(f"case moe-step-overlap fused={fused}", flush=True)
    inp = workloads.moe_device(5, tokens=2048, hidden=256, ffn=384, experts=8, device=dev)
    a = MoEStep(*inp[:8], inp[8], av.MXFP4, overlap=True, fuse_gate_up=fused)
    b = MoEStep(*inp[:8], inp[8], av.MXFP4, overlap=False, fuse_gate_up=fused)
    b.run()
    a.run()
    torch.cuda.synchronize()
    outs = lambda st: [kw[k] for _, _, kw in st.gemms for k in ("out", "dw") if k in kw]  # noqa: E731

    def check(tag):
        for i, (ta, tb) in enumerate(zip(outs(a), outs(b))):
            assert torch.equal(ta, tb), f"{tag} output {i}"

    check("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        a.run()
    for r in range(3):
        for t in outs(a):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {r}")


def test_moe_step_fused_gate_up_matches_separate():
    # gate and up as one projection hidden -> 2 ffn: with MXFP4 the means, Y = [Y_gate | Y_up]
    # and dW = [dW_gate | dW_up] equal the separate projections' bit for bit, and the one
    # input-gradient GEMM gives D_gate W_gate^T + D_up W_up^T (fp32 outputs here: within the
    # fp32 summation order of the two terms)
    from fp4_quantized_amd.step import MoEStep
    dev = device()
    print("case moe-step-fused-gate-up", flush=True)
    inp = workloads.moe_device(6, tokens=1024, hidden=512, ffn=384, experts=8, device=dev)
    f = 384
    a = MoEStep(*inp[:8], inp[8], av.MXFP4, out_dtype=torch.float32, overlap=False, fuse_gate_up=True)
    b = MoEStep(*inp[:8], inp[8], av.MXFP4, out_dtype=torch.float32, overlap=False, fuse_gate_up=False)
    a.run()
    b.run()
    torch.cuda.synchronize()
    ma, mg, mu = a.q["dgu"]["mean"], b.q["dg"]["mean"], b.q["du"]["mean"]
    assert torch.equal(ma[:, :f], mg) and torch.equal(ma[:, f:], mu), "output-gradient means"
    ya, yg, yu = a.gemms[0][2]["out"], b.gemms[0][2]["out"], b.gemms[3][2]["out"]
    assert torch.equal(ya[:, :f], yg) and torch.equal(ya[:, f:], yu), "forward"
    wa, wg, wu = a.gemms[2][2]["dw"], b.gemms[2][2]["dw"], b.gemms[5][2]["dw"]
    assert torch.equal(wa[:, :, :f], wg) and torch.equal(wa[:, :, f:], wu), "weight gradient"
    for i in (3, 4, 5):  # the down projection is the same in both
        ka = "out" if "out" in a.gemms[i][2] else "dw"
        assert torch.equal(a.gemms[i][2][ka], b.gemms[i + 3][2][ka]), f"down gemm {i}"
    dxa = a.gemms[1][2]["out"].double()
    dxs = b.gemms[1][2]["out"].double() + b.gemms[4][2]["out"].double()
    e = float(torch.linalg.norm(dxa - dxs) / torch.linalg.norm(dxs))
    assert e <= 1e-6, f"input gradient: {e:.3e}"
