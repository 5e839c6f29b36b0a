"""GPU parity of the batched split + quantization (averis_split_quant_batch).

Each batched tensor is quantized on its own, so every output must be bit-identical to a single
averis_split_quant call on the same tensor (whose parity with the oracle the single-call tests
establish); one tensor per batch is also checked against the oracle directly.  Shapes mix row
counts (with an empty tensor and ragged tails), column counts and, in one batch, the seven
weights of the Qwen3-0.6B-shaped layer.
"""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok, to_oracle

pytestmark = pytest.mark.gpu

SHAPES = [(300, 384), (0, 96), (1000, 1056), (64, 32), (2048, 512)]
LAYER_W = [(1024, 2048), (1024, 1024), (1024, 1024), (2048, 1024), (1024, 3072), (1024, 3072), (3072, 1024)]


def same(a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    if isinstance(a, torch.Tensor):
        assert torch.equal(a, b), what
        return
    assert torch.equal(a.codes, b.codes), f"{what} codes"
    assert torch.equal(a.scales, b.scales), f"{what} scales"
    if a.tensor_scale is not None:
        assert torch.equal(a.tensor_scale, b.tensor_scale), f"{what} tensor scale"


def check_batch(xs, fmt, split, hadamard, tag):
    print(f"case {tag} n={len(xs)} fmt={fmt} split={split} h16={hadamard}", flush=True)
    outs = av.split_quant_batch(xs, fmt, split=split, hadamard=hadamard)
    singles = [av.split_quant(x, fmt, split=split, hadamard=hadamard) for x in xs]
    torch.cuda.synchronize()
    for i, (g, r) in enumerate(zip(outs, singles)):
        for k in ("mean", "row", "col", "mean_q"):
            same(g[k], r[k], f"{tag} tensor {i} {k}")
    # the largest tensor against the oracle as well
    i = max(range(len(xs)), key=lambda j: xs[j].numel())
    xh = xs[i].float().cpu().numpy()
    mu = outs[i]["mean"].cpu().numpy() if split else None
    if split:
        assert mean_ok(mu, xh), f"{tag}: mean"
    o = O.split_quant(xh, fmt, split=split, hadamard=hadamard, mean=mu)
    assert_q_equal(outs[i]["row"], o["row"], f"{tag} oracle row layout")
    assert_q_equal(outs[i]["col"], o["col"], f"{tag} oracle column layout")


@pytest.mark.parametrize("fmt,fname", [(av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")])
@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_batch_matches_single_calls(fmt, fname, split, hadamard, dt):
    dev = device()
    xs = [workloads.to_torch(workloads.up_proj_like(70 + i, r, c, 32).x, dt, dev) for i, (r, c) in enumerate(SHAPES)]
    check_batch(xs, fmt, split, hadamard, f"mixed-{fname}-{dt}")


@pytest.mark.parametrize("fmt,fname", [(av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")])
def test_batch_of_the_layer_weights(fmt, fname):
    # the seven weights of the layer in one launch pair (no split), and eight tensors (the most a
    # batch takes) with the split
    dev = device()
    rng = np.random.default_rng(75)
    ws = [torch.from_numpy((rng.standard_normal(s) * 0.02).astype(np.float32)).to(dev).to(torch.bfloat16) for s in LAYER_W]
    check_batch(ws, fmt, False, False, f"layer-weights-{fname}")
    xs = [workloads.to_torch(workloads.up_proj_like(80 + i, 512 + 96 * i, 256, 32).x, "bf16", dev) for i in range(8)]
    check_batch(xs, fmt, True, False, f"eight-{fname}")


def test_batch_reuses_workspaces():
    # a second batch on the same workspaces (the strip counters are back at zero) gives the same
    # bytes; two items on one workspace are refused
    dev = device()
    print("case batch-reuse", flush=True)
    xs = [workloads.to_torch(workloads.up_proj_like(90 + i, 700, 512, 32).x, "bf16", dev) for i in range(3)]
    wss = [av.split_quant_workspace(700, 512, av.MXFP4, True, False, dev) for _ in xs]
    a = av.split_quant_batch(xs, av.MXFP4, wss=wss)
    b = av.split_quant_batch(xs, av.MXFP4, wss=wss)
    torch.cuda.synchronize()
    for i in range(3):
        for k in ("mean", "row", "col", "mean_q"):
            same(a[i][k], b[i][k], f"reuse tensor {i} {k}")
    with pytest.raises(av.AverisError, match="workspace"):
        av.split_quant_batch(xs[:2], av.MXFP4, wss=[wss[0], wss[0]])


@pytest.mark.parametrize("fmt,fname", [(av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")])
def test_layer_step_batched_quantization_is_unchanged(fmt, fname):
    # the layer step's batched launches (weights; q/k/v and gate/up output gradients) write the
    # same bytes as one launch per tensor
    from fp4_quantized_amd.step import LayerStep
    dev = device()
    print(f"case layer-step-batched-{fname}", flush=True)
    layers = workloads.layer_device(3, 1000, dev, shared=True)
    a = LayerStep(layers, fmt, split=True, batched=True)
    b = LayerStep(layers, fmt, split=True, batched=False)
    assert max(len(g) for g in a.groups) == 7 and len(a.groups) < len(b.groups)
    a.quantize()
    b.quantize()
    torch.cuda.synchronize()
    for i, (qa, qb) in enumerate(zip(a.quants, b.quants)):
        for k in ("mean", "row", "col", "mean_q"):
            same(qa[2][k], qb[2][k], f"{fname} tensor {i} {k}")


def test_layer_step_training_order_is_unchanged():
    # run() interleaves splits and GEMMs in a training step's order; every output equals that of
    # all splits followed by all GEMMs
    from fp4_quantized_amd.step import LayerStep
    dev = device()
    print("case layer-step-order", flush=True)
    layers = workloads.layer_device(3, 1000, dev, shared=True, cat=True)
    a = LayerStep(layers, av.MXFP4, split=True)
    b = LayerStep(layers, av.MXFP4, split=True)
    a.run()
    b.quantize()
    b.gemms()
    torch.cuda.synchronize()
    for ca, cb in zip(a.lin, b.lin):
        for k in ("y", "dx", "dw"):
            assert torch.equal(ca[k], cb[k]), f"{ca['name']} {k}"


@pytest.mark.parametrize("fmt,fname", [(av.MXFP4, "mxfp4"), (av.NVFP4, "nvfp4")])
def test_layer_step_overlap_matches_one_stream(fmt, fname):
    # the two-stream step (weights and weight gradients on a second stream), eager and replayed
    # from a graph three times (outputs cleared between replays), equals the one-stream step
    from fp4_quantized_amd.step import LayerStep
    dev = device()
    print(f"case layer-step-overlap-{fname}", flush=True)
    layers = workloads.layer_device(3, 1000, dev, shared=True, cat=True)
    a = LayerStep(layers, fmt, split=True, overlap=True)
    b = LayerStep(layers, fmt, split=True, overlap=False)
    assert a.side is not None and b.side is None
    b.run()
    a.run()
    torch.cuda.synchronize()

    def check(tag):
        for ca, cb in zip(a.lin, b.lin):
            for k in ("y", "dx", "dw"):
                assert torch.equal(ca[k], cb[k]), f"{tag} {ca['name']} {k}"

    check("eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        a.run()
    for r in range(3):
        for c in a.lin:
            for k in ("y", "dx", "dw"):
                c[k].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(f"replay {r}")


@pytest.mark.parametrize("cat", [False, True])
@pytest.mark.parametrize("split", [True, False])
def test_layer_step_fused_shared_input_gemms(split, cat):
    # q, k and v share their input, so their weight gradients are the column blocks of one GEMM
    # X_R^T [D_q D_k D_v] (+ l mu_X^T [mu_Dq mu_Dk mu_Dv]), and q/k/v and gate/up have one
    # forward GEMM each, X_R [W_1 .. W_k]^T: every quantized operand equals the unfused step's
    # (the D column layouts, their means and the weights' K = m layouts are views into one
    # operand), Y is bit-identical, dW agrees up to fp32 summation order (the unfused launches
    # split K) and against the oracle.  cat: the D_i and W_i of q/k/v and of gate/up are column
    # blocks of one tensor each, which are then split once, and each group runs one input
    # gradient GEMM, [D_1 .. D_k] [W_1 .. W_k]^T + 1 mu_D W^T: the sum of the unfused dX_i up to
    # fp32 summation order, and the oracle's dX of the concatenated operands
    from fp4_quantized_amd.step import LayerStep
    from tests.gpu_util import rel_fro
    dev = device()
    print(f"case layer-step-fused split={split} cat={cat}", flush=True)
    layers = workloads.layer_device(3, 1000, dev, shared=True, cat=cat)
    a = LayerStep(layers, av.MXFP4, split=split, out_dtype=torch.float32)
    b = LayerStep(layers, av.MXFP4, split=split, out_dtype=torch.float32, fuse_dw=False, fuse_fwd=False,
                  fuse_dx=False)
    assert list(a.dw_fused) == [0] and not b.dw_fused  # q/k/v fused; gate/up would need two tile rounds
    assert list(a.fwd_fused) == [0, 2] and not b.fwd_fused  # q/k/v and gate/up
    assert list(a.dx_fused) == ([0, 2] if cat else []) and not b.dx_fused
    # 4 inputs, then 7 output gradients and 7 weights, or with cat 2 + 2 of each
    assert len(a.quants) == (4 + 2 * 4 if cat else 18) and len(b.quants) == 18
    a.run()
    b.run()
    torch.cuda.synchronize()
    grouped = ("q", "k", "v", "gate", "up") if cat else ()
    for ca, cb in zip(a.lin, b.lin):
        for k in ("mean", "row", "col", "mean_q"):
            same(ca["sx"][k], cb["sx"][k], f"{ca['name']} X {k}")
        for k in ("mean", "col", "mean_q") + (() if ca["name"] in grouped else ("row",)):
            same(ca["sd"][k], cb["sd"][k], f"{ca['name']} D {k}")
        same(ca["sw"]["col"], cb["sw"]["col"], f"{ca['name']} W col")
        if ca["name"] not in grouped:
            same(ca["sw"]["row"], cb["sw"]["row"], f"{ca['name']} W row")
        assert torch.equal(ca["y"], cb["y"]), ca["name"]
        e = rel_fro(ca["dw"].cpu().numpy(), cb["dw"].cpu().numpy())
        assert e <= 1e-6, f"{ca['name']} dW: {e:.3e}"
    for pi, (_, _, lins) in enumerate(a.x_plan):
        got = a.lin[lins[0]]["dx"]
        if pi not in a.dx_fused:
            for li in lins:
                assert torch.equal(a.lin[li]["dx"], b.lin[li]["dx"]), a.lin[li]["name"]
            continue
        assert all(a.lin[li]["dx"] is got for li in lins)
        e = rel_fro(got.cpu().numpy(), sum(b.lin[li]["dx"].double() for li in lins).cpu().numpy())
        assert e <= 1e-6, f"group {pi} dX against the sum of the unfused dX_i: {e:.3e}"
    # the fused block of k against the oracle
    name, x, d, w = layers[1]
    c = a.lin[1]
    assert name == "k" == c["name"]
    xh, dh = x.float().cpu().numpy(), d.float().cpu().numpy()
    assert_q_equal(c["sw"]["col"], O.split_quant(w.float().cpu().numpy(), av.MXFP4, split=False)["col"],
                   "k: W K = m layout (view)")
    ox = O.split_quant(xh, av.MXFP4, split=split, mean=c["sx"]["mean"].cpu().numpy() if split else None)
    od = O.split_quant(dh, av.MXFP4, split=split, mean=c["sd"]["mean"].cpu().numpy() if split else None)
    assert_q_equal(c["sd"]["col"], od["col"], "k: D column layout (view)")
    if split:
        assert_q_equal(c["sd"]["mean_q"], od["mean"], "k: quantized mean of D (view)")
    ref = O.linear_bwd_dw(ox["col"], od["col"], ox["mean"], od["mean"], x.shape[0])
    e = rel_fro(c["dw"].cpu().numpy(), ref)
    assert e <= 1e-5, f"k dW against the oracle: {e:.3e}"
    if cat:
        # gate/up's one input gradient against the oracle on the concatenated D and W
        f = a.dx_fused[2]
        dp = torch.cat([cc[2] for cc in layers if cc[0] in ("gate", "up")], 1).float().cpu().numpy()
        wp = torch.cat([cc[3] for cc in layers if cc[0] in ("gate", "up")], 1).float().cpu().numpy()
        if split:
            assert mean_ok(f["d"]["mean"].cpu().numpy(), dp), "gate/up: mean of D"
        odp = O.split_quant(dp, av.MXFP4, split=split, mean=f["d"]["mean"].cpu().numpy() if split else None)
        owp = O.split_quant(wp, av.MXFP4, split=False)
        assert_q_equal(f["d"]["row"], odp["row"], "gate/up: D row layout")
        assert_q_equal(f["w"]["row"], owp["row"], "gate/up: W row layout")
        ref = O.linear_bwd_dx(odp["row"], odp["mean"] if split else None, owp["row"])
        e = rel_fro(f["dx"].cpu().numpy(), ref)
        assert e <= 1e-5, f"gate/up dX against the oracle: {e:.3e}"
