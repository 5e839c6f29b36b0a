"""GPU parity of the producers with column statistics (RMSNorm, SwiGLU) and of the split that
starts from their statistics.

Per case:
  * the output against the oracle's RMSNorm / SwiGLU of the same input: within one bf16 unit in
    the last place of the oracle's value (the kernels sum the squares in fp32 and use the
    device exp, the oracle sums in fp64 and rounds exp correctly), and equal for at least 99 %
    of the elements (fp32 outputs: within 2^-20 relative);
  * the same output bit for bit when no statistics are asked for;
  * the partial sums are those of the stored output (20 * 2^-24 of the magnitude sum of each
    64-row part: sixteen rows per lane in order, then four waves), minima and maxima exact;
  * the split from the statistics: mean within the mean tolerance of the oracle's column mean of
    the stored output; given that mean every code, block scale and tensor scale bit-exact
    against the oracle's split of the same output.
"""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok
from tests.test_gpu_stats import check_partials

pytestmark = pytest.mark.gpu


def close_to_oracle(got, ref, bf16, tag):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if bf16:
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        bad = np.abs(got - ref) > ulp
        assert not bad.any(), f"{tag}: {int(bad.sum())} elements more than one bf16 ulp off"
        same = np.mean(got == ref)
        assert same >= 0.99, f"{tag}: only {same:.4f} of the elements equal"
    else:
        bad = np.abs(got - ref) > 2.0 ** -20 * np.abs(ref) + 1e-30
        assert not bad.any(), f"{tag}: {int(bad.sum())} elements off"


def split_from(y, st, fmt, hadamard, tag):
    sq = av.split_quant_stats(y, st, fmt, hadamard=hadamard)
    torch.cuda.synchronize()
    yh = y.float().cpu().numpy()
    muh = sq["mean"].cpu().numpy()
    assert mean_ok(muh, yh), f"{tag}: mean from the statistics"
    ref = O.split_quant(yh, fmt, hadamard=hadamard, mean=muh)
    for lay in ("row", "col"):
        assert_q_equal(sq[lay], ref[lay], f"{tag}: {lay} layout")
    assert_q_equal(sq["mean_q"], ref["mean"], f"{tag}: quantized mean")


def inputs(l, m, seed, dt):
    lin = workloads.up_proj_like(seed, l, m, 32, dtype=dt)
    return lin.x


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("l,m", [(1000, 1024), (130, 1056), (64, 32)])
def test_rmsnorm_stats(l, m, dt):
    dev = device()
    tag = f"rmsnorm-{l}x{m}-{dt}"
    print(f"case {tag}", flush=True)
    xh = inputs(l, m, 50, dt)
    x = workloads.to_torch(xh, dt, dev)
    w = torch.from_numpy(np.random.default_rng(51).standard_normal(m).astype(np.float32) * 0.5 + 1).to(dev)
    st = av.ColStats(l, m, minmax=True)
    y = av.rmsnorm(x, w, 1e-6, stats=st)
    y0 = av.rmsnorm(x, w, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(y, y0), f"{tag}: output differs without statistics"
    assert st.part_rows == 64
    ref = O.rmsnorm(np.asarray(xh, np.float32), w.cpu().numpy(), 1e-6, out_bf16=dt == "bf16")
    close_to_oracle(y.float().cpu().numpy(), ref, dt == "bf16", tag)
    check_partials(st, y.float().cpu().numpy(), depth=20)
    if dt == "bf16":
        for fmt, h in ((av.MXFP4, False), (av.NVFP4, False), (av.NVFP4, True)):
            split_from(y, st, fmt, h, f"{tag}-{fmt}{'-h16' if h else ''}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("l,m", [(1000, 3072), (70, 544)])
def test_swiglu_stats(l, m, dt):
    dev = device()
    tag = f"swiglu-{l}x{m}-{dt}"
    print(f"case {tag}", flush=True)
    gh = inputs(l, m, 52, dt)
    uh = inputs(l, m, 53, dt)
    g, u = workloads.to_torch(gh, dt, dev), workloads.to_torch(uh, dt, dev)
    st = av.ColStats(l, m, minmax=True)
    y = av.swiglu(g, u, stats=st)
    y0 = av.swiglu(g, u)
    torch.cuda.synchronize()
    assert torch.equal(y, y0), f"{tag}: output differs without statistics"
    ref = O.swiglu(np.asarray(gh, np.float32), np.asarray(uh, np.float32), out_bf16=dt == "bf16")
    close_to_oracle(y.float().cpu().numpy(), ref, dt == "bf16", tag)
    check_partials(st, y.float().cpu().numpy(), depth=20)
    if dt == "bf16":
        for fmt in (av.MXFP4, av.NVFP4):
            split_from(y, st, fmt, False, f"{tag}-{fmt}")


def test_layer_shape_producers():
    # the block's two producer shapes at 16384 tokens: RMSNorm of the residual stream (1024),
    # SwiGLU of the gate and up outputs (3072); sums only (MXFP4 consumers), sampled comparison
    dev = device()
    print("case layer-producers", flush=True)
    layers = workloads.layer_device(3, 16384, dev, shared=True)
    x = next(c for c in layers if c[0] == "gate")[1]
    w = torch.ones(x.shape[1], dtype=torch.float32, device=dev)
    st = av.ColStats(*x.shape)
    y = av.rmsnorm(x, w, 1e-6, stats=st)
    g = next(c for c in layers if c[0] == "down")[1]
    u = torch.flip(g, dims=[0])  # an up operand of the same distribution
    st2 = av.ColStats(*g.shape)
    z = av.swiglu(g, u, stats=st2)
    torch.cuda.synchronize()
    rows = np.random.default_rng(54).choice(x.shape[0], 256, replace=False)
    close_to_oracle(y.float().cpu().numpy()[rows],
                    O.rmsnorm(x.float().cpu().numpy()[rows], w.cpu().numpy(), 1e-6), True, "layer rmsnorm rows")
    close_to_oracle(z.float().cpu().numpy()[rows],
                    O.swiglu(g.float().cpu().numpy()[rows], u.float().cpu().numpy()[rows]), True, "layer swiglu rows")
    check_partials(st, y.float().cpu().numpy(), depth=20)
    check_partials(st2, z.float().cpu().numpy(), depth=20)
    split_from(y, st, av.MXFP4, False, "layer rmsnorm mxfp4")
    split_from(z, st2, av.MXFP4, False, "layer swiglu mxfp4")


def test_producer_argument_errors():
    dev = device()
    print("case producer-errors", flush=True)
    x = torch.zeros(128, 96, dtype=torch.bfloat16, device=dev)
    w = torch.ones(96, dtype=torch.float32, device=dev)
    with pytest.raises(av.AverisError, match="sizes"):
        av.rmsnorm(x[:, :48], w)                       # cols % 32
    with pytest.raises(av.AverisError, match="sizes"):
        av.rmsnorm(x, w, stats=av.ColStats(64, 96))    # capacity for 64 rows, not 128
    with pytest.raises(av.AverisError, match="sizes"):
        av.rmsnorm(x, w, eps=-1.0)
    y = av.rmsnorm(torch.zeros(0, 96, dtype=torch.bfloat16, device=dev), w, stats=av.ColStats(0, 96))
    assert y.shape == (0, 96)
    torch.cuda.synchronize()
