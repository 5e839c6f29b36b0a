"""GPU parity of averis_split_quant_sr (stochastic rounding) against the CPU oracle.

Both sides draw from Philox4x32-10 under the same seed with the same counter per element, so
codes are compared bit-exactly, as for round to nearest: means within the mean tolerance,
block and tensor scales those of round to nearest, every code equal to the oracle's
stochastically rounded code given the GPU's mean.
"""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok, rel_fro, to_oracle

pytestmark = pytest.mark.gpu

FMTS = [(av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")]


def sr_case(x_np, dtype, fmt, split, hadamard, seed, tag):
    dev = device()
    print(f"case {tag} shape={x_np.shape} dtype={dtype} fmt={fmt} split={split} h16={hadamard} seed={seed}",
          flush=True)
    x = workloads.to_torch(x_np, dtype, dev)
    g = av.split_quant(x, fmt, split=split, hadamard=hadamard, sr_seed=seed)
    torch.cuda.synchronize()
    mu = g["mean"].cpu().numpy() if split else None
    if split:
        assert mean_ok(mu, x_np), f"{tag}: mean"
    o = O.split_quant(x_np, fmt, split=split, hadamard=hadamard, mean=mu, sr_seed=seed)
    assert_q_equal(g["row"], o["row"], f"{tag} row layout")
    assert_q_equal(g["col"], o["col"], f"{tag} column layout")
    if split:
        assert_q_equal(g["mean_q"], o["mean"], f"{tag} quantized mean")
    return g, o


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("split", [True, False])
def test_sr_small(fmt, fname, hadamard, split):
    lin = workloads.up_proj_like(71, 333, 384, 160)
    sr_case(lin.d, "bf16", fmt, split, hadamard, 0x1234_5678_9ABC_DEF0, f"sr-d-{fname}")
    sr_case(lin.x, "f32", fmt, split, hadamard, 3, f"sr-x-f32-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_sr_seeds_differ_and_repeat(fmt, fname):
    dev = device()
    lin = workloads.up_proj_like(72, 256, 256, 128)
    x = workloads.to_torch(lin.d, "bf16", dev)
    a = av.split_quant(x, fmt, sr_seed=11)
    b = av.split_quant(x, fmt, sr_seed=11)
    c = av.split_quant(x, fmt, sr_seed=12)
    r = av.split_quant(x, fmt)
    torch.cuda.synchronize()
    assert torch.equal(a["row"].codes, b["row"].codes) and torch.equal(a["col"].codes, b["col"].codes)
    assert not torch.equal(a["row"].codes, c["row"].codes)
    assert not torch.equal(a["row"].codes, r["row"].codes)
    assert torch.equal(a["row"].scales, r["row"].scales)


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_sr_up_proj_gradient_full_size_and_input_gradient(fmt, fname):
    # the up_proj output gradient D [8192, 3072] quantized stochastically in both layouts, then
    # the input-gradient GEMM on it against the oracle's product of the same operands
    dev = device()
    lin = workloads.up_proj()
    g, o = sr_case(lin.d, "bf16", fmt, True, False, 2026, f"sr-up-proj-D-{fname}")
    sw = av.split_quant(workloads.to_torch(lin.w, "bf16", dev), fmt, split=False)
    dx = av.linear_bwd_dx(g["row"], g["mean_q"], sw["row"])
    torch.cuda.synchronize()
    ref = O.linear_bwd_dx(o["row"], o["mean"], to_oracle(sw["row"]))
    err = rel_fro(dx.cpu().numpy(), ref)
    assert err <= 1e-5, f"input gradient on stochastically rounded D: {err:.3e}"
