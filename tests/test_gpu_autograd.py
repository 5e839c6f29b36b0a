"""The autograd wrapper: forward and backward through torch.autograd give exactly the library's
own entry-point results, and those match the oracle's products of the dequantized operands."""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from fp4_quantized_amd.autograd import AverisLinear, averis_linear
from oracle import averis_oracle as O
from tests.gpu_util import device, rel_fro, to_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", [av.MXFP4, av.NVFP4])
@pytest.mark.parametrize("split", [True, False])
def test_autograd_matches_entry_points_and_oracle(fmt, split):
    dev = device()
    lin = workloads.up_proj_like(31, 640, 256, 384)
    x = workloads.to_torch(lin.x, "f32", dev).requires_grad_(True)
    w = workloads.to_torch(lin.w, "f32", dev).requires_grad_(True)
    d = workloads.to_torch(lin.d, "f32", dev)
    print(f"case autograd fmt={fmt} split={split}", flush=True)
    y = averis_linear(x, w, fmt, split)
    y.backward(d)
    torch.cuda.synchronize()
    # the same calls made directly
    sx = av.split_quant(x.detach(), fmt, split)
    sw = av.split_quant(w.detach(), fmt, False)
    sd = av.split_quant(d, fmt, split)
    mx, md = (sx["mean_q"], sd["mean_q"]) if split else (None, None)
    y2 = av.linear_fwd(sx["row"], mx, sw["col"])
    dx2 = av.linear_bwd_dx(sd["row"], md, sw["row"])
    dw2 = av.linear_bwd_dw(sx["col"], sd["col"], mx, md, 640)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y2) and torch.equal(x.grad, dx2) and torch.equal(w.grad, dw2)
    omx, omd = (to_oracle(mx), to_oracle(md)) if split else (None, None)
    assert rel_fro(y2.cpu().numpy(), O.linear_fwd(to_oracle(sx["row"]), omx, to_oracle(sw["col"]))) <= 1e-5
    assert rel_fro(dx2.cpu().numpy(), O.linear_bwd_dx(to_oracle(sd["row"]), omd, to_oracle(sw["row"]))) <= 1e-5
    assert rel_fro(dw2.cpu().numpy(), O.linear_bwd_dw(to_oracle(sx["col"]), to_oracle(sd["col"]), omx, omd,
                                                       640)) <= 1e-5


def test_module_bf16_shapes_and_dtypes():
    dev = device()
    torch.manual_seed(0)
    layer = AverisLinear(256, 384, device=dev)
    x = (torch.randn(2, 320, 256, device=dev) + 2.0).to(torch.bfloat16).requires_grad_(True)
    y = layer(x)
    assert y.shape == (2, 320, 384) and y.dtype == torch.bfloat16
    y.float().square().mean().backward()
    torch.cuda.synchronize()
    assert x.grad.shape == x.shape and x.grad.dtype == torch.bfloat16
    assert layer.weight.grad.shape == (256, 384) and layer.weight.grad.dtype == torch.bfloat16
    # against the unquantized product: FP4 error, not a wrong result
    ref = x.detach().float().reshape(-1, 256) @ layer.weight.detach().float()
    err = float((y.detach().float().reshape(-1, 384) - ref).norm() / ref.norm())
    assert err < 0.2, err
