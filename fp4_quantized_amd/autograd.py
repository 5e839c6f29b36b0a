"""A W4A4G4 linear layer as a torch.autograd.Function on top of the C-ABI.

Forward quantizes X (split into its column mean and residual) and W, and returns
Y = 1 (mu_X W) + X_R W; backward quantizes the output gradient D the same way and returns
dX = 1 (mu_D W^T) + D_R W^T and dW = X_R^T D_R + l mu_X^T mu_D ("均值偏置的诅咒与祝福" explainer,
paper.rainbus.top, section 方法步骤详情).  With split=False it is the vanilla FP4 linear.
Every product runs in the HIP library; torch supplies memory and the stream.
"""
from __future__ import annotations

import torch

from . import averis as av


class AverisLinearFn(torch.autograd.Function):
    """y = linear(x, w) for x [l, m], w [m, n] (bf16 or fp32, row-major), y [l, n] in x's dtype."""

    @staticmethod
    def forward(ctx, x, w, fmt=av.MXFP4, split=True, hadamard=False):
        x = x.contiguous()
        w = w.contiguous()
        sx = av.split_quant(x, fmt, split, hadamard)
        sw = av.split_quant(w, fmt, False, hadamard)
        y = av.linear_fwd(sx["row"], sx["mean_q"] if split else None, sw["col"], out_dtype=x.dtype)
        ctx.sx, ctx.sw = sx, sw
        ctx.cfg = (fmt, split, hadamard, x.shape[0], x.dtype, w.dtype)
        return y

    @staticmethod
    def backward(ctx, dy):
        fmt, split, hadamard, l, xdt, wdt = ctx.cfg
        sx, sw = ctx.sx, ctx.sw
        sd = av.split_quant(dy.contiguous(), fmt, split, hadamard)
        mx = sx["mean_q"] if split else None
        md = sd["mean_q"] if split else None
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = av.linear_bwd_dx(sd["row"], md, sw["row"], out_dtype=xdt)
        if ctx.needs_input_grad[1]:
            dw = av.linear_bwd_dw(sx["col"], sd["col"], mx, md, l)
            if wdt != torch.float32:
                dw = dw.to(wdt)
        ctx.sx = ctx.sw = None
        return dx, dw, None, None, None


def averis_linear(x, w, fmt=av.MXFP4, split=True, hadamard=False):
    """Functional form: x [l, m] @ w [m, n] with FP4 operands and the mean-residual split."""
    return AverisLinearFn.apply(x, w, fmt, split, hadamard)


class AverisLinear(torch.nn.Module):
    """Bias-free linear layer y = x W with weight [in_features, out_features]."""

    def __init__(self, in_features, out_features, fmt=av.MXFP4, split=True, hadamard=False, device=None,
                 dtype=torch.bfloat16):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.empty(in_features, out_features, device=device, dtype=dtype))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.fmt, self.split, self.hadamard = fmt, split, hadamard

    def forward(self, x):
        lead = x.shape[:-1]
        y = averis_linear(x.reshape(-1, x.shape[-1]), self.weight, self.fmt, self.split, self.hadamard)
        return y.reshape(*lead, y.shape[-1])
