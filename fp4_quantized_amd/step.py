"""One linear layer's quantized training step on preallocated buffers.

The step is the whole Averis hot path of one linear layer ("均值偏置的诅咒与祝福" explainer,
paper.rainbus.top, section 方法步骤详情): split + quantize the activations X and the output
gradients D, quantize the weights W, then the forward GEMM Y, the input-gradient GEMM dX and
the weight-gradient GEMM dW with the mean terms.  With split=False it is the vanilla FP4
quantize + GEMM step the overhead is measured against.  Every buffer is allocated once, so a
step can be replayed from a HIP graph.
"""
from __future__ import annotations

import torch

from . import averis as av


class LinearStep:
    def __init__(self, x, d, w, fmt, split=True, hadamard=False, out_dtype=torch.bfloat16):
        l, m = x.shape
        n = d.shape[1]
        assert w.shape == (m, n) and d.shape[0] == l
        dev = x.device
        self.x, self.d, self.w = x, d, w
        self.fmt, self.split, self.hadamard, self.l = fmt, split, hadamard, l
        self.sx = av.split_quant_outputs(l, m, fmt, split, hadamard, device=dev)
        self.sd = av.split_quant_outputs(l, n, fmt, split, hadamard, device=dev)
        self.sw = av.split_quant_outputs(m, n, fmt, False, hadamard, device=dev)
        self.ws_x = av.split_quant_workspace(l, m, fmt, split, hadamard, dev)
        self.ws_d = av.split_quant_workspace(l, n, fmt, split, hadamard, dev)
        self.ws_w = av.split_quant_workspace(m, n, fmt, False, hadamard, dev)
        self.y = torch.empty((l, n), dtype=out_dtype, device=dev)
        self.dx = torch.empty((l, m), dtype=out_dtype, device=dev)
        self.dw = torch.empty((m, n), dtype=torch.float32, device=dev)
        self.ws_fwd = av.linear_workspace(self.sx["row"], self.sw["col"])
        self.ws_dx = av.linear_workspace(self.sd["row"], self.sw["row"])
        self.ws_dw = av.linear_bwd_dw_workspace(self.sx["col"], self.sd["col"], l)

    @property
    def flops(self):
        """GEMM flops of fwd + dX + dW (the mean terms are not counted)."""
        l, m = self.x.shape
        return 6 * l * m * self.d.shape[1]

    def quantize(self, stream=None):
        av.split_quant(self.x, self.fmt, self.split, self.hadamard, stream=stream, out=self.sx, ws=self.ws_x)
        av.split_quant(self.d, self.fmt, self.split, self.hadamard, stream=stream, out=self.sd, ws=self.ws_d)
        av.split_quant(self.w, self.fmt, False, self.hadamard, stream=stream, out=self.sw, ws=self.ws_w)

    def gemms(self, stream=None):
        av.linear_fwd(self.sx["row"], self.sx["mean_q"], self.sw["col"], stream=stream, out=self.y, ws=self.ws_fwd)
        av.linear_bwd_dx(self.sd["row"], self.sd["mean_q"], self.sw["row"], stream=stream, out=self.dx,
                         ws=self.ws_dx)
        av.linear_bwd_dw(self.sx["col"], self.sd["col"], self.sx["mean_q"], self.sd["mean_q"], self.l,
                         dw=self.dw, stream=stream, ws=self.ws_dw)

    def run(self, stream=None):
        self.quantize(stream)
        self.gemms(stream)
