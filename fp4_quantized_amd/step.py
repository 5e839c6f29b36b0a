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


class MoEStep:
    """One MoE feed-forward layer's quantized training step over expert-contiguous routed rows,
    every kernel a grouped launch over all experts: gate and up (hidden -> ffn, sharing X's
    split) and down (ffn -> hidden), each forward, input gradient and weight gradient.

    x [L, h] routed token states, x_down [L, f] the down projection's input, d_gu [L, f] the
    output gradient used for both gate and up, d_dn [L, h]; w_gate and w_up [E * h, f] (E stacked
    [h, f]), w_down [E * f, h]; offsets [E + 1] over the L rows (host array)."""

    def __init__(self, x, x_down, d_gu, d_dn, w_gate, w_up, w_down, offsets, fmt, split=True,
                 out_dtype=torch.bfloat16):
        import numpy as np
        dev = x.device
        self.fmt, self.split = fmt, split
        E = len(offsets) - 1
        L, h = x.shape
        f = x_down.shape[1]
        self.E, self.h, self.f = E, h, f
        self.grp = av.Groups(offsets, dev)
        wgrp_h = av.Groups(np.arange(E + 1) * h, dev)
        wgrp_f = av.Groups(np.arange(E + 1) * f, dev)
        self.quants = []
        self.q = {}
        for name, t, grp, sp in (("x", x, self.grp, split), ("xd", x_down, self.grp, split),
                                 ("dgu", d_gu, self.grp, split), ("ddn", d_dn, self.grp, split),
                                 ("wg", w_gate, wgrp_h, False), ("wu", w_up, wgrp_h, False),
                                 ("wd", w_down, wgrp_f, False)):
            out = av.split_quant_grouped_outputs(grp, t.shape[1], fmt, sp, device=dev)
            ws = av.split_quant_grouped_workspace(t.shape[0], t.shape[1], grp.E, fmt, sp, device=dev)
            self.quants.append((t, grp, sp, out, ws))
            self.q[name] = out
        q = self.q
        mu = (lambda n: q[n]["mean_q"]) if split else (lambda n: None)
        self.gemms = []
        for wq, xin, din, k_in, n_out in (("wg", "x", "dgu", h, f), ("wu", "x", "dgu", h, f), ("wd", "xd", "ddn", f, h)):
            y = torch.empty((L, n_out), dtype=out_dtype, device=dev)
            dx = torch.empty((L, k_in), dtype=out_dtype, device=dev)
            dw = torch.empty((E, k_in, n_out), dtype=torch.float32, device=dev)
            w_fwd = av.stacked_weight_view(q[wq]["col"], E, k_in)
            self.gemms.append((av.linear_fwd_grouped, (q[xin]["row"], mu(xin), w_fwd, self.grp),
                               dict(out=y, ws=av.linear_grouped_workspace(n_out, E, fmt, dev))))
            self.gemms.append((av.linear_bwd_dx_grouped, (q[din]["row"], mu(din), q[wq]["row"], self.grp),
                               dict(out=dx, ws=av.linear_grouped_workspace(k_in, E, fmt, dev))))
            self.gemms.append((av.linear_bwd_dw_grouped, (q[xin]["col"], q[din]["col"], mu(xin), mu(din), self.grp),
                               dict(dw=dw, ws=av.linear_bwd_dw_grouped_workspace(k_in, n_out, E, fmt, dev))))

    @property
    def flops(self):
        """GEMM flops of the three linears' fwd + dX + dW (the mean terms are not counted)."""
        return 3 * 6 * self.grp.rows * self.h * self.f

    def run(self, stream=None):
        for t, grp, sp, out, ws in self.quants:
            av.split_quant_grouped(t, grp, self.fmt, sp, stream=stream, out=out, ws=ws)
        for fn, args, kw in self.gemms:
            fn(*args, stream=stream, **kw)
