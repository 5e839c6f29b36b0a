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


def _column_blocks(ts):
    """The tensor [r, N] whose adjacent column blocks, in order, are the 2-D tensors ts, or None."""
    t0 = ts[0]
    r, N = t0.shape[0], sum(t.shape[1] for t in ts)
    off = 0
    for t in ts:
        if (t.dim() != 2 or r == 0 or t.shape[0] != r or t.dtype != t0.dtype or t.device != t0.device
                or t.untyped_storage().data_ptr() != t0.untyped_storage().data_ptr()
                or t.stride() != (N, 1) or t.storage_offset() != t0.storage_offset() + off):
            return None
        off += t.shape[1]
    return t0.as_strided((r, N), (N, 1))


def _rows(q, off, n):
    """Rows [off, off + n) of a quantized operand (off a multiple of 32): a view."""
    return av.QTensor(q.codes[off:off + n], q.scales[off:off + n], None, n, q.k, q.fmt, q.rotated)


def _k_block(q, off, n):
    """Elements [off, off + n) of a one-row quantized operand (off, n multiples of 256): a view
    (the tiled scales of one 256-element K-step of a 32-row group are contiguous)."""
    g = av.BLOCK[q.fmt]
    piece = 32 * (256 // g)
    sc = q.scales.view(-1)[(off // 256) * piece:((off + n) // 256) * piece].view(32, n // g)
    return av.QTensor(q.codes[:, off // 2:(off + n) // 2], sc, None, 1, n, q.fmt, q.rotated)


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
        """The step in training order: the weight, then the forward (split X, Y), then the
        backward (split D, dX, dW)."""
        sx, sd, sw = self.sx, self.sd, self.sw
        av.split_quant(self.w, self.fmt, False, self.hadamard, stream=stream, out=sw, ws=self.ws_w)
        av.split_quant(self.x, self.fmt, self.split, self.hadamard, stream=stream, out=sx, ws=self.ws_x)
        av.linear_fwd(sx["row"], sx["mean_q"], sw["col"], stream=stream, out=self.y, ws=self.ws_fwd)
        av.split_quant(self.d, self.fmt, self.split, self.hadamard, stream=stream, out=sd, ws=self.ws_d)
        av.linear_bwd_dx(sd["row"], sd["mean_q"], sw["row"], stream=stream, out=self.dx, ws=self.ws_dx)
        av.linear_bwd_dw(sx["col"], sd["col"], sx["mean_q"], sd["mean_q"], self.l, dw=self.dw, stream=stream,
                         ws=self.ws_dw)


class LayerStep:
    """One layer's quantized training step over several linears whose inputs may be shared:
    every distinct input tensor X is split and quantized once (q, k and v read one X; gate and
    up read one X), every output gradient D and weight W once per linear, then each linear's
    forward, input-gradient and weight-gradient GEMMs.  linears: [(name, x, d, w)].

    batched: tensors that become ready together are split and quantized in one batched launch
    pair (averis_split_quant_batch): every weight at the start of the step, and the output
    gradients of the linears that share an input (q/k/v: attention's backward returns them at
    once; gate/up: the SwiGLU backward).

    run() keeps a training step's order: the weights; the forward, input by input (split X, the
    forward GEMMs of the linears reading it); the backward in reverse (split the output
    gradients of those linears, their dX and dW GEMMs).

    overlap: nothing on the step's critical path waits for the weight quantization until the
    first forward GEMM, or for a weight gradient at all (the next layer down needs dX, not dW).
    With overlap the weights are quantized and every dW GEMM runs on a second stream (default
    priority) that forks from the caller's stream at the start of run() and joins it at the
    end; each dW waits only for its output gradient's split.  The two streams' kernels then
    fill each other's ramp and tail.  Every result is the same as without overlap.

    fuse_fwd / fuse_dw (MXFP4): linears that share an input run one forward GEMM (q/k/v,
    gate/up) and, where it fills the GPU in one round of tiles, one weight-gradient GEMM (q/k/v),
    whose output column blocks are the linears' Y_i and dW_i (see _fuse_fwd, _fuse_dw); the
    per-linear "y" and "dw" are then views of those outputs.

    fuse_dx (MXFP4): where the output gradients and the weights of the linears sharing an input
    are adjacent column blocks of one tensor each (as a fused q/k/v or gate/up projection stores
    them), those two tensors are split and quantized once each and the linears run one
    input-gradient GEMM, whose output is the input's gradient, the sum over the linears (see
    _concat); every such linear's "dx" is that one tensor.  Otherwise each linear has its own
    dX (the sum is left to the caller)."""

    def __init__(self, linears, fmt, split=True, hadamard=False, out_dtype=torch.bfloat16, batched=True,
                 overlap=True, fuse_dw=True, fuse_fwd=True, fuse_dx=True):
        self.fmt, self.split, self.hadamard = fmt, split, hadamard
        self.side = torch.cuda.Stream(device=linears[0][1].device) if overlap else None
        self.quants = []  # (tensor, split, outputs, workspace)
        self.lin = []
        self.dw_fused = {}  # x_plan index -> the fused weight gradient of its linears
        self.fwd_fused = {}  # x_plan index -> the fused forward GEMM of its linears
        self.dx_fused = {}  # x_plan index -> the one input-gradient GEMM of its linears
        by_x = {}  # linears grouped by their input (callers list each group's linears together)
        for item in linears:
            by_x.setdefault(id(item[1]), []).append(item)
        chunks = lambda ix: [ix[i:i + av.BATCH_MAX] for i in range(0, len(ix), av.BATCH_MAX)]  # noqa: E731
        one = lambda ix: [[i] for i in ix]  # noqa: E731
        w_idx = []  # indices into quants of the weights
        self.x_plan = []  # (X group, D groups, indices into lin), one per distinct X
        for pi, items in enumerate(by_x.values()):
            x = items[0][1]
            l, m = x.shape
            xi, sx = self._add(x, split, l, m)
            li0 = len(self.lin)
            parents = None
            if fuse_dx and len(items) >= 2 and fmt == av.MXFP4 and all(it[2].shape[1] % 256 == 0 for it in items):
                dp, wp = _column_blocks([it[2] for it in items]), _column_blocks([it[3] for it in items])
                if dp is not None and wp is not None:
                    parents = (dp, wp)
            if parents is not None:
                d_idx = [self._concat(pi, items, sx, parents, out_dtype, fuse_fwd, fuse_dw, w_idx)]
            else:
                d_idx = []
                for name, _, d, w in items:
                    n = d.shape[1]
                    di, sd = self._add(d, split, l, n)
                    wi, sw = self._add(w, False, m, n)
                    d_idx.append(di)
                    w_idx.append(wi)
                    dev = x.device
                    self.lin.append(dict(name=name, l=l, m=m, n=n, sx=sx, sd=sd, sw=sw,
                                         y=torch.empty((l, n), dtype=out_dtype, device=dev),
                                         dx=torch.empty((l, m), dtype=out_dtype, device=dev),
                                         dw=torch.empty((m, n), dtype=torch.float32, device=dev),
                                         ws_fwd=av.linear_workspace(sx["row"], sw["col"]),
                                         ws_dx=av.linear_workspace(sd["row"], sw["row"]),
                                         ws_dw=av.linear_bwd_dw_workspace(sx["col"], sd["col"], l)))
                if fuse_dw:
                    self._fuse_dw(pi, self.lin[li0:])
                if fuse_fwd:
                    self._fuse_fwd(pi, self.lin[li0:])
            self.x_plan.append(([xi], chunks(d_idx) if batched else one(d_idx), list(range(li0, len(self.lin)))))
        # launch groups: the weights, then per distinct X its split and its D's
        self.w_groups = chunks(w_idx) if batched else one(w_idx)
        self.groups = list(self.w_groups)
        for xg, dgs, _ in self.x_plan:
            self.groups += [xg] + dgs

    def _add(self, t, sp, rows, cols):
        """A split (+ quantization) of t [rows, cols] with its outputs and workspace."""
        dev = t.device
        out = av.split_quant_outputs(rows, cols, self.fmt, sp, self.hadamard, device=dev)
        self.quants.append((t, sp, out, av.split_quant_workspace(rows, cols, self.fmt, sp, self.hadamard, dev)))
        return len(self.quants) - 1, out

    def _concat(self, pi, items, sx, parents, out_dtype, fuse_fwd, fuse_dw, w_idx):
        """Linears that share their input X and whose output gradients D_i and weights W_i are
        adjacent column blocks of one tensor each, D = [D_1 .. D_k] [l, N] and W = [W_1 .. W_k]
        [m, N] (a fused projection's storage), are one linear of width N for the split: the column
        means are per column and MXFP4 blocks never straddle a block boundary (widths multiples of
        256), so D and W are split and quantized once and every D_i, W_i operand that the
        per-linear GEMMs read (the K = tokens layout of D_i, its quantized mean, the K = m layout
        of W_i) is a view of D's or W's.  The input gradient of X is the sum over the linears,
        sum_i 1 (mu_Di W_i^T) + D_R,i W_i^T = 1 (mu_D W^T) + D_R W^T ([rainbus] 方法步骤详情,
        input gradient, over D and W): one GEMM with K = N, which the per-linear launches would
        leave to a separate sum.  Forward: one GEMM (as _fuse_fwd); weight gradient: one GEMM
        where it fills the GPU in one round of 128 x 128 tiles (as _fuse_dw), else one per
        linear on the views.  Returns the index of D's split."""
        dp, wp = parents
        split = self.split
        l, m, N = dp.shape[0], wp.shape[0], dp.shape[1]
        dev = dp.device
        di, sdc = self._add(dp, split, l, N)
        wi, swc = self._add(wp, False, m, N)
        w_idx.append(wi)
        y = torch.empty((l, N), dtype=out_dtype, device=dev)
        dx = torch.empty((l, m), dtype=out_dtype, device=dev)
        one_dw = fuse_dw and -(-m // 128) * -(-N // 128) <= 256
        dw = torch.empty((m, N), dtype=torch.float32, device=dev) if one_dw else None
        off = 0
        for name, _, d, w in items:
            n = d.shape[1]
            sd = dict(mean=sdc["mean"][off:off + n] if split else None, row=None, col=_rows(sdc["col"], off, n),
                      mean_q=_k_block(sdc["mean_q"], off, n) if split else None)
            sw = dict(mean=None, row=None, col=_rows(swc["col"], off, n), mean_q=None)
            self.lin.append(dict(name=name, l=l, m=m, n=n, sx=sx, sd=sd, sw=sw, y=y[:, off:off + n], dx=dx,
                                 dw=dw[:, off:off + n] if one_dw else torch.empty((m, n), dtype=torch.float32,
                                                                                   device=dev),
                                 ws_fwd=av.linear_workspace(sx["row"], sw["col"]),
                                 ws_dw=av.linear_bwd_dw_workspace(sx["col"], sd["col"], l)))
            off += n
        if fuse_fwd:
            self.fwd_fused[pi] = dict(w=swc["col"], y=y, sx=sx, ws=av.linear_workspace(sx["row"], swc["col"]))
        self.dx_fused[pi] = dict(d=sdc, w=swc, dx=dx, ws=av.linear_workspace(sdc["row"], swc["row"]))
        if one_dw:
            self.dw_fused[pi] = dict(col=sdc["col"], mean_q=sdc["mean_q"], dw=dw, l=l, sx=sx,
                                     ws=av.linear_bwd_dw_workspace(sx["col"], sdc["col"], l))
        return di

    def _fuse_fwd(self, pi, cs):
        """Linears that share their input X have forward outputs 1 (mu_X W_i) + X_R W_i that are
        the column blocks of X_R [W_1 .. W_k] plus the mean row ([rainbus] 方法步骤详情, forward):
        the weights' K = m layouts are written as adjacent row blocks of one operand and the Y_i
        are column blocks of one output, so one launch replaces one per linear.  MXFP4 (no
        tensor scale per W_i to keep apart); every Y_i is bit-identical to its own launch's."""
        if len(cs) < 2 or self.fmt != av.MXFP4 or any(c["n"] % 32 for c in cs):
            return
        l, m = cs[0]["l"], cs[0]["m"]
        N = sum(c["n"] for c in cs)
        dev = cs[0]["y"].device
        wcol = av.empty_qtensor(N, m, self.fmt, self.hadamard, dev)
        y = torch.empty((l, N), dtype=cs[0]["y"].dtype, device=dev)
        off = 0
        for c in cs:
            n, sw = c["n"], c["sw"]  # sw is the dict the weight quantization writes
            sw["col"] = _rows(wcol, off, n)
            c["y"] = y[:, off:off + n]
            off += n
        self.fwd_fused[pi] = dict(w=wcol, y=y, sx=cs[0]["sx"], ws=av.linear_workspace(cs[0]["sx"]["row"], wcol))

    def _fwds(self, pi, lins, stream):
        """The forward GEMMs of the linears reading input pi: one fused launch or one each."""
        f = self.fwd_fused.get(pi)
        if f is None:
            for li in lins:
                self._fwd(self.lin[li], stream)
            return
        mx = f["sx"]["mean_q"] if self.split else None
        av.linear_fwd(f["sx"]["row"], mx, f["w"], stream=stream, out=f["y"], ws=f["ws"])

    def _fuse_dw(self, pi, cs):
        """Linears that share their input X have weight gradients X_R^T D_i + l mu_X^T mu_D_i that
        form the column blocks of one GEMM, X_R^T [D_1 .. D_k] + l mu_X^T [mu_D_1 .. mu_D_k]
        ([rainbus] 方法步骤详情, weight gradient, applied to each D_i): the D_i's K = tokens layouts
        and quantized means are written as adjacent row blocks of one operand and the dW_i as
        column blocks of one output, so one launch replaces one per linear (and their split-K
        reductions).  MXFP4 (no tensor scale per D_i to keep apart), D_i widths that are
        multiples of 256, and only when the fused GEMM fills the GPU with one round of
        128 x 128 tiles (q/k/v: 8 x 32 = 256 tiles): every quantized operand is the same as
        without fusion, dW the same up to fp32 summation order."""
        if len(cs) < 2 or self.fmt != av.MXFP4 or any(c["n"] % 256 for c in cs):
            return
        l, m = cs[0]["l"], cs[0]["m"]
        N = sum(c["n"] for c in cs)
        if -(-m // 128) * -(-N // 128) > 256:
            return
        dev = cs[0]["dw"].device
        fmt, h16 = self.fmt, self.hadamard
        col = av.empty_qtensor(N, l, fmt, h16, dev)
        mq = av.empty_qtensor(1, N, fmt, h16, dev) if self.split else None
        dw = torch.empty((m, N), dtype=torch.float32, device=dev)
        off = 0
        for c in cs:
            n, sd = c["n"], c["sd"]  # sd is the dict the D split writes (shared with self.quants)
            sd["col"] = _rows(col, off, n)
            if self.split:
                sd["mean_q"] = _k_block(mq, off, n)
            c["dw"] = dw[:, off:off + n]
            off += n
        self.dw_fused[pi] = dict(col=col, mean_q=mq, dw=dw, l=l, sx=cs[0]["sx"],
                                 ws=av.linear_bwd_dw_workspace(cs[0]["sx"]["col"], col, l))

    def _dws(self, pi, lins, stream):
        """The weight gradients of the linears reading input pi: one fused launch or one each."""
        f = self.dw_fused.get(pi)
        if f is None:
            for li in lins:
                self._dw(self.lin[li], stream)
            return
        mx = f["sx"]["mean_q"] if self.split else None
        av.linear_bwd_dw(f["sx"]["col"], f["col"], mx, f["mean_q"], f["l"], dw=f["dw"], stream=stream, ws=f["ws"])

    @property
    def flops(self):
        """GEMM flops of every linear's fwd + dX + dW (the mean terms are not counted)."""
        return sum(6 * c["l"] * c["m"] * c["n"] for c in self.lin)

    def quant_bytes(self, in_bytes=2):
        """Algorithmic bytes of the split+quant launches: each input read once, both packed
        layouts written (codes and block scales), the mean vector and its quantized copy."""
        g = av.BLOCK[self.fmt]
        tot = 0.0
        for t, sp, _, _ in self.quants:
            r, c = t.shape
            tot += r * c * (in_bytes + 2 * (0.5 + 1.0 / g)) + (c * (4 + 0.5 + 1.0 / g) if sp else 0.0)
        return tot

    def _split(self, grp, stream):
        qs = [self.quants[i] for i in grp]
        if len(qs) == 1:
            t, sp, out, ws = qs[0]
            av.split_quant(t, self.fmt, sp, self.hadamard, stream=stream, out=out, ws=ws)
        else:
            av.split_quant_batch([q[0] for q in qs], self.fmt, qs[0][1], self.hadamard,
                                 outs=[q[2] for q in qs], wss=[q[3] for q in qs], stream=stream)

    def _fwd(self, c, stream):
        mx = c["sx"]["mean_q"] if self.split else None
        av.linear_fwd(c["sx"]["row"], mx, c["sw"]["col"], stream=stream, out=c["y"], ws=c["ws_fwd"])

    def _dx(self, c, stream):
        md = c["sd"]["mean_q"] if self.split else None
        av.linear_bwd_dx(c["sd"]["row"], md, c["sw"]["row"], stream=stream, out=c["dx"], ws=c["ws_dx"])

    def _dxs(self, pi, lins, stream):
        """The input gradients of the linears reading input pi: their one summed launch or one each."""
        f = self.dx_fused.get(pi)
        if f is None:
            for li in lins:
                self._dx(self.lin[li], stream)
            return
        md = f["d"]["mean_q"] if self.split else None
        av.linear_bwd_dx(f["d"]["row"], md, f["w"]["row"], stream=stream, out=f["dx"], ws=f["ws"])

    def _dw(self, c, stream):
        mx = c["sx"]["mean_q"] if self.split else None
        md = c["sd"]["mean_q"] if self.split else None
        av.linear_bwd_dw(c["sx"]["col"], c["sd"]["col"], mx, md, c["l"], dw=c["dw"], stream=stream, ws=c["ws_dw"])

    def quantize(self, stream=None):
        """Every split + quantization of the step, alone."""
        for grp in self.groups:
            self._split(grp, stream)

    def gemms(self, stream=None):
        """Every GEMM of the step, alone (on operands quantize() wrote)."""
        for pi, (_, _, lins) in enumerate(self.x_plan):
            self._fwds(pi, lins, stream)
            self._dxs(pi, lins, stream)
            self._dws(pi, lins, stream)

    def run(self, stream=None):
        if self.side is None:
            for grp in self.w_groups:
                self._split(grp, stream)
            for pi, (xg, _, lins) in enumerate(self.x_plan):
                self._split(xg, stream)
                self._fwds(pi, lins, stream)
            for pi in reversed(range(len(self.x_plan))):
                _, dgs, lins = self.x_plan[pi]
                for grp in dgs:
                    self._split(grp, stream)
                self._dxs(pi, lins, stream)
                self._dws(pi, lins, stream)
            return
        main = stream if stream is not None else torch.cuda.current_stream()
        side = self.side
        side.wait_stream(main)  # fork
        for grp in self.w_groups:
            self._split(grp, side)
        weights = torch.cuda.Event()
        weights.record(side)
        for k, (xg, _, lins) in enumerate(self.x_plan):
            self._split(xg, main)
            if k == 0:
                main.wait_event(weights)
            self._fwds(k, lins, main)
        for pi in reversed(range(len(self.x_plan))):
            _, dgs, lins = self.x_plan[pi]
            for grp in dgs:
                self._split(grp, main)
            grads = torch.cuda.Event()
            grads.record(main)
            side.wait_event(grads)
            self._dxs(pi, lins, main)
            self._dws(pi, lins, side)
        main.wait_stream(side)  # join


class MoEStep:
    """One MoE feed-forward layer's quantized training step over expert-contiguous routed rows,
    every kernel a grouped launch over all experts: gate and up (hidden -> ffn, sharing X's
    split) and down (ffn -> hidden), each forward, input gradient and weight gradient.

    x [L, h] routed token states, x_down [L, f] the down projection's input, d_gate and d_up
    [L, f] the output gradients of gate and up, d_dn [L, h]; w_gate and w_up [E * h, f] (E stacked
    [h, f]), w_down [E * f, h]; offsets [E + 1] over the L rows (host array).

    fuse_gate_up: gate and up as one projection hidden -> 2 ffn, the layout of a gated MLP whose
    two input projections share their input: per expert W = [W_gate | W_up] [h, 2f] and
    D = [D_gate | D_up] [L, 2f].  One forward GEMM writes [Y_gate | Y_up], one weight-gradient
    GEMM [dW_gate | dW_up], and one input-gradient GEMM (K = 2f) writes the input gradient of
    X, D_gate W_gate^T + D_up W_up^T, which the separate projections leave as two terms.  The
    column means, residuals and blocks of the concatenated tensors are those of the parts (the
    blocks never straddle the boundary, f % 32 == 0), so with MXFP4 every quantized operand,
    Y and dW equal the separate projections' bit for bit; NVFP4 has one tensor scale per
    concatenated tensor (per expert for the weights) instead of one per part."""

    def __init__(self, x, x_down, d_gate, d_up, d_dn, w_gate, w_up, w_down, offsets, fmt, split=True,
                 out_dtype=torch.bfloat16, overlap=True, fuse_gate_up=False):
        import numpy as np
        dev = x.device
        self.fmt, self.split, self.fused = fmt, split, fuse_gate_up
        self.side = torch.cuda.Stream(device=dev) if overlap else None  # as in LayerStep
        E = len(offsets) - 1
        L, h = x.shape
        f = x_down.shape[1]
        self.E, self.h, self.f = E, h, f
        self.grp = av.Groups(offsets, dev)
        wgrp_h = av.Groups(np.arange(E + 1) * h, dev)
        wgrp_f = av.Groups(np.arange(E + 1) * f, dev)
        if fuse_gate_up:
            assert f % 32 == 0
            # (w, x, d, rows of one expert's weight, output columns) per projection
            projs = [("wgu", "x", "dgu", h, 2 * f), ("wd", "xd", "ddn", f, h)]
            tensors = (("x", x, self.grp, split), ("xd", x_down, self.grp, split),
                       ("dgu", torch.cat([d_gate, d_up], dim=1), self.grp, split), ("ddn", d_dn, self.grp, split),
                       ("wgu", torch.cat([w_gate, w_up], dim=1), wgrp_h, False), ("wd", w_down, wgrp_f, False))
        else:
            projs = [("wg", "x", "dg", h, f), ("wu", "x", "du", h, f), ("wd", "xd", "ddn", f, h)]
            tensors = (("x", x, self.grp, split), ("xd", x_down, self.grp, split),
                       ("dg", d_gate, self.grp, split), ("du", d_up, self.grp, split),
                       ("ddn", d_dn, self.grp, split),
                       ("wg", w_gate, wgrp_h, False), ("wu", w_up, wgrp_h, False),
                       ("wd", w_down, wgrp_f, False))
        self.projs = projs
        self.quants = []
        self.q = {}
        self.qi = {}
        for name, t, grp, sp in tensors:
            out = av.split_quant_grouped_outputs(grp, t.shape[1], fmt, sp, device=dev)
            ws = av.split_quant_grouped_workspace(t.shape[0], t.shape[1], grp.E, fmt, sp, device=dev)
            self.qi[name] = len(self.quants)
            self.quants.append((t, grp, sp, out, ws))
            self.q[name] = out
        q = self.q
        mu = (lambda n: q[n]["mean_q"]) if split else (lambda n: None)
        self.gemms = []  # per projection p: 3 p forward, 3 p + 1 input gradient, 3 p + 2 weight gradient
        for wq, xin, din, k_in, n_out in projs:
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
        """The step in training order: the weights; the forward (split X, gate and up; split the
        down input, down); the backward (split down's output gradient, its dX and dW; split the
        gate and up gradients, their dX and dW).  With overlap the weights and the dW GEMMs run on
        the second stream, as in LayerStep.run; the gate and up forward wait only for their own
        weights, the down forward for the down weight."""
        main = stream if stream is not None else torch.cuda.current_stream()
        side = self.side if self.side is not None else main
        gu = list(range(len(self.projs) - 1))  # the gate / up projections; the last one is down
        dn = len(self.projs) - 1

        def split(name, s):
            t, grp, sp, out, ws = self.quants[self.qi[name]]
            av.split_quant_grouped(t, grp, self.fmt, sp, stream=s, out=out, ws=ws)

        def gemm(i, s):
            fn, args, kw = self.gemms[i]
            fn(*args, stream=s, **kw)

        def hand_over(src, dst):  # dst waits for what src has enqueued so far
            if src is not dst:
                e = torch.cuda.Event()
                e.record(src)
                dst.wait_event(e)

        hand_over(main, side)  # fork
        for p in gu:
            split(self.projs[p][0], side)
        gate_up_w = torch.cuda.Event()
        gate_up_w.record(side)
        split(self.projs[dn][0], side)  # needed from the down forward on
        split("x", main)
        main.wait_event(gate_up_w)
        for p in gu:
            gemm(3 * p, main)  # gate and up forward
        split("xd", main)
        hand_over(side, main)  # the down weight
        gemm(3 * dn, main)  # down forward
        split("ddn", main)
        hand_over(main, side)
        gemm(3 * dn + 1, main)  # down dX
        gemm(3 * dn + 2, side)  # down dW
        for p in gu:
            split(self.projs[p][2], main)  # the gate and up output gradients
        hand_over(main, side)
        for p in gu:
            gemm(3 * p + 1, main)  # gate and up dX
        for p in gu:
            gemm(3 * p + 2, side)  # gate and up dW
        hand_over(side, main)  # join
