"""A short synthetic training run through the autograd linear: BF16 vs vanilla FP4 vs Averis.

A two-layer feed-forward block y = relu2(x W1) W2 (W1 [m, h], W2 [h, m]) is fitted by Adam to a
fixed random teacher of the same shape, on mean-biased inputs drawn like the activations of the
up_proj workload (a coherent rank-one mean with 3x the residual RMS and spike channels, Student-t
residuals).  The explainer (section 实验结果) reports that removing the mean before FP4
quantization narrows the gap to BF16 training; this run shows the same effect qualitatively on
synthetic data: no dataset and no pretrained weights are involved, so it claims no parity with the
pages' loss numbers.

    python -m fp4_quantized_amd.train_demo [steps]
"""
from __future__ import annotations

import sys

import torch

from . import averis as av
from . import workloads
from .autograd import averis_linear


def teacher_and_data(m=1024, h=3072, tokens=4096, batches=8, seed=5, device="cuda"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w1 = torch.randn(m, h, generator=g, device=device) * m ** -0.5
    w2 = torch.randn(h, m, generator=g, device=device) * h ** -0.5
    xs = [workloads.activations_device(seed * 100 + b, tokens, m, device) for b in range(batches)]
    with torch.no_grad():
        ys = [torch.relu(x.float() @ w1).square() @ w2 for x in xs]
    return xs, ys


def run(xs, ys, mode, fmt=av.MXFP4, steps=200, h=3072, lr=2e-3, seed=9):
    """mode: 'bf16' (torch matmuls), 'vanilla' (FP4, no split) or 'averis'.  Returns the losses."""
    dev = xs[0].device
    m = xs[0].shape[1]
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    w1 = (torch.randn(m, h, generator=g, device=dev) * m ** -0.5).requires_grad_(True)
    w2 = (torch.randn(h, m, generator=g, device=dev) * h ** -0.5).requires_grad_(True)
    opt = torch.optim.Adam([w1, w2], lr=lr)
    losses = []
    for it in range(steps):
        x, y = xs[it % len(xs)], ys[it % len(ys)]
        if mode == "bf16":
            a = torch.relu(x @ w1.to(torch.bfloat16)).square()
            out = a @ w2.to(torch.bfloat16)
        else:
            split = mode == "averis"
            a = torch.relu(averis_linear(x, w1.to(torch.bfloat16), fmt, split)).square()
            out = averis_linear(a, w2.to(torch.bfloat16), fmt, split)
        loss = (out.float() - y).square().mean() / y.square().mean()
        opt.zero_grad(set_to_none=True)
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    return losses


def main(steps=200):
    torch.manual_seed(0)
    xs, ys = teacher_and_data()
    rows = []
    for name, mode, fmt in (("bf16", "bf16", av.MXFP4), ("MXFP4 vanilla", "vanilla", av.MXFP4),
                            ("MXFP4 Averis", "averis", av.MXFP4), ("NVFP4 vanilla", "vanilla", av.NVFP4),
                            ("NVFP4 Averis", "averis", av.NVFP4)):
        ls = run(xs, ys, mode, fmt, steps)
        tail = sum(ls[-20:]) / 20
        rows.append((name, ls[0], tail))
        print(f"{name:14s} relative loss: first {ls[0]:.4f}, mean of the last 20 steps {tail:.4f}", flush=True)
    return rows


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 200)
