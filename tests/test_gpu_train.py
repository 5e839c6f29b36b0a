"""Short synthetic training through the autograd linear (GPU): BF16, vanilla FP4 and Averis all
learn (finite losses that fall).  Their ordering on this toy problem is reported by the demo,
not asserted: a few hundred steps on synthetic data resolve no stable gap."""
import math

import pytest

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import train_demo

pytestmark = pytest.mark.gpu


def test_training_runs_for_every_variant():
    print("case train_demo 60 steps", flush=True)
    xs, ys = train_demo.teacher_and_data(tokens=2048, batches=4)
    res = {mode: train_demo.run(xs, ys, mode, av.MXFP4, steps=60) for mode in ("bf16", "vanilla", "averis")}
    for mode, ls in res.items():
        assert all(math.isfinite(v) for v in ls), mode
        assert sum(ls[-10:]) / 10 < 0.7 * ls[0], f"{mode} did not learn: {ls[0]:.3f} -> {ls[-1]:.3f}"


def test_transformer_training_runs_for_every_variant():
    # a 2-block decoder-only transformer (d 512, 8 heads, SwiGLU 1536) whose q, k, v, o, gate, up
    # and down linears are FP4 autograd linears, trained on a synthetic Markov-chain language
    from fp4_quantized_amd import transformer_demo
    print("case transformer_demo 40 steps", flush=True)
    for mode, fmt in (("bf16", av.MXFP4), ("vanilla", av.MXFP4), ("averis", av.MXFP4), ("averis", av.NVFP4)):
        ls, ev, h = transformer_demo.run(mode, fmt, steps=40, pool=16)
        assert all(math.isfinite(v) for v in ls + [ev]), mode
        assert sum(ls[-5:]) / 5 < ls[0] - 1.5, f"{mode}/{fmt} did not learn: {ls[0]:.3f} -> {ls[-1]:.3f}"
