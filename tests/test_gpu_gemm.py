"""GPU parity of the three quantized GEMMs (forward, input gradient, weight gradient) against
the CPU oracle's exact (fp64) products of the dequantized operands.

The GPU quantizes every operand; the same bytes are handed to the oracle (whose own
quantization of the same inputs is checked bit-exact in test_gpu_quant.py), and fp32 outputs
must be within 1e-5 relative Frobenius error.  bf16 outputs are checked at bf16's own
rounding (2^-8 relative per element).
"""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from oracle import averis_oracle as O
from tests.gpu_util import device, rel_fro, to_oracle

pytestmark = pytest.mark.gpu

FMTS = [(av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")]
TOL = 1e-5


def quantize_layer(lin, fmt, hadamard, dev, split=True):
    dt = lin.dtype
    x = workloads.to_torch(lin.x, dt, dev)
    d = workloads.to_torch(lin.d, dt, dev)
    w = workloads.to_torch(lin.w, dt, dev)
    sx = av.split_quant(x, fmt, split=split, hadamard=hadamard)
    sd = av.split_quant(d, fmt, split=split, hadamard=hadamard)
    sw = av.split_quant(w, fmt, split=False, hadamard=hadamard)
    return sx, sd, sw


def check_layer(lin, fmt, hadamard, tag, split=True, out_dtype=torch.float32):
    dev = device()
    print(f"case {tag} l={lin.x.shape[0]} m={lin.x.shape[1]} n={lin.d.shape[1]} fmt={fmt} h16={hadamard} "
          f"split={split} out={out_dtype}", flush=True)
    l = lin.x.shape[0]
    sx, sd, sw = quantize_layer(lin, fmt, hadamard, dev, split)
    mx = sx["mean_q"] if split else None
    md = sd["mean_q"] if split else None
    y = av.linear_fwd(sx["row"], mx, sw["col"], out_dtype)
    dx = av.linear_bwd_dx(sd["row"], md, sw["row"], out_dtype)
    dw = av.linear_bwd_dw(sx["col"], sd["col"], mx, md, l)
    torch.cuda.synchronize()
    omx = to_oracle(mx) if split else None
    omd = to_oracle(md) if split else None
    y_ref = O.linear_fwd(to_oracle(sx["row"]), omx, to_oracle(sw["col"]))
    dx_ref = O.linear_bwd_dx(to_oracle(sd["row"]), omd, to_oracle(sw["row"]))
    dw_ref = O.linear_bwd_dw(to_oracle(sx["col"]), to_oracle(sd["col"]), omx, omd, l)
    outs = [("Y", y, y_ref), ("dX", dx, dx_ref), ("dW", dw, dw_ref)]
    for name, got, ref in outs:
        g = got.float().cpu().numpy()
        assert g.shape == ref.shape, (tag, name)
        if got.dtype == torch.bfloat16:
            bad = np.abs(g - ref) > 2.0 ** -8 * np.abs(ref) + 1e-30 + 1e-5 * np.abs(ref).max()
            assert not bad.any(), f"{tag} {name}: {bad.sum()} bf16 outputs off"
        else:
            err = rel_fro(g, ref)
            assert err <= TOL, f"{tag} {name}: relative Frobenius error {err:.3e}"
    return y, dx, dw


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_tiny_forward(fmt, fname):
    dev = device()
    lin = workloads.tiny(0)
    x = workloads.to_torch(lin.x, "f32", dev)
    w = workloads.to_torch(lin.w, "f32", dev)
    sx = av.split_quant(x, fmt)
    sw = av.split_quant(w, fmt, split=False)
    y = av.linear_fwd(sx["row"], sx["mean_q"], sw["col"])
    torch.cuda.synchronize()
    ref = O.linear_fwd(to_oracle(sx["row"]), to_oracle(sx["mean_q"]), to_oracle(sw["col"]))
    assert rel_fro(y.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
@pytest.mark.parametrize("split", [True, False])
def test_small_layer(fmt, fname, hadamard, split):
    # ragged: l = 1000 tokens (not a tile multiple), m = 256, n = 384 (not a 128-tile multiple of 256)
    lin = workloads.up_proj_like(21, 1000, 256, 384)
    check_layer(lin, fmt, hadamard, f"small-{fname}-h{int(hadamard)}-s{int(split)}", split)


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("l", [1, 17, 130])
def test_few_tokens(fmt, fname, l):
    lin = workloads.up_proj_like(22, l, 128, 256)
    check_layer(lin, fmt, False, f"few-{fname}-{l}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_bf16_outputs(fmt, fname):
    lin = workloads.up_proj_like(23, 512, 256, 384)
    check_layer(lin, fmt, False, f"bf16-{fname}", out_dtype=torch.bfloat16)


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_up_proj_full_size(fmt, fname):
    # l = 8192, m = 1024, n = 3072: full outputs of Y, dX and dW against the oracle
    check_layer(workloads.up_proj(), fmt, False, f"up_proj-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_ragged_tokens_256x128_tiles(fmt, fname):
    # l = 8300 tokens: MXFP4's forward and input-gradient GEMMs run on 256 x 128 tiles (33 x 24 and
    # 33 x 8 of them) with a ragged last row of tiles; full outputs against the oracle
    check_layer(workloads.up_proj_like(26, 8300, 1024, 3072), fmt, False, f"ragged-256-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_long_k_ragged_128x96_tiles(fmt, fname):
    # the weight gradient of m = 1024 by n = 3072 over l = 4100 tokens (K padded to 17 K-steps,
    # ragged): on 256 CUs its 8 x 24 tiles of 128 x 128 leave a quarter of the CUs idle, so it
    # runs on 8 x 32 tiles of 128 x 96; rank-one term with rotated means
    lin = workloads.up_proj_like(25, 4100, 1024, 3072)
    check_layer(lin, fmt, True, f"long-k-{fname}")


def test_dw_accumulate_and_determinism():
    dev = device()
    lin = workloads.up_proj_like(24, 3000, 256, 384)
    sx, sd, _ = quantize_layer(lin, av.MXFP4, False, dev)
    base = torch.randn(256, 384, device=dev)
    dw1 = av.linear_bwd_dw(sx["col"], sd["col"], sx["mean_q"], sd["mean_q"], 3000)
    dw2 = av.linear_bwd_dw(sx["col"], sd["col"], sx["mean_q"], sd["mean_q"], 3000)
    acc = av.linear_bwd_dw(sx["col"], sd["col"], sx["mean_q"], sd["mean_q"], 3000, dw=base.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw2)
    assert torch.allclose(acc, base + dw1, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_long_k_mean_term_gemv(fmt, fname):
    # K = 8320 features: past the longest mean row the GEMM keeps in LDS (8192), so the MXFP4
    # forward takes its mean term from the GEMV launch, as NVFP4 always does
    lin = workloads.up_proj_like(61, 96, 8320, 128)
    check_layer(lin, fmt, False, f"long-k-gemv-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
def test_column_counts_multiple_of_32(fmt, fname, hadamard):
    # m = 160 and n = 96 features: K of the forward and input-gradient GEMMs ends mid K-step and
    # the row layouts' last 256-element piece is mostly padding
    lin = workloads.up_proj_like(64, 300, 160, 96)
    check_layer(lin, fmt, hadamard, f"cols-160-96-{fname}")


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_split_k_bf16_outputs(fmt, fname):
    # 256 x 256 outputs with K = 4096: few tiles, so the forward and input-gradient GEMMs split K
    # and the fixed-order reduce writes the bf16 outputs (and adds the MXFP4 split shares of the
    # mean term, the NVFP4 GEMV row)
    lin = workloads.up_proj_like(62, 256, 4096, 256)
    l, m = lin.x.shape
    n = lin.d.shape[1]
    assert lib_splits(fmt, l, n, m) > 1 and lib_splits(fmt, l, m, n) == 1
    check_layer(lin, fmt, False, f"split-k-bf16-{fname}", out_dtype=torch.bfloat16)
    lin2 = workloads.up_proj_like(63, 256, 256, 4096)
    assert lib_splits(fmt, 256, 256, 4096) > 1
    check_layer(lin2, fmt, False, f"split-k-bf16-dx-{fname}", out_dtype=torch.bfloat16)


def lib_splits(fmt, M, N, K):
    """Split-K count the library picks for an M x N x K GEMM, read from its workspace size (the
    fixed header plus, when K is split, one fp32 M x N partial per split)."""
    base = av.lib().averis_linear_workspace_size(M, N, 256, fmt)  # K = 256: one K-step, never split
    ws = av.lib().averis_linear_workspace_size(M, N, K, fmt)
    return (ws - base) // (4 * M * N) if ws > base else 1
