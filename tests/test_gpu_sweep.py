"""GPU parity at full size, in the launch configuration bench.py times, on sampled outputs.

Every linear goes through LinearStep (the entry points, workspaces, bf16 Y / dX and fp32 dW the
bench uses) and its inputs are copied to the oracle.  Per linear:
  * both column means in full (1e-6 relative, as in test_gpu_quant.py);
  * sampled rows of the row-layout operands of X and D, and sampled 32-token blocks of their
    column-layout operands, bit-exact against the oracle's quantization of the same residuals
    given the GPU mean (NVFP4 with the scale of the whole operand's amax, after rotation);
  * sampled rows of Y and dX, and a sampled 32 x 32 block of dW, against the oracle's exact fp64
    products of the dequantized operands (the GPU's bytes, checked above).
Workloads: the seven Qwen3-0.6B-shaped sweep linears at l = 16384 (q 1024->2048, k and v
1024->1024, o 2048->1024, gate and up 1024->3072, down 3072->1024) on the bench's own device
draws, and the down_proj layer (l = 16384, 3072 -> 1024, SwiGLU-like input) with and without the
16x16 Hadamard; and the layer step with q/k/v and gate/up stored as fused projections (one
split of each group's output gradient and weight, one summed input gradient per group).  At
these sizes a short-K GEMM workgroup loops over up to six tiles and the long-K weight gradients
run over 64 K-steps.
"""
import functools

import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from fp4_quantized_amd.step import LinearStep
from oracle import averis_oracle as O
from tests.gpu_util import assert_q_equal, device, mean_ok, rel_fro, to_oracle

pytestmark = pytest.mark.gpu

FMTS = [(av.NVFP4, "nvfp4"), (av.MXFP4, "mxfp4")]


def sub(q, rows):
    """The oracle QTensor restricted to some outer rows."""
    return O.QTensor(q.codes[rows], q.scales[rows], q.s_dec, q.fmt, q.k, q.rotated)


def operand(r, hadamard):
    """An fp32 operand [outer, K] as the quantizer sees it: rotated along K if asked."""
    return O.hadamard16_f32(r) if hadamard else r


def check_rows_quantized(q_gpu, r_full, fmt, hadamard, rows, what):
    """Row-layout rows of the GPU operand == the oracle's quantization of the same residual rows."""
    r = O.pad_k(operand(r_full[rows], hadamard))
    if fmt == av.NVFP4:
        s_dec = O.nvfp4_tensor_scale(np.max(np.abs(operand(r_full, hadamard))))
        codes, scales = O.quantize_nvfp4(r, s_dec)
        assert np.float32(q_gpu.s_dec) == s_dec, f"{what}: tensor scale"
    else:
        codes, scales = O.quantize_mxfp4(r)
    assert np.array_equal(q_gpu.codes[rows], codes), f"{what}: codes differ"
    assert np.array_equal(q_gpu.scales[rows], scales), f"{what}: scales differ"


def check_token_blocks_quantized(q_gpu, r_full, fmt, hadamard, groups, what):
    """Column-layout (K = tokens) blocks of the GPU operand for 32-token groups == the oracle's
    quantization of those tokens' residuals, transposed (rotated along the tokens if asked)."""
    g = O.BLOCK[fmt]
    s_dec = None
    if fmt == av.NVFP4:
        s_dec = O.nvfp4_tensor_scale(np.max(np.abs(operand(np.ascontiguousarray(r_full.T), hadamard))))
        assert np.float32(q_gpu.s_dec) == s_dec, f"{what}: tensor scale"
    for t in groups:
        r = operand(np.ascontiguousarray(r_full[32 * t:32 * t + 32].T), hadamard)  # [cols, 32 tokens]
        codes, scales = O.quantize_nvfp4(r, s_dec) if fmt == av.NVFP4 else O.quantize_mxfp4(r)
        spg = 32 // g  # scale bytes per 32 tokens
        assert np.array_equal(q_gpu.codes[:, 16 * t:16 * t + 16], codes), f"{what}: codes of tokens {32 * t}.."
        assert np.array_equal(q_gpu.scales[:, spg * t:spg * t + spg], scales), f"{what}: scales of tokens {32 * t}.."


def check_bf16(got, ref, what):
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} sampled bf16 outputs off"


def mean_vector(q):
    """The dequantized mean row, rotation undone (the dW rank-one factor)."""
    v = O.dequantize(q)[0]
    return (O.unrotate16_f64(v) if q.rotated else v)[:q.k]


def check_linear_sampled(name, x, d, w, fmt, hadamard, rng):
    l, m = x.shape
    n = d.shape[1]
    print(f"case {name} l={l} m={m} n={n} fmt={fmt} h16={hadamard}", flush=True)
    st = LinearStep(x, d, w, fmt, split=True, hadamard=hadamard)
    st.run()
    torch.cuda.synchronize()
    xh, dh = x.float().cpu().numpy(), d.float().cpu().numpy()
    mux, mud = st.sx["mean"].cpu().numpy(), st.sd["mean"].cpu().numpy()
    assert mean_ok(mux, xh), f"{name}: mean of X"
    assert mean_ok(mud, dh), f"{name}: mean of D"
    rx, rd = O.residual(xh, mux), O.residual(dh, mud)
    del xh, dh

    rows = np.unique(np.concatenate([[0, 127, 128, l - 1], rng.choice(l, 44, replace=False)]))
    q_xr, q_dr = to_oracle(st.sx["row"]), to_oracle(st.sd["row"])
    check_rows_quantized(q_xr, rx, fmt, hadamard, rows, f"{name}: X row layout")
    check_rows_quantized(q_dr, rd, fmt, hadamard, rows, f"{name}: D row layout")
    groups = sorted({0, l // 32 - 1, *rng.choice(l // 32, 2, replace=False).tolist()})
    q_xc, q_dc = to_oracle(st.sx["col"]), to_oracle(st.sd["col"])
    check_token_blocks_quantized(q_xc, rx, fmt, hadamard, groups, f"{name}: X column layout")
    check_token_blocks_quantized(q_dc, rd, fmt, hadamard, groups, f"{name}: D column layout")

    q_mx, q_md = to_oracle(st.sx["mean_q"]), to_oracle(st.sd["mean_q"])
    y_ref = O.linear_fwd(sub(q_xr, rows), q_mx, to_oracle(st.sw["col"]))
    check_bf16(st.y.float().cpu().numpy()[rows], y_ref, f"{name}: Y")
    dx_ref = O.linear_bwd_dx(sub(q_dr, rows), q_md, to_oracle(st.sw["row"]))
    check_bf16(st.dx.float().cpu().numpy()[rows], dx_ref, f"{name}: dX")

    # dW on a 32 x 32 sample of (X feature, D feature) pairs: the token-axis operands' rows of
    # those features and those features of the dequantized means
    rm = np.sort(rng.choice(m, 32, replace=False))
    cn = np.sort(rng.choice(n, 32, replace=False))
    dw_ref = O.dw_dense(O.dequantize(sub(q_xc, rm)), O.dequantize(sub(q_dc, cn)), mean_vector(q_mx)[rm],
                        mean_vector(q_md)[cn], l)
    err = rel_fro(st.dw.cpu().numpy()[np.ix_(rm, cn)], dw_ref)
    assert err <= 1e-5, f"{name}: dW sampled block relative Frobenius error {err:.3e}"


@pytest.mark.parametrize("fmt,fname", FMTS)
def test_layer_sweep_sampled(fmt, fname):
    dev = device()
    rng = np.random.default_rng(11)
    for name, x, d, w in workloads.sweep_device(3, 16384, dev):
        check_linear_sampled(f"sweep-{name}-{fname}", x, d, w, fmt, False, rng)


@functools.lru_cache(maxsize=1)
def _down_proj():
    return workloads.down_proj()


@pytest.mark.parametrize("fmt,fname", FMTS)
@pytest.mark.parametrize("hadamard", [False, True])
def test_down_proj_sampled(fmt, fname, hadamard):
    dev = device()
    lin = _down_proj()
    x, d, w = (workloads.to_torch(a, "bf16", dev) for a in (lin.x, lin.d, lin.w))
    check_linear_sampled(f"down_proj-{fname}{'-h16' if hadamard else ''}", x, d, w, fmt, hadamard,
                         np.random.default_rng(12))


def test_layer_fused_projections_sampled():
    # The layer step as the bench times it with q/k/v and gate/up stored as fused projections
    # (MXFP4, two streams, l = 16384): per group, the mean of the concatenated output gradient
    # D = [D_1 .. D_k] in full, sampled rows of D's row layout and the whole weight W = [W_1 .. W_k]
    # in its K = N layout bit-exact, and sampled rows of the group's forward output and of its one
    # input gradient 1 (mu_D W^T) + D_R W^T against the oracle's exact products
    from fp4_quantized_amd.step import LayerStep
    dev = device()
    rng = np.random.default_rng(13)
    print("case layer-fused-projections l=16384 mxfp4", flush=True)
    layers = workloads.layer_device(3, 16384, dev, shared=True, cat=True)
    st = LayerStep(layers, av.MXFP4, split=True)
    assert sorted(st.dx_fused) == [0, 2]
    st.run()
    torch.cuda.synchronize()
    fmt = av.MXFP4
    for pi, names in ((0, ("q", "k", "v")), (2, ("gate", "up"))):
        what = "/".join(names)
        grp = [c for c in layers if c[0] in names]
        f, fw = st.dx_fused[pi], st.fwd_fused[pi]
        x = grp[0][1]
        l = x.shape[0]
        dh = torch.cat([c[2] for c in grp], 1).float().cpu().numpy()
        wh = torch.cat([c[3] for c in grp], 1).float().cpu().numpy()
        mud = f["d"]["mean"].cpu().numpy()
        assert mean_ok(mud, dh), f"{what}: mean of D"
        rows = np.unique(np.concatenate([[0, 127, 128, l - 1], rng.choice(l, 44, replace=False)]))
        q_dr = to_oracle(f["d"]["row"])
        check_rows_quantized(q_dr, O.residual(dh, mud), fmt, False, rows, f"{what}: D row layout")
        del dh
        ow = O.split_quant(wh, fmt, split=False)
        assert_q_equal(f["w"]["row"], ow["row"], f"{what}: W row layout")
        assert_q_equal(fw["w"], ow["col"], f"{what}: W column layout")
        q_wr, q_wc = to_oracle(f["w"]["row"]), to_oracle(fw["w"])
        dx_ref = O.linear_bwd_dx(sub(q_dr, rows), to_oracle(f["d"]["mean_q"]), q_wr)
        check_bf16(f["dx"].float().cpu().numpy()[rows], dx_ref, f"{what}: summed dX")
        sx = fw["sx"]
        y_ref = O.linear_fwd(sub(to_oracle(sx["row"]), rows), to_oracle(sx["mean_q"]), q_wc)
        check_bf16(fw["y"].float().cpu().numpy()[rows], y_ref, f"{what}: Y")
