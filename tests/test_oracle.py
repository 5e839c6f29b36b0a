"""Pins for the CPU oracle: each test checks the oracle against something other than itself
(brute force, closed forms, invariants, library routines, hand-worked fixtures).

Sources: "均值偏置的诅咒与祝福：FP4量化大语言模型训练" explainer (paper.rainbus.top), sections
前置知识 (FP4量化, 块量化, Hadamard变换) and 方法步骤详情 (the split and the three GEMMs);
paperlayer.ai summary of v2, §3 Method and Appendix D.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import averis_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.json")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# ----------------------------------------------------------------------------- E2M1 -----

def _nearest_e2m1(v):
    """Exhaustive nearest-grid search in fp64, ties to the even code."""
    a = np.minimum(np.abs(v.astype(np.float64)), 7.0)  # beyond 6 the nearest point is 6
    d = np.abs(a[:, None] - GRID[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates take the even code index (codes 0..7 are grid positions)
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (code | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_value_is_the_format_grid():
    vals = O.e2m1_value(np.arange(16))
    assert list(vals[:8]) == list(GRID)
    assert list(vals[8:]) == list(-GRID)


def test_e2m1_all_bf16_patterns():
    u = np.arange(1 << 16, dtype=np.uint32) << 16
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    np.testing.assert_array_equal(O.e2m1_encode(v), _nearest_e2m1(v))


def test_e2m1_every_fp32_in_the_rounding_range():
    # every positive fp32 in [2^-3, 2^3): all codes and all ties live here; below 2^-3 the
    # result is 0 and above 8 it saturates, which the random test covers.
    start = np.float32(2.0 ** -3).view(np.uint32)
    stop = np.float32(8.0).view(np.uint32)
    for lo in range(int(start), int(stop), 1 << 23):
        u = np.arange(lo, min(lo + (1 << 23), int(stop)), dtype=np.uint32)
        v = u.view(np.float32)
        got = O.e2m1_encode(v)
        np.testing.assert_array_equal(got, _nearest_e2m1(v))
        np.testing.assert_array_equal(O.e2m1_encode(-v), got | 8)


def test_e2m1_random_fp32_patterns():
    rng = np.random.default_rng(123)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    np.testing.assert_array_equal(O.e2m1_encode(v), _nearest_e2m1(v))


# ----------------------------------------------------------------------------- E4M3 -----

E4M3_VALUES = np.array([O.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)


def _nearest_e4m3(v):
    v = np.minimum(v.astype(np.float64), 448.0)
    d = np.abs(v[:, None] - E4M3_VALUES[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(0x7F)[None, :] % 2 == 0)
    return np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1)).astype(np.uint8)


def test_e4m3_value_matches_torch_float8():
    codes = torch.arange(0x7F, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e4m3_value(np.arange(0x7F)), ref)


def test_e4m3_encode_exhaustive_over_mantissa_tops():
    # every exponent in [2^-12, 2^9], all 2^7 top mantissa bits, and low-bit patterns that
    # put the value exactly on, just below and just above every rounding midpoint
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x3FFFF, 0x40000, 0x40001,
                     0x7FFFF, 0x80000, 0x80001, 0xFFFFF], dtype=np.uint32)
    exps = np.arange(127 - 12, 127 + 10, dtype=np.uint32)
    tops = np.arange(1 << 3, dtype=np.uint32) << 20
    mids = np.arange(1 << 4, dtype=np.uint32) << 16
    u = (exps[:, None, None, None] << 23) | tops[None, :, None, None] | \
        mids[None, None, :, None] | lows[None, None, None, :]
    v = u.ravel().view(np.float32)
    v = np.concatenate([v, np.float32([0.0, 2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -11, 448, 464,
                                       465, 1e6])])
    np.testing.assert_array_equal(O.e4m3_encode(v), _nearest_e4m3(v))


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(7)
    v = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 500_000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(v), ref)


# ----------------------------------------------------------------------------- E8M0 -----

def _floor_log2_bits(v):
    """floor(log2 v) from the fp32 bit pattern (exponent field, or subnormal bit length)."""
    u = v.view(np.uint32).astype(np.int64)
    e = (u >> 23) & 0xFF
    m = u & 0x7FFFFF
    sub = np.array([int(x).bit_length() for x in m[e == 0]], dtype=np.int64) - 150
    out = e - 127
    out[e == 0] = sub
    return out


def test_mx_scale_exponent_all_binades():
    rng = np.random.default_rng(3)
    u = (np.arange(1, 255, dtype=np.uint32)[:, None] << 23) | \
        rng.integers(0, 1 << 23, size=(254, 64)).astype(np.uint32)
    sub = rng.integers(1, 1 << 23, size=2000).astype(np.uint32)
    v = np.concatenate([u.ravel(), sub, np.uint32([1, 0x7FFFFF, 0x800000])]).view(np.float32)
    want = np.clip(_floor_log2_bits(v) - 2, -127, 127)
    np.testing.assert_array_equal(O.mx_scale_exponent(v), want)
    assert O.mx_scale_exponent(np.float32(0.0)) == -127


# ---------------------------------------------------------------- hand-worked blocks -----

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", range(5))
def test_golden_mxfp4_blocks(case):
    c = _golden()["mxfp4"][case]
    v = np.array(c["values"], dtype=np.float32)[None, :]
    codes, scales = O.quantize_mxfp4(v)
    assert int(scales[0, 0]) == c["scale"], c["name"]
    np.testing.assert_array_equal(O.unpack_nibbles(codes)[0], c["codes"], err_msg=c["name"])


@pytest.mark.parametrize("case", range(3))
def test_golden_nvfp4_blocks(case):
    c = _golden()["nvfp4"][case]
    v = np.array(c["values"], dtype=np.float32)[None, :]
    q = O.quantize(v, O.NVFP4)
    assert q.s_dec == np.float32(c["s_dec"]), c["name"]
    np.testing.assert_array_equal(q.scales[0], c["scales"], err_msg=c["name"])
    np.testing.assert_array_equal(O.unpack_nibbles(q.codes)[0], c["codes"], err_msg=c["name"])


def test_golden_nvfp4_hadamard_block():
    # reading: the NVFP4 tensor scale of a rotated operand comes from its rotated amax
    c = _golden()["nvfp4_hadamard"][0]
    v = np.array(c["values"], dtype=np.float32)[None, :]
    q = O.quantize(v, O.NVFP4, rotate=True)
    assert q.s_dec == np.float32(c["s_dec"]), c["name"]
    np.testing.assert_array_equal(q.scales[0], c["scales"], err_msg=c["name"])
    np.testing.assert_array_equal(O.unpack_nibbles(q.codes)[0], c["codes"], err_msg=c["name"])


def test_pack_nibble_order():
    c = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    assert list(O.pack_nibbles(c)[0]) == [0x21, 0x43]
    np.testing.assert_array_equal(O.unpack_nibbles(O.pack_nibbles(c)), c)


# ------------------------------------------------------------------------ dequantize -----

def test_dequantize_by_hand():
    # MXFP4: byte 124 -> 2^-3; code 0xD = -3 -> -0.375.  NVFP4: scale 0x22 = 0.15625,
    # s_dec 2 -> block scale 0.3125; code 6 -> 4 * 0.3125 = 1.25.
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 0xD
    q = O.QTensor(O.pack_nibbles(codes), np.uint8([[124]]), None, O.MXFP4, 32, False)
    assert O.dequantize(q)[0, 0] == -0.375 and not O.dequantize(q)[0, 1:].any()
    codes = np.zeros((1, 16), np.uint8)
    codes[0, 3] = 6
    q = O.QTensor(O.pack_nibbles(codes), np.uint8([[0x22]]), np.float32(2.0), O.NVFP4, 16, False)
    assert O.dequantize(q)[0, 3] == 1.25


# ---------------------------------------------------------------------------- split -----

def test_column_mean_is_the_exact_mean():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((777, 40)) * 3 + rng.standard_normal(40) * 50).astype(np.float32)
    mu64, mu32 = O.column_mean(x)
    exact = np.array([math.fsum(float(t) for t in x[:, j]) / x.shape[0] for j in range(40)])
    np.testing.assert_allclose(mu64, exact, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(mu32, exact.astype(np.float32))


def test_residual_columns_sum_to_zero():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((512, 64)) + rng.standard_normal(64) * 10).astype(np.float32)
    mu64, _ = O.column_mean(x)
    s = np.sum(x.astype(np.float64) - mu64[None, :], axis=0)
    assert np.all(np.abs(s) <= 1e-12 * np.sum(np.abs(x), axis=0))


def test_residual_is_one_fp32_subtraction():
    x = np.float32([[1.0, 3.0], [2.0, -1.0]])
    mu = np.float32([1.5, 1.0])
    np.testing.assert_array_equal(O.residual(x, mu), np.float32([[-0.5, 2.0], [0.5, -2.0]]))


def _rand_layer(seed, l=96, m=64, n=48):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((l, m)) + rng.standard_normal(m) * 5
    d = rng.standard_normal((l, n)) * 1e-3 + rng.standard_normal(n) * 1e-3
    w = rng.standard_normal((m, n)) * 0.02
    return x, d, w


def test_split_algebra_unquantized_fwd_dx_dw():
    # [rainbus] 方法步骤详情: with exact arithmetic the split is algebra:
    # 1(mu W) + X_R W = XW, 1(mu_D W^T) + D_R W^T = DW^T, X_R^T D_R + l mu_X^T mu_D = X^T D.
    x, d, w = _rand_layer(5)
    l = x.shape[0]
    mx, md = x.mean(axis=0), d.mean(axis=0)
    xr, dr = x - mx, d - md
    y = O.fwd_dense(xr, mx, w.T)
    dx = O.dx_dense(dr, md, w)
    dw = O.dw_dense(xr.T, dr.T, mx, md, l)
    for got, want in ((y, x @ w), (dx, d @ w.T), (dw, x.T @ d)):
        assert np.linalg.norm(got - want) <= 1e-10 * np.linalg.norm(want)


def test_split_algebra_brute_force_tiny():
    x, d, w = _rand_layer(6, l=5, m=4, n=3)
    mx, md = x.mean(axis=0), d.mean(axis=0)
    y = O.fwd_dense(x - mx, mx, w.T)
    dw = O.dw_dense((x - mx).T, (d - md).T, mx, md, 5)
    for i in range(5):
        for k in range(3):
            assert abs(y[i, k] - math.fsum(x[i, j] * w[j, k] for j in range(4))) < 1e-12
    for j in range(4):
        for k in range(3):
            assert abs(dw[j, k] - math.fsum(x[i, j] * d[i, k] for i in range(5))) < 1e-12


def test_split_quant_vs_unquantized_is_close():
    # Quantization error is bounded: fwd output stays within FP4 noise of X W.
    x, d, w = _rand_layer(7, l=256, m=128, n=64)
    for fmt in (O.NVFP4, O.MXFP4):
        sx = O.split_quant(x, fmt)
        sw = O.split_quant(w, fmt, split=False)
        y = O.linear_fwd(sx["row"], sx["mean"], sw["col"])
        assert O.relative_error(y, x @ w) < 0.15


def test_hadamard_split_quant_fwd_dx_close_to_unquantized():
    # With the split and the rotation both on, every operand of the forward and input-gradient
    # GEMMs (residual, mean and weight) is rotated along K, so the products stay within FP4
    # noise of X W and D W^T.  The mean dominates these inputs: a mean quantized without the
    # rotation would meet a rotated weight and miss by far more than the noise.
    rng = np.random.default_rng(8)
    l, m, n = 256, 128, 64
    x = rng.standard_normal((l, m)) + rng.standard_normal(m) * 6
    d = rng.standard_normal((l, n)) * 1e-3 + rng.standard_normal(n) * 4e-3
    w = rng.standard_normal((m, n)) * 0.02
    for fmt in (O.NVFP4, O.MXFP4):
        sx = O.split_quant(x, fmt, hadamard=True)
        sd = O.split_quant(d, fmt, hadamard=True)
        sw = O.split_quant(w, fmt, split=False, hadamard=True)
        y = O.linear_fwd(sx["row"], sx["mean"], sw["col"])
        dx = O.linear_bwd_dx(sd["row"], sd["mean"], sw["row"])
        # FP4 noise of the three operands: 0.13-0.19 here; an unrotated mean gives about 1.4
        assert O.relative_error(y, x @ w) < 0.3
        assert O.relative_error(dx, d @ w.T) < 0.3


# ----------------------------------------------------------------------- quantizer -----

@pytest.mark.parametrize("fmt", [O.NVFP4, O.MXFP4])
def test_quantizer_idempotent(fmt):
    rng = np.random.default_rng(21)
    # row scales within e^+-2 keep every NVFP4 block scale in E4M3's normal range, where the
    # largest element of a block always comes back as code 7 and the scale is re-derived
    r = (rng.standard_t(4, (64, 256)) * np.exp(rng.uniform(-2, 2, (64, 1)))).astype(np.float32)
    q = O.quantize(r, fmt)
    back = O.dequantize(q).astype(np.float32)
    if fmt == O.MXFP4:
        q2 = O.quantize(back, fmt)
    else:  # hold the tensor scale fixed: re-derived s_dec may differ by an ulp
        c2, s2 = O.quantize_nvfp4(back, q.s_dec)
        q2 = O.QTensor(c2, s2, q.s_dec, fmt, q.k, False)
    np.testing.assert_array_equal(q2.codes, q.codes)
    np.testing.assert_array_equal(q2.scales, q.scales)


def test_mxfp4_on_grid_round_trip():
    rng = np.random.default_rng(22)
    codes = rng.integers(0, 16, (32, 64)).astype(np.uint8)
    codes[:, ::32] = 7  # each block holds +6 so its amax is 6 * 2^k
    k = rng.integers(-20, 20, (32, 2))
    v = O.e2m1_value(codes) * np.repeat(np.ldexp(1.0, k), 32, axis=1)
    codes[O.e2m1_value(codes) == 0] = 0  # -0 inputs come back as code 8; compare on values
    q = O.quantize(v.astype(np.float32), O.MXFP4)
    np.testing.assert_array_equal(q.scales, (k + 127).astype(np.uint8))
    np.testing.assert_array_equal(O.dequantize(q), v)


def test_zero_mean_input_gives_vanilla_codes():
    # integer columns with exact zero sums: mu == 0, so Averis codes equal vanilla codes
    rng = np.random.default_rng(23)
    h = rng.integers(-50, 50, (64, 128)).astype(np.float32)
    x = np.concatenate([h, -h], axis=0)
    for fmt in (O.NVFP4, O.MXFP4):
        a = O.split_quant(x, fmt)
        v = O.split_quant(x, fmt, split=False)
        assert not a["mu32"].any()
        for lay in ("row", "col"):
            np.testing.assert_array_equal(a[lay].codes, v[lay].codes)
            np.testing.assert_array_equal(a[lay].scales, v[lay].scales)


def test_rank_one_input_has_zero_residual():
    rng = np.random.default_rng(24)
    mu = (rng.standard_normal(64) * 8).astype(np.float32)
    x = np.repeat(mu[None, :], 40, axis=0)
    w = (rng.standard_normal((64, 32)) * 0.02).astype(np.float32)
    for fmt in (O.NVFP4, O.MXFP4):
        s = O.split_quant(x, fmt)
        assert not s["row"].codes.any() and not s["col"].codes.any()
        sw = O.split_quant(w, fmt, split=False)
        y = O.linear_fwd(s["row"], s["mean"], sw["col"])
        want = O.dequantize(s["mean"])[:, :64] @ O.dequantize(sw["col"])[:, :64].T
        np.testing.assert_array_equal(y, np.repeat(want, 40, axis=0))


def test_col_layout_is_zero_padded_transpose():
    rng = np.random.default_rng(25)
    x = rng.standard_normal((37, 64)).astype(np.float32)
    s = O.split_quant(x, O.MXFP4, split=False)
    assert s["col"].codes.shape == (64, 128)  # 37 rows padded to 256 -> 128 bytes
    dq = O.dequantize(s["col"])
    assert not dq[:, 37:].any()
    # same values as quantizing each column's 32-row blocks directly
    ref = O.quantize(np.pad(x.T, ((0, 0), (0, 219))), O.MXFP4)
    np.testing.assert_array_equal(s["col"].codes, ref.codes)


# ----------------------------------------------------------------------- Hadamard -----

def test_sylvester_matches_scipy():
    np.testing.assert_array_equal(O.sylvester16(), scipy.linalg.hadamard(16))


def test_hadamard_butterflies_match_matrix():
    rng = np.random.default_rng(31)
    r = (rng.standard_normal((50, 64)) * 10).astype(np.float32)
    got = O.hadamard16_f32(r).astype(np.float64)
    want = (r.astype(np.float64).reshape(-1, 16) @ (scipy.linalg.hadamard(16).T / 4.0)).reshape(50, 64)
    scale = np.abs(r.astype(np.float64)).reshape(-1, 16).sum(axis=1).repeat(16).reshape(50, 64)
    assert np.all(np.abs(got - want) <= 4 * 2.0 ** -24 * scale)
    # orthogonal and an involution
    back = O.unrotate16_f64(got)
    np.testing.assert_allclose(back, r, rtol=0, atol=1e-5 * np.abs(r).max())
    h = scipy.linalg.hadamard(16) / 4.0
    np.testing.assert_allclose(h @ h, np.eye(16), atol=1e-15)


def test_rotation_cancels_in_the_unquantized_products():
    x, d, w = _rand_layer(32, l=64, m=64, n=32)
    xr = x - x.mean(axis=0)
    xh = O.unrotate16_f64(xr)          # X_R H (H symmetric, so "unrotate" is the same map)
    wh = O.unrotate16_f64(w.T)         # (H W)^T, rotated along m
    assert np.linalg.norm(xh @ wh.T - xr @ w) <= 1e-12 * np.linalg.norm(xr @ w)


def test_hadamard_split_quant_dw_rank_one_uses_unrotated_mean():
    x, d, w = _rand_layer(33, l=128, m=64, n=32)
    for fmt in (O.NVFP4, O.MXFP4):
        sx = O.split_quant(x, fmt, hadamard=True)
        sd = O.split_quant(d, fmt, hadamard=True)
        dw = O.linear_bwd_dw(sx["col"], sd["col"], sx["mean"], sd["mean"], 128)
        # the exact answer X^T D is recovered to FP4 noise, not to the rotated mean
        assert O.relative_error(dw, x.T @ d) < 0.2


# ------------------------------------------------------------------ directional claim -----

def test_mean_removal_lowers_quantization_error_on_mean_biased_data():
    # [paperlayer] §2/§3: mean bias inflates block scales; after removing it the residual
    # quantizes with a much smaller error than the raw tensor does.  (The FP4 error of the
    # quantized mean itself is a separate, rank-one term and is not part of this claim.)
    from fp4_quantized_amd import workloads
    lin = workloads.up_proj_like(9, 512, 256, 128)
    x = lin.x.astype(np.float64)
    for fmt in (O.NVFP4, O.MXFP4):
        a = O.split_quant(lin.x, fmt)
        v = O.split_quant(lin.x, fmt, split=False)
        e_res = np.linalg.norm(O.dequantize(a["row"]) - (x - a["mu32"][None, :]))
        e_van = np.linalg.norm(O.dequantize(v["row"]) - x)
        assert e_res < 0.5 * e_van


# ------------------------------------------------------------------------ grouped -----

def test_grouped_equals_per_expert_calls():
    rng = np.random.default_rng(41)
    offs = np.array([0, 0, 17, 17, 100, 101])
    x = (rng.standard_normal((101, 64)) + 3).astype(np.float32)
    g = O.split_quant_grouped(x, offs, O.MXFP4)
    assert g[0] is None and g[2] is None
    s = O.split_quant(x[17:100], O.MXFP4)
    np.testing.assert_array_equal(g[3]["row"].codes, s["row"].codes)
    np.testing.assert_array_equal(g[3]["col"].codes, s["col"].codes)
    np.testing.assert_array_equal(g[3]["mu32"], x[17:100].astype(np.float64).mean(axis=0).astype(np.float32))


def test_grouped_linear_stacks_per_expert_results():
    # the grouped GEMMs are the per-expert GEMMs stacked in expert order; an empty expert adds
    # no rows and gets dW = 0; each expert's rank-one factor is its own token count
    rng = np.random.default_rng(43)
    offs = np.array([0, 40, 40, 90])
    m, n = 64, 32
    x = (rng.standard_normal((90, m)) + 2).astype(np.float32)
    d = (rng.standard_normal((90, n)) * 1e-3 + 1e-3).astype(np.float32)
    ws = [(rng.standard_normal((m, n)) * 0.02).astype(np.float32) for _ in range(3)]
    sx = O.split_quant_grouped(x, offs, O.NVFP4)
    sd = O.split_quant_grouped(d, offs, O.NVFP4)
    qw = [O.split_quant(w, O.NVFP4, split=False) for w in ws]
    y = O.linear_fwd_grouped(sx, [q["col"] for q in qw], offs, n)
    dx = O.linear_bwd_dx_grouped(sd, [q["row"] for q in qw], offs, m)
    dw = O.linear_bwd_dw_grouped(sx, sd, offs, m, n)
    assert y.shape == (90, n) and dx.shape == (90, m) and dw.shape == (3, m, n)
    np.testing.assert_array_equal(y[40:], O.linear_fwd(sx[2]["row"], sx[2]["mean"], qw[2]["col"]))
    np.testing.assert_array_equal(dx[:40], O.linear_bwd_dx(sd[0]["row"], sd[0]["mean"], qw[0]["row"]))
    assert not dw[1].any()
    ref = O.linear_bwd_dw(sx[2]["col"], sd[2]["col"], sx[2]["mean"], sd[2]["mean"], 50)
    np.testing.assert_array_equal(dw[2], ref)
    # the rank-one term uses l_e = 50, not the total 90: removing it leaves X_R^T D_R alone
    no_mean = O.linear_bwd_dw(sx[2]["col"], sd[2]["col"], None, None, 50)
    u = O.dequantize(sx[2]["mean"])[0, :m]
    v = O.dequantize(sd[2]["mean"])[0, :n]
    np.testing.assert_allclose(dw[2] - no_mean, 50.0 * np.outer(u, v), rtol=1e-12, atol=1e-18)


# ------------------------------------------------------------- stochastic rounding -----

def test_philox4x32_10_known_answers():
    # the known-answer vectors published with the Random123 library for philox4x32 with 10
    # rounds (counter, key -> output)
    kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
           ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
           ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
            (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in kat:
        got = O.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
        assert [int(v) for v in got] == list(want)


def _grid_floor_ceil(a):
    """Largest grid magnitude <= a and smallest >= a (capped at 6), by exhaustive search."""
    g = GRID[None, :]
    fl = np.where(g <= a[:, None], g, -1.0).max(axis=1)
    ce = np.where(g >= a[:, None], g, 99.0).min(axis=1)
    return fl, np.minimum(ce, 6.0)


def test_sr_extreme_draws_are_directed_roundings():
    # every positive bf16 value below 8: the draw u = 0 rounds every magnitude up to the next
    # grid value (ties: values on the grid stay), the draw u = 2^16 - 1 rounds down unless the
    # value is within 2^-16 of a step below the next grid value
    u = np.arange(1 << 16, dtype=np.uint32) << 16
    v = u.view(np.float32)
    v = v[np.isfinite(v) & (v > 0) & (v < 8)]
    fl, ce = _grid_floor_ceil(v.astype(np.float64))
    up = O.e2m1_value(O.e2m1_encode_sr(v, np.zeros(v.shape, np.uint32)))
    np.testing.assert_array_equal(up, np.where(v >= 6, 6.0, ce))
    down = O.e2m1_value(O.e2m1_encode_sr(v, np.full(v.shape, 0xFFFF, np.uint32)))
    step = np.where(ce > fl, ce - fl, 1.0)
    near_top = (v.astype(np.float64) - fl) / step > 65535 / 65536
    np.testing.assert_array_equal(down, np.where(v >= 6, 6.0, np.where(near_top, ce, fl)))
    np.testing.assert_array_equal(O.e2m1_encode_sr(-v, np.zeros(v.shape, np.uint32)) >> 3, 1)


def test_sr_is_unbiased_over_every_draw():
    # averaged over all 2^16 draws the rounded magnitude equals the input to within
    # step * 2^-16 (exactly when the position between the neighbours has <= 16 fraction bits)
    rng = np.random.default_rng(51)
    v = np.concatenate([rng.uniform(0, 6, 200), [0.0, 0.5, 0.3, 2.75, 5.999, 4.0]]).astype(np.float32)
    draws = np.arange(1 << 16, dtype=np.uint32)
    for x in v:
        mean = O.e2m1_value(O.e2m1_encode_sr(np.full(draws.shape, x, np.float32), draws)).mean()
        fl, ce = _grid_floor_ceil(np.array([float(x)]))
        assert abs(mean - float(x)) <= (ce[0] - fl[0]) * 2.0 ** -16 + 1e-12, x


def test_sr_split_quant_is_seeded_and_one_step_from_nearest():
    # same seed -> same codes; another seed -> other codes; every stochastically rounded value is
    # one of the two grid neighbours of the scaled input (scales are those of round to nearest)
    x, _, _ = _rand_layer(52, l=96, m=64, n=32)
    for fmt in (O.NVFP4, O.MXFP4):
        a = O.split_quant(x, fmt, sr_seed=7)
        b = O.split_quant(x, fmt, sr_seed=7)
        c = O.split_quant(x, fmt, sr_seed=8)
        r = O.split_quant(x, fmt)
        for lay in ("row", "col", "mean"):
            np.testing.assert_array_equal(a[lay].codes, b[lay].codes)
            np.testing.assert_array_equal(a[lay].scales, r[lay].scales)
        assert not np.array_equal(a["row"].codes, c["row"].codes)
        dq_sr, dq_rn = O.dequantize(a["row"]), O.dequantize(r["row"])
        g = O.BLOCK[fmt]
        scale = np.repeat(O.dequantize(O.QTensor(np.full_like(r["row"].codes, 0x22), r["row"].scales,
                                                 r["row"].s_dec, fmt, r["row"].k, False))[:, ::g], g, axis=1)
        steps = np.abs(dq_sr - dq_rn) / np.where(scale > 0, scale, 1.0)  # in units of the block scale
        assert steps.max() <= 2.0 + 1e-9  # neighbours differ by at most one grid step (<= 2 units)


# ---------------- producers of the linear inputs (RMSNorm, SwiGLU) ----------------

def test_rmsnorm_closed_form():
    # row [3, 4]: mean of squares 12.5, so y = [3, 4] / sqrt(12.5); a zero row stays zero with eps
    x = np.array([[3.0, 4.0], [0.0, 0.0]], np.float32)
    y = O.rmsnorm(x[:1], np.ones(2, np.float32), 0.0, out_bf16=False)
    np.testing.assert_allclose(y[0], np.array([3.0, 4.0]) / np.sqrt(12.5), rtol=3e-7)
    y = O.rmsnorm(x, np.array([2.0, -1.0], np.float32), 1e-6, out_bf16=False)
    np.testing.assert_allclose(y[0], np.array([6.0, -4.0]) / np.sqrt(12.5 + 1e-6), rtol=3e-7)
    assert not y[1].any()


def test_rmsnorm_matches_torch_and_is_scale_invariant():
    rng = np.random.default_rng(40)
    x = rng.standard_normal((64, 96)).astype(np.float32) * 3
    w = rng.standard_normal(96).astype(np.float32)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (96,), torch.from_numpy(w).double(), eps=1e-5)
    y = O.rmsnorm(x, w, 1e-5, out_bf16=False)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-6, atol=1e-6)
    # scaling a row by a power of two scales its root mean square by the same power (eps = 0)
    assert np.array_equal(O.rmsnorm(x * np.float32(4), w, 0.0), O.rmsnorm(x, w, 0.0))
    # bf16 output: the fp32 result rounded to nearest even
    yb = O.rmsnorm(x, w, 1e-5)
    assert np.array_equal(yb, torch.from_numpy(y).to(torch.bfloat16).float().numpy())


def test_swiglu_matches_torch_and_special_values():
    rng = np.random.default_rng(41)
    g = (rng.standard_normal((32, 64)) * 4).astype(np.float32)
    u = rng.standard_normal((32, 64)).astype(np.float32)
    ref = torch.nn.functional.silu(torch.from_numpy(g).double()) * torch.from_numpy(u).double()
    np.testing.assert_allclose(O.swiglu(g, u, out_bf16=False), ref.numpy(), rtol=1e-6, atol=1e-7)
    s = O.swiglu(np.array([[0.0, 40.0, -40.0, 1.0]], np.float32), np.ones((1, 4), np.float32), out_bf16=False)
    assert s[0, 0] == 0.0 and s[0, 1] == 40.0 and abs(s[0, 2]) < 1e-15
    np.testing.assert_allclose(s[0, 3], 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-7)
