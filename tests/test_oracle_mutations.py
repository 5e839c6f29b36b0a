"""Planted mistakes: each test breaks the CPU oracle in one plausible way (a dropped term, a
wrong sign, a transposed operand, a wrong tie rule) and checks that one of the pins in
test_oracle.py then fails.  This shows the pins constrain the oracle, not only re-run it."""
import numpy as np
import pytest

from oracle import averis_oracle as O
from tests import test_oracle as P


def _fails(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_dropped_mean_term_is_caught(monkeypatch):
    orig = O.fwd_dense
    monkeypatch.setattr(O, "fwd_dense", lambda xr, mu, w: orig(xr, None, w))
    _fails(P.test_split_algebra_unquantized_fwd_dx_dw)


def test_missing_token_count_in_rank_one_term_is_caught(monkeypatch):
    orig = O.dw_dense
    monkeypatch.setattr(O, "dw_dense", lambda a, b, mx, md, l: orig(a, b, mx, md, 1))
    _fails(P.test_split_algebra_unquantized_fwd_dx_dw)


def test_misindexed_weight_is_caught(monkeypatch):
    orig = O.dx_dense
    monkeypatch.setattr(O, "dx_dense", lambda dr, md, w: orig(dr, md, w[:, ::-1]))
    _fails(P.test_split_algebra_unquantized_fwd_dx_dw)


def test_wrong_residual_sign_is_caught(monkeypatch):
    monkeypatch.setattr(O, "residual", lambda x, mu: np.asarray(mu, np.float32)[None, :] - np.asarray(x, np.float32))
    _fails(P.test_residual_is_one_fp32_subtraction)


def test_ties_away_from_even_is_caught(monkeypatch):
    orig = O.e2m1_encode

    def bad(v):
        c = orig(v)
        a = np.abs(np.asarray(v, np.float32))
        c[a == 2.5] = (c[a == 2.5] & 8) | 5
        return c
    monkeypatch.setattr(O, "e2m1_encode", bad)
    _fails(P.test_e2m1_all_bf16_patterns)


def test_missing_divide_by_six_in_nvfp4_scale_is_caught(monkeypatch):
    orig = O.quantize_nvfp4
    monkeypatch.setattr(O, "quantize_nvfp4", lambda r, s, u16=None: orig(r, np.float32(s) * np.float32(6), u16))
    _fails(P.test_golden_nvfp4_blocks, 0)


def test_mx_exponent_off_by_one_is_caught(monkeypatch):
    orig = O.mx_scale_exponent
    monkeypatch.setattr(O, "mx_scale_exponent", lambda a: orig(a) + 1)
    _fails(P.test_golden_mxfp4_blocks, 0)


def test_swapped_nibbles_are_caught(monkeypatch):
    monkeypatch.setattr(O, "pack_nibbles",
                        lambda c: ((np.asarray(c, np.uint8)[..., 1::2] & 15) |
                                   ((np.asarray(c, np.uint8)[..., 0::2] & 15) << 4)))
    _fails(P.test_pack_nibble_order)


def test_nvfp4_amax_before_rotation_is_caught(monkeypatch):
    orig = O.quantize

    def bad(r, fmt, rotate=False, k=None):
        if fmt != O.NVFP4 or not rotate:
            return orig(r, fmt, rotate, k)
        r = np.asarray(r, np.float32)
        s_dec = O.nvfp4_tensor_scale(np.max(np.abs(r)) if r.size else 0.0)  # unrotated amax
        codes, scales = O.quantize_nvfp4(O.hadamard16_f32(r), s_dec)
        return O.QTensor(codes, scales, s_dec, fmt, r.shape[1] if k is None else k, True)
    monkeypatch.setattr(O, "quantize", bad)
    _fails(P.test_golden_nvfp4_hadamard_block)


def test_subnormal_decode_scale_not_zeroed_is_caught(monkeypatch):
    def bad(r, s_dec, u16=None):  # the NVFP4 block quantizer without the "decode scale below 2^-126" rule
        r = np.asarray(r, dtype=np.float32)
        outer, K = r.shape
        blk = r.reshape(outer, K // 16, 16)
        amax = np.max(np.abs(blk), axis=2)
        s_dec = np.float32(s_dec)
        with np.errstate(all="ignore"):
            e = O.e4m3_encode(((amax / np.float32(6.0)).astype(np.float32) / s_dec).astype(np.float32))
            S = (O.e4m3_value(e).astype(np.float32) * s_dec).astype(np.float32)
            codes = O.e2m1_encode((blk * (np.float32(1.0) / S)[:, :, None]).astype(np.float32))
        codes[e == 0] = 0
        return O.pack_nibbles(codes.reshape(outer, K)), e
    monkeypatch.setattr(O, "quantize_nvfp4", bad)
    _fails(P.test_golden_nvfp4_blocks, 2)


def test_unrotated_mean_under_hadamard_is_caught(monkeypatch):
    orig = O.split_quant

    def bad(x, fmt, split=True, hadamard=False, mean=None):
        out = orig(x, fmt, split, hadamard, mean)
        if split and hadamard:  # the mean quantized without the rotation, labelled rotated
            q = O.quantize(O.pad_k(out["mu32"][None, :]), fmt, rotate=False, k=out["mu32"].shape[0])
            q.rotated = True
            out["mean"] = q
        return out
    monkeypatch.setattr(O, "split_quant", bad)
    _fails(P.test_hadamard_split_quant_fwd_dx_close_to_unquantized)


def test_philox_key_bumped_before_the_first_round_is_caught(monkeypatch):
    orig = O.philox4x32_10

    def bad(ctr, key):  # one bump too many: the first round already uses the bumped key
        return orig(ctr, ((key[0] + O.PHILOX_W[0]) & 0xFFFFFFFF, (key[1] + O.PHILOX_W[1]) & 0xFFFFFFFF))
    monkeypatch.setattr(O, "philox4x32_10", bad)
    _fails(P.test_philox4x32_10_known_answers)


def test_sr_rounding_up_on_equal_draw_is_caught(monkeypatch):
    def bad(v, u16):  # "<=" in place of "<": values on the grid round up on the draw 0
        v = np.asarray(v, np.float32)
        a = np.abs(v)
        grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
        lo_i = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 6)
        p = ((a - grid[lo_i]) / (grid[lo_i + 1] - grid[lo_i])).astype(np.float32)
        up = np.asarray(u16, np.float64) / 65536.0 <= p
        c = np.where(a >= 6, 7, lo_i + up).astype(np.uint8)
        return c | (np.signbit(v).astype(np.uint8) << 3)
    monkeypatch.setattr(O, "e2m1_encode_sr", bad)
    _fails(P.test_sr_extreme_draws_are_directed_roundings)


def test_rmsnorm_mean_over_wrong_count_is_caught(monkeypatch):
    orig = O.rmsnorm

    def bad(x, w, eps, out_bf16=True):  # the mean of squares over cols + 1
        x = np.asarray(x, np.float32)
        xz = np.concatenate([x, np.zeros((x.shape[0], 1), np.float32)], 1)
        return orig(xz, np.append(np.asarray(w, np.float32), np.float32(1.0)), eps, out_bf16)[:, :-1]
    monkeypatch.setattr(O, "rmsnorm", bad)
    _fails(P.test_rmsnorm_closed_form)


def test_swiglu_sigmoid_without_gate_factor_is_caught(monkeypatch):
    def bad(g, u, out_bf16=True):
        g = np.asarray(g, np.float32)
        y = (np.float32(1.0) / (np.float32(1.0) + np.float32(np.exp(-g.astype(np.float64))))) * np.asarray(u, np.float32)
        return O.round_bf16(y) if out_bf16 else y
    monkeypatch.setattr(O, "swiglu", bad)
    _fails(P.test_swiglu_matches_torch_and_special_values)
