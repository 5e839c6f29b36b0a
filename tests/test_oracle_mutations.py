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
    monkeypatch.setattr(O, "quantize_nvfp4", lambda r, s: orig(r, np.float32(s) * np.float32(6)))
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
