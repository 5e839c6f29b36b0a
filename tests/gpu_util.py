"""Helpers shared by the GPU parity tests (no arithmetic of the method lives here)."""
import numpy as np
import pytest
import torch

from oracle import averis_oracle as O


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_quantized_amd.averis as av
    av.lib()  # a missing library on a GPU machine is an error, not a skip
    return torch.device("cuda:0")


def untile_scales(tiled, outer, k_pad, g):
    """Device scale layout (per 32-row group and 256-element K-step, 32 x 256/g contiguous
    bytes) -> row-major [round_up(outer, 32), k_pad / g]."""
    spb = 256 // g
    t = np.asarray(tiled, np.uint8).reshape(-1)
    rp = (outer + 31) // 32 * 32
    t = t.reshape(rp // 32, k_pad // 256, 32, spb).transpose(0, 2, 1, 3)
    return t.reshape(rp, k_pad // g)


def row_scales(q):
    return untile_scales(q.scales.cpu().numpy(), q.outer, q.k_pad, O.BLOCK[q.fmt])


def to_oracle(q):
    """Copy a device QTensor into the oracle's QTensor (same bytes, scales untiled)."""
    ts = None if q.tensor_scale is None else np.float32(q.tensor_scale[0].item())
    return O.QTensor(q.codes.cpu().numpy(), row_scales(q)[:q.outer], ts, q.fmt, q.k, q.rotated)


def mean_ok(mu_gpu, x):
    """Mean tolerance: |d| <= 1e-6 (|mu| + mean |x|) per column and ||d|| <= 1e-6 ||mu||."""
    mu64, _ = O.column_mean(x)
    if x.shape[0] == 0:
        return bool(np.all(mu_gpu == 0))
    d = np.abs(mu_gpu.astype(np.float64) - mu64)
    scale = np.abs(mu64) + np.abs(np.asarray(x, np.float64)).mean(axis=0)
    ok_col = np.all(d <= 1e-6 * scale)
    ok_norm = np.linalg.norm(d) <= 1e-6 * max(np.linalg.norm(mu64), 1e-30) or not np.any(mu64)
    return bool(ok_col and ok_norm)


def assert_q_equal(g, o, what):
    """Codes and scales bit-exact, NVFP4 tensor scale exact; group-padding scale rows zero."""
    gc, full = g.codes.cpu().numpy(), row_scales(g)
    gs = full[:g.outer]
    assert not full[g.outer:].any(), f"{what}: scale rows past outer are not zero"
    assert gc.shape == o.codes.shape and gs.shape == o.scales.shape, what
    if not np.array_equal(gs, o.scales):
        bad = np.argwhere(gs != o.scales)
        raise AssertionError(f"{what}: {len(bad)} scale bytes differ, first at {bad[0].tolist()}: "
                             f"gpu {gs[tuple(bad[0])]} oracle {o.scales[tuple(bad[0])]}")
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()}: "
                             f"gpu {gc[tuple(bad[0])]:#04x} oracle {o.codes[tuple(bad[0])]:#04x}")
    if o.s_dec is not None:
        gt = np.float32(g.tensor_scale[0].item())
        assert gt == o.s_dec, f"{what}: tensor scale gpu {gt!r} oracle {o.s_dec!r}"


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))
