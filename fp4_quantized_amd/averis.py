"""Thin ctypes binding of libaveris.so (C ABI in include/averis.h).

Argument marshalling only: torch supplies device memory and the current HIP stream; every
step of the computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or no GPU is present, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

NVFP4 = 1
MXFP4 = 2
F32 = 0
BF16 = 1
SPLIT = 1 << 0
HADAMARD16 = 1 << 1
MEAN_GIVEN = 1 << 2
CHECK_FINITE = 1 << 3
STATUS_NONFINITE = 1 << 0
STATUS_UNDERFLOW = 1 << 1
ACCUMULATE = 1 << 4
KPAD = 256
BLOCK = {NVFP4: 16, MXFP4: 32}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaveris.so")

EXPORTS = [
    "averis_abi_version", "averis_status_string", "averis_source_digest",
    "averis_split_quant_workspace_size", "averis_split_quant", "averis_split_quant_sr", "averis_split_quant_batch",
    "averis_split_quant_noalloc_max_bytes", "averis_split_quant_noalloc",
    "averis_linear_workspace_size", "averis_linear_fwd", "averis_linear_bwd_dx",
    "averis_colstats_capacity", "averis_linear_fwd_stats", "averis_linear_bwd_dx_stats", "averis_split_quant_stats",
    "averis_rmsnorm_stats", "averis_swiglu_stats",
    "averis_linear_bwd_dw_workspace_size", "averis_linear_bwd_dw",
    "averis_split_quant_grouped_workspace_size", "averis_split_quant_grouped",
    "averis_linear_grouped_workspace_size", "averis_linear_fwd_grouped", "averis_linear_bwd_dx_grouped",
    "averis_linear_bwd_dw_grouped_workspace_size", "averis_linear_bwd_dw_grouped",
]


class CQTensor(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_void_p),
        ("outer", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("k_pad", ctypes.c_int64),
        ("fmt", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class CSplitQuantItem(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("ldx", ctypes.c_int64),
        ("mean", ctypes.c_void_p),
        ("q_row", ctypes.POINTER(CQTensor)),
        ("q_col", ctypes.POINTER(CQTensor)),
        ("q_mean", ctypes.POINTER(CQTensor)),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
    ]


BATCH_MAX = 8


class CColStats(ctypes.Structure):
    _fields_ = [
        ("sum", ctypes.c_void_p),
        ("min", ctypes.c_void_p),
        ("max", ctypes.c_void_p),
        ("capacity", ctypes.c_int64),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("parts", ctypes.c_int64),
        ("part_rows", ctypes.c_int64),
    ]


_lib = None


def is_current() -> bool:
    """True when libaveris.so exists and was built from the sources next to it."""
    from .build import source_digest
    if not os.path.exists(LIB_PATH):
        return False
    L = ctypes.CDLL(LIB_PATH)
    f = L.averis_source_digest
    f.restype = ctypes.c_char_p
    return f().decode() == source_digest()


def lib():
    """Load libaveris.so once; raise if it has not been built, or was built from other sources."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        if not is_current():
            raise RuntimeError(f"{LIB_PATH} was built from other sources than the ones beside it: "
                               "rebuild it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        Q = ctypes.POINTER(CQTensor)
        CS = ctypes.POINTER(CColStats)
        sig = {
            "averis_abi_version": (I32, []),
            "averis_status_string": (ctypes.c_char_p, [I32]),
            "averis_source_digest": (ctypes.c_char_p, []),
            "averis_split_quant_workspace_size": (SZ, [I64, I64, I32, U32]),
            "averis_split_quant": (I32, [P, I32, I64, I64, I64, I32, U32, P, Q, Q, Q, P, SZ, P]),
            "averis_split_quant_sr": (I32, [P, I32, I64, I64, I64, I32, U32, ctypes.c_uint64, P, Q, Q, Q, P, SZ, P]),
            "averis_split_quant_batch": (I32, [I32, ctypes.POINTER(CSplitQuantItem), I32, I32, U32, P]),
            "averis_split_quant_noalloc_max_bytes": (SZ, []),
            "averis_split_quant_noalloc": (I32, [P, I32, I64, I64, I64, I32, U32, P, Q, Q, Q, P]),
            "averis_linear_workspace_size": (SZ, [I64, I64, I64, I32]),
            "averis_linear_fwd": (I32, [Q, Q, Q, P, I32, I64, P, SZ, P]),
            "averis_linear_bwd_dx": (I32, [Q, Q, Q, P, I32, I64, P, SZ, P]),
            "averis_colstats_capacity": (I64, [I64, I64]),
            "averis_linear_fwd_stats": (I32, [Q, Q, Q, P, I32, I64, CS, P, SZ, P]),
            "averis_linear_bwd_dx_stats": (I32, [Q, Q, Q, P, I32, I64, CS, P, SZ, P]),
            "averis_split_quant_stats": (I32, [P, I32, I64, I64, I64, I32, U32, CS, P, Q, Q, Q, P, SZ, P]),
            "averis_rmsnorm_stats": (I32, [P, I32, I64, I64, I64, P, ctypes.c_float, P, I64, CS, P]),
            "averis_swiglu_stats": (I32, [P, P, I32, I64, I64, I64, P, I64, CS, P]),
            "averis_linear_bwd_dw_workspace_size": (SZ, [I64, I64, I64, I32]),
            "averis_linear_bwd_dw": (I32, [Q, Q, Q, Q, I64, P, I64, U32, P, SZ, P]),
            "averis_split_quant_grouped_workspace_size": (SZ, [I64, I64, I32, I32, U32]),
            "averis_split_quant_grouped": (I32, [P, I32, I64, I64, P, P, I32, I32, U32, P, Q, Q, Q, P, SZ, P]),
            "averis_linear_grouped_workspace_size": (SZ, [I64, I32, I32]),
            "averis_linear_fwd_grouped": (I32, [Q, Q, Q, P, P, I32, P, I32, I64, P, SZ, P]),
            "averis_linear_bwd_dx_grouped": (I32, [Q, Q, Q, P, P, I32, P, I32, I64, P, SZ, P]),
            "averis_linear_bwd_dw_grouped_workspace_size": (SZ, [I64, I64, I32, I32]),
            "averis_linear_bwd_dw_grouped": (I32, [Q, Q, Q, Q, P, P, I32, P, I64, U32, P, SZ, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


class AverisError(RuntimeError):
    pass


def _check(status):
    if status != 0:
        raise AverisError(f"averis status {status}: {lib().averis_status_string(status).decode()}")


@dataclass
class QTensor:
    """Device buffers of one quantized operand [outer, k] (blocks along k)."""
    codes: torch.Tensor         # uint8 [outer, k_pad/2]
    scales: torch.Tensor        # uint8, round_up(outer, 32) * k_pad/g bytes, tiled (see include/averis.h)
    tensor_scale: torch.Tensor | None  # fp32 [1] (NVFP4)
    outer: int
    k: int
    fmt: int
    rotated: bool
    kpad: int | None = None  # storage length along k when it is not round_up(k, 256) (grouped)

    @property
    def k_pad(self):
        return self.kpad if self.kpad is not None else (self.k + KPAD - 1) // KPAD * KPAD

    def c(self):
        return CQTensor(self.codes.data_ptr(), self.scales.data_ptr(),
                        self.tensor_scale.data_ptr() if self.tensor_scale is not None else None,
                        self.outer, self.k, self.k_pad, self.fmt, HADAMARD16 if self.rotated else 0)


def empty_qtensor(outer, k, fmt, rotated=False, device="cuda", groups=1, kpad=None):
    kp = kpad if kpad is not None else (k + KPAD - 1) // KPAD * KPAD
    g = BLOCK[fmt]
    rp = (outer + 31) // 32 * 32
    return QTensor(torch.empty((outer, kp // 2), dtype=torch.uint8, device=device),
                   torch.empty((rp, kp // g), dtype=torch.uint8, device=device),
                   torch.empty(groups, dtype=torch.float32, device=device) if fmt == NVFP4 else None,
                   outer, k, fmt, rotated, kpad)


def _ptr(q):
    return ctypes.byref(q.c()) if q is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes, device):
    # zero-filled once: split_quant's workspace carries counters that must start at zero (each
    # call leaves them at zero again)
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def split_quant_outputs(rows, cols, fmt, split=True, hadamard=False, row=True, col=True, device="cuda"):
    """Allocate the outputs of split_quant (for callers that reuse them, e.g. under graph capture)."""
    return dict(mean=torch.empty(cols, dtype=torch.float32, device=device) if split else None,
                row=empty_qtensor(rows, cols, fmt, hadamard, device) if row else None,
                col=empty_qtensor(cols, rows, fmt, hadamard, device) if col else None,
                mean_q=empty_qtensor(1, cols, fmt, hadamard, device) if split else None)


def split_quant_workspace(rows, cols, fmt, split=True, hadamard=False, device="cuda"):
    flags = (SPLIT if split else 0) | (HADAMARD16 if hadamard else 0)
    return _workspace(lib().averis_split_quant_workspace_size(rows, cols, fmt, flags), device)


def split_quant(x: torch.Tensor, fmt: int, split: bool = True, hadamard: bool = False,
                mean: torch.Tensor | None = None, row: bool = True, col: bool = True, stream=None,
                out=None, ws=None, sr_seed: int | None = None, check_finite: bool = False):
    """Mean, residual and FP4 quantization of x [rows, cols] (bf16 or fp32, row-major).

    Returns dict(mean=fp32 [cols] or None, row=QTensor [rows, cols] or None,
    col=QTensor [cols, rows] or None, mean_q=QTensor [1, cols] or None).
    `mean` given: used instead of the column mean (MEAN_GIVEN).  `out` / `ws`: preallocated
    outputs (from split_quant_outputs) and workspace (from split_quant_workspace).  `sr_seed`:
    stochastic rounding of the E2M1 codes with this 64-bit seed (averis_split_quant_sr).
    `check_finite`: the result also holds "status", a device uint32 [1] view of the workspace's
    status word (AVERIS_STATUS_* bits; read it after the stream reaches the call)."""
    assert x.dim() == 2 and x.is_cuda
    rows, cols = x.shape
    assert rows == 0 or x.stride(1) == 1, "x must be row-major"
    ldx = x.stride(0) if rows > 0 else cols
    dev = x.device
    flags = (SPLIT if split else 0) | (HADAMARD16 if hadamard else 0) | \
        (MEAN_GIVEN if (split and mean is not None) else 0) | (CHECK_FINITE if check_finite else 0)
    if out is None:
        out = split_quant_outputs(rows, cols, fmt, split, hadamard, row, col, dev)
    if split and mean is not None:
        out = dict(out, mean=mean.contiguous())
    mu = out["mean"]
    if ws is None:
        ws = split_quant_workspace(rows, cols, fmt, split, hadamard, dev)
    L = lib()
    xp, dt, mp = x.data_ptr() if rows else None, _dtype_code(x), mu.data_ptr() if mu is not None else None
    if sr_seed is None:
        _check(L.averis_split_quant(xp, dt, rows, cols, ldx, fmt, flags, mp, _ptr(out["row"]), _ptr(out["col"]),
                                    _ptr(out["mean_q"]), ws.data_ptr(), ws.numel(), _stream(stream)))
    else:
        _check(L.averis_split_quant_sr(xp, dt, rows, cols, ldx, fmt, flags, int(sr_seed), mp, _ptr(out["row"]),
                                       _ptr(out["col"]), _ptr(out["mean_q"]), ws.data_ptr(), ws.numel(),
                                       _stream(stream)))
    if check_finite:
        out = dict(out, status=ws[:4].view(torch.int32))
    return out


def split_quant_batch(xs, fmt: int, split: bool = True, hadamard: bool = False, outs=None, wss=None,
                      row: bool = True, col: bool = True, stream=None):
    """split_quant of up to BATCH_MAX independent tensors xs (one dtype) in one statistics and one
    quantizing launch (averis_split_quant_batch).  Returns one split_quant-style dict per tensor;
    `outs` / `wss`: preallocated outputs and workspaces, one per tensor."""
    n = len(xs)
    assert 1 <= n <= BATCH_MAX
    dev = xs[0].device
    flags = (SPLIT if split else 0) | (HADAMARD16 if hadamard else 0)
    if outs is None:
        outs = [split_quant_outputs(x.shape[0], x.shape[1], fmt, split, hadamard, row, col, dev) for x in xs]
    if wss is None:
        wss = [split_quant_workspace(x.shape[0], x.shape[1], fmt, split, hadamard, dev) for x in xs]
    items = (CSplitQuantItem * n)()
    keep = []  # the CQTensor structs the items point to
    for i, (x, o, ws) in enumerate(zip(xs, outs, wss)):
        assert x.dim() == 2 and x.is_cuda and x.dtype == xs[0].dtype
        rows, cols = x.shape
        assert rows == 0 or x.stride(1) == 1, "x must be row-major"
        qs = [o[k].c() if o[k] is not None else None for k in ("row", "col", "mean_q")]
        keep.append(qs)
        ptr = [ctypes.pointer(q) if q is not None else None for q in qs]
        items[i] = CSplitQuantItem(x.data_ptr() if rows else None, rows, cols, x.stride(0) if rows > 0 else cols,
                                   o["mean"].data_ptr() if o["mean"] is not None else None, ptr[0], ptr[1], ptr[2],
                                   ws.data_ptr(), ws.numel())
    _check(lib().averis_split_quant_batch(n, items, _dtype_code(xs[0]), fmt, flags, _stream(stream)))
    return outs


def split_quant_noalloc(x: torch.Tensor, fmt: int, split: bool = True, hadamard: bool = False, out=None,
                        stream=None):
    """split_quant on the library's own device scratch array (no workspace argument): for callers
    that cannot allocate; `out` from split_quant_outputs."""
    assert x.dim() == 2 and x.is_cuda
    rows, cols = x.shape
    assert rows == 0 or x.stride(1) == 1, "x must be row-major"
    ldx = x.stride(0) if rows > 0 else cols
    flags = (SPLIT if split else 0) | (HADAMARD16 if hadamard else 0)
    if out is None:
        out = split_quant_outputs(rows, cols, fmt, split, hadamard, device=x.device)
    mu = out["mean"]
    _check(lib().averis_split_quant_noalloc(x.data_ptr() if rows else None, _dtype_code(x), rows, cols, ldx, fmt,
                                            flags, mu.data_ptr() if mu is not None else None, _ptr(out["row"]),
                                            _ptr(out["col"]), _ptr(out["mean_q"]), _stream(stream)))
    return out


def linear_workspace(a: QTensor, w: QTensor):
    return _workspace(lib().averis_linear_workspace_size(a.outer, w.outer, a.k_pad, a.fmt), a.codes.device)


def _linear(fn, a: QTensor, mu: QTensor | None, w: QTensor, out_dtype, stream, out, ws):
    dev = a.codes.device
    if out is None:
        out = torch.empty((a.outer, w.outer), dtype=out_dtype, device=dev)
    if ws is None:
        ws = linear_workspace(a, w)
    _check(fn(_ptr(a), _ptr(mu), _ptr(w), out.data_ptr() if out.numel() else None, _dtype_code(out), out.stride(0),
              ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


def linear_fwd(xr: QTensor, mu_x: QTensor | None, w: QTensor, out_dtype=torch.float32, stream=None,
               out=None, ws=None):
    """Y [l, n] = 1 (Q(mu_X) Q(W)) + Q(X_R) Q(W); w is the [n, m] (K = m) weight operand."""
    return _linear(lib().averis_linear_fwd, xr, mu_x, w, out_dtype, stream, out, ws)


def linear_bwd_dx(dr: QTensor, mu_d: QTensor | None, w: QTensor, out_dtype=torch.float32, stream=None,
                  out=None, ws=None):
    """dX [l, m] = 1 (Q(mu_D) Q(W)^T) + Q(D_R) Q(W)^T; w is the [m, n] (K = n) weight operand."""
    return _linear(lib().averis_linear_bwd_dx, dr, mu_d, w, out_dtype, stream, out, ws)


class ColStats:
    """Caller-owned column partials of a GEMM output (averis_colstats): fp32 sums, and minima /
    maxima when `minmax`, sized for any producer of a [rows, cols] output.  The producer fills in
    rows, cols, parts and part_rows."""

    def __init__(self, rows, cols, minmax=False, device="cuda"):
        cap = int(lib().averis_colstats_capacity(rows, cols))
        mk = lambda: torch.empty(max(cap, 1), dtype=torch.float32, device=device)  # noqa: E731
        self.sum = mk()
        self.min = mk() if minmax else None
        self.max = mk() if minmax else None
        self.cs = CColStats(self.sum.data_ptr(), self.min.data_ptr() if minmax else None,
                            self.max.data_ptr() if minmax else None, cap, 0, 0, 0, 0)

    @property
    def parts(self):
        return self.cs.parts

    @property
    def part_rows(self):
        return self.cs.part_rows

    def view(self, which="sum"):
        """The written partials [parts, cols] of `which` ('sum', 'min' or 'max')."""
        t = getattr(self, which)
        return t[: self.cs.parts * self.cs.cols].view(self.cs.parts, self.cs.cols)


def _linear_stats(fn, a: QTensor, mu: QTensor | None, w: QTensor, stats: ColStats, out_dtype, stream, out, ws):
    dev = a.codes.device
    if out is None:
        out = torch.empty((a.outer, w.outer), dtype=out_dtype, device=dev)
    if ws is None:
        ws = linear_workspace(a, w)
    _check(fn(_ptr(a), _ptr(mu), _ptr(w), out.data_ptr() if out.numel() else None, _dtype_code(out), out.stride(0),
              ctypes.byref(stats.cs), ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


def linear_fwd_stats(xr: QTensor, mu_x: QTensor | None, w: QTensor, stats: ColStats, out_dtype=torch.bfloat16,
                     stream=None, out=None, ws=None):
    """linear_fwd that also writes the column statistics of Y (as stored) into `stats`."""
    return _linear_stats(lib().averis_linear_fwd_stats, xr, mu_x, w, stats, out_dtype, stream, out, ws)


def linear_bwd_dx_stats(dr: QTensor, mu_d: QTensor | None, w: QTensor, stats: ColStats, out_dtype=torch.bfloat16,
                        stream=None, out=None, ws=None):
    """linear_bwd_dx that also writes the column statistics of dX (as stored) into `stats`."""
    return _linear_stats(lib().averis_linear_bwd_dx_stats, dr, mu_d, w, stats, out_dtype, stream, out, ws)


def rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, stats: ColStats | None = None, out=None,
            stream=None):
    """RMSNorm of x [rows, cols] (bf16 or fp32) with fp32 weight [cols]; writes the column
    statistics of the output into `stats` when given."""
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1 and weight.dtype == torch.float32
    rows, cols = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().averis_rmsnorm_stats(x.data_ptr() if rows else None, _dtype_code(x), rows, cols,
                                      x.stride(0) if rows else cols, weight.data_ptr(), float(eps),
                                      out.data_ptr() if rows else None, out.stride(0) if rows else cols,
                                      ctypes.byref(stats.cs) if stats is not None else None, _stream(stream)))
    return out


def swiglu(gate: torch.Tensor, up: torch.Tensor, stats: ColStats | None = None, out=None, stream=None):
    """silu(gate) * up for gate, up [rows, cols] (same dtype and strides); writes the column
    statistics of the output into `stats` when given."""
    assert gate.shape == up.shape and gate.dtype == up.dtype and gate.stride() == up.stride()
    assert gate.dim() == 2 and gate.is_cuda and gate.stride(1) == 1
    rows, cols = gate.shape
    if out is None:
        out = torch.empty_like(gate)
    _check(lib().averis_swiglu_stats(gate.data_ptr() if rows else None, up.data_ptr() if rows else None,
                                     _dtype_code(gate), rows, cols, gate.stride(0) if rows else cols,
                                     out.data_ptr() if rows else None, out.stride(0) if rows else cols,
                                     ctypes.byref(stats.cs) if stats is not None else None, _stream(stream)))
    return out


def split_quant_stats(x: torch.Tensor, stats: ColStats, fmt: int, hadamard: bool = False, row: bool = True,
                      col: bool = True, stream=None, out=None, ws=None, check_finite: bool = False):
    """split_quant (SPLIT) of x from the column statistics its producer wrote into `stats`;
    returns the same dict as split_quant."""
    assert x.dim() == 2 and x.is_cuda
    rows, cols = x.shape
    assert rows == 0 or x.stride(1) == 1, "x must be row-major"
    ldx = x.stride(0) if rows > 0 else cols
    dev = x.device
    flags = SPLIT | (HADAMARD16 if hadamard else 0) | (CHECK_FINITE if check_finite else 0)
    if out is None:
        out = split_quant_outputs(rows, cols, fmt, True, hadamard, row, col, dev)
    if ws is None:
        ws = split_quant_workspace(rows, cols, fmt, True, hadamard, dev)
    _check(lib().averis_split_quant_stats(x.data_ptr() if rows else None, _dtype_code(x), rows, cols, ldx, fmt, flags,
                                          ctypes.byref(stats.cs), out["mean"].data_ptr(), _ptr(out["row"]),
                                          _ptr(out["col"]), _ptr(out["mean_q"]), ws.data_ptr(), ws.numel(),
                                          _stream(stream)))
    if check_finite:
        out = dict(out, status=ws[:4].view(torch.int32))
    return out


def linear_bwd_dw_workspace(xr_t: QTensor, dr_t: QTensor, l: int):
    return _workspace(lib().averis_linear_bwd_dw_workspace_size(xr_t.outer, dr_t.outer, l, xr_t.fmt),
                      xr_t.codes.device)


def linear_bwd_dw(xr_t: QTensor, dr_t: QTensor, mu_x: QTensor | None, mu_d: QTensor | None, l: int,
                  dw: torch.Tensor | None = None, accumulate: bool = False, stream=None, ws=None):
    """dW [m, n] = Q(X_R)^T Q(D_R) + l Q(mu_X)^T Q(mu_D) (fp32), optionally accumulated into dw."""
    dev = xr_t.codes.device
    if dw is None:
        dw = torch.empty((xr_t.outer, dr_t.outer), dtype=torch.float32, device=dev)
    if ws is None:
        ws = linear_bwd_dw_workspace(xr_t, dr_t, l)
    L = lib()
    _check(L.averis_linear_bwd_dw(_ptr(xr_t), _ptr(dr_t), _ptr(mu_x), _ptr(mu_d), l,
                                  dw.data_ptr() if dw.numel() else None, dw.stride(0),
                                  ACCUMULATE if accumulate else 0, ws.data_ptr(), ws.numel(), _stream(stream)))
    return dw


# ------------------------------------------------------------------------------------------
# Grouped (MoE) variants: group e = rows [offsets[e], offsets[e+1]) of a token-major input.
# ------------------------------------------------------------------------------------------
def _ru(a, b):
    return (a + b - 1) // b * b


class Groups:
    """Group offsets [E + 1] kept on the device (read by the kernels) and on the host (launch
    sizing); plus the sizes of the grouped layouts."""

    def __init__(self, offsets, device="cuda"):
        offs = [int(v) for v in offsets]
        self.offsets = offs
        self.E = len(offs) - 1
        self.lens = [offs[e + 1] - offs[e] for e in range(self.E)]
        self.rows = offs[-1]
        self.row_starts = [0]
        self.tok_starts = [0]
        for n in self.lens:
            self.row_starts.append(self.row_starts[-1] + _ru(n, 32))
            self.tok_starts.append(self.tok_starts[-1] + _ru(n, KPAD))
        self.rows32 = self.row_starts[-1]
        self.tok256 = self.tok_starts[-1]
        self.h = (ctypes.c_int64 * (self.E + 1))(*offs)
        self.d = torch.tensor(offs, dtype=torch.int64, device=device)


def split_quant_grouped_outputs(grp: Groups, cols, fmt, split=True, hadamard=False, row=True, col=True,
                                device="cuda"):
    E = grp.E
    return dict(mean=torch.empty((E, cols), dtype=torch.float32, device=device) if split else None,
                row=empty_qtensor(grp.rows32, cols, fmt, hadamard, device, groups=E) if row else None,
                col=empty_qtensor(cols, grp.rows, fmt, hadamard, device, groups=E, kpad=grp.tok256) if col else None,
                mean_q=empty_qtensor(E, cols, fmt, hadamard, device, groups=E) if split else None)


def split_quant_grouped(x: torch.Tensor, grp: Groups, fmt: int, split: bool = True, hadamard: bool = False,
                        means: torch.Tensor | None = None, row: bool = True, col: bool = True, stream=None,
                        out=None, ws=None):
    """Per group, exactly split_quant on its rows; outputs in the grouped layouts of
    include/averis.h (row layout [sum round_up(l_e, 32), cols], column layout [cols, L] with
    per-group token padding, means [E, cols], quantized means [E, cols], one tensor scale per
    group)."""
    assert x.dim() == 2 and x.is_cuda and x.shape[0] == grp.rows
    rows, cols = x.shape
    assert rows == 0 or x.stride(1) == 1, "x must be row-major"
    ldx = x.stride(0) if rows > 0 else cols
    dev = x.device
    flags = (SPLIT if split else 0) | (HADAMARD16 if hadamard else 0) | \
        (MEAN_GIVEN if (split and means is not None) else 0)
    if out is None:
        out = split_quant_grouped_outputs(grp, cols, fmt, split, hadamard, row, col, dev)
    if split and means is not None:
        out = dict(out, mean=means.contiguous())
    mu = out["mean"]
    L = lib()
    if ws is None:
        ws = _workspace(L.averis_split_quant_grouped_workspace_size(rows, cols, grp.E, fmt, flags), dev)
    _check(L.averis_split_quant_grouped(x.data_ptr() if rows else None, _dtype_code(x), cols, ldx,
                                        grp.d.data_ptr(), grp.h, grp.E, fmt, flags,
                                        mu.data_ptr() if mu is not None else None, _ptr(out["row"]),
                                        _ptr(out["col"]), _ptr(out["mean_q"]), ws.data_ptr(), ws.numel(),
                                        _stream(stream)))
    return out


def split_quant_grouped_workspace(rows, cols, E, fmt, split=True, hadamard=False, device="cuda"):
    flags = (SPLIT if split else 0) | (HADAMARD16 if hadamard else 0)
    return _workspace(lib().averis_split_quant_grouped_workspace_size(rows, cols, E, fmt, flags), device)


def linear_grouped_workspace(N, E, fmt, device="cuda"):
    """Workspace of a grouped forward or input-gradient GEMM with N output columns per group."""
    return _workspace(lib().averis_linear_grouped_workspace_size(N, E, fmt), device)


def linear_bwd_dw_grouped_workspace(m, n, E, fmt, device="cuda"):
    return _workspace(lib().averis_linear_bwd_dw_grouped_workspace_size(m, n, E, fmt), device)


def stacked_weight_view(col_q: QTensor, E: int, m: int) -> QTensor:
    """The column layout of grouped weights (E groups of m rows, outer = n) seen as E stacked
    [n, m] operands (outer = E * n): the same bytes, the forward GEMM's B operand."""
    n = col_q.outer
    kp = _ru(m, KPAD)
    return QTensor(col_q.codes.view(-1).view(E * n, kp // 2), col_q.scales.view(-1).view(E * n, kp // BLOCK[col_q.fmt]),
                   col_q.tensor_scale, E * n, m, col_q.fmt, col_q.rotated)


def _linear_grouped(fn, a: QTensor, mu: QTensor | None, w: QTensor, grp: Groups, out_dtype, stream, out, ws):
    dev = a.codes.device
    N = w.outer // grp.E
    if out is None:
        out = torch.empty((grp.rows, N), dtype=out_dtype, device=dev)
    if ws is None:
        ws = _workspace(lib().averis_linear_grouped_workspace_size(N, grp.E, a.fmt), dev)
    _check(fn(_ptr(a), _ptr(mu), _ptr(w), grp.d.data_ptr(), grp.h, grp.E, out.data_ptr() if out.numel() else None,
              _dtype_code(out), out.stride(0), ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


def linear_fwd_grouped(xr: QTensor, mu_x: QTensor | None, w: QTensor, grp: Groups, out_dtype=torch.float32,
                       stream=None, out=None, ws=None):
    """Y [L, n]: per group the forward GEMM with its own mean term; w = E stacked [n, m] operands."""
    return _linear_grouped(lib().averis_linear_fwd_grouped, xr, mu_x, w, grp, out_dtype, stream, out, ws)


def linear_bwd_dx_grouped(dr: QTensor, mu_d: QTensor | None, w: QTensor, grp: Groups, out_dtype=torch.float32,
                          stream=None, out=None, ws=None):
    """dX [L, m]: per group the input-gradient GEMM; w = E stacked [m, n] operands."""
    return _linear_grouped(lib().averis_linear_bwd_dx_grouped, dr, mu_d, w, grp, out_dtype, stream, out, ws)


def linear_bwd_dw_grouped(xr_t: QTensor, dr_t: QTensor, mu_x: QTensor | None, mu_d: QTensor | None, grp: Groups,
                          dw: torch.Tensor | None = None, accumulate: bool = False, stream=None, ws=None):
    """dW [E, m, n] (fp32): per group Q(X_R)^T Q(D_R) + l_e Q(mu_X)^T Q(mu_D)."""
    dev = xr_t.codes.device
    m, n = xr_t.outer, dr_t.outer
    if dw is None:
        dw = torch.empty((grp.E, m, n), dtype=torch.float32, device=dev)
    L = lib()
    if ws is None:
        ws = _workspace(L.averis_linear_bwd_dw_grouped_workspace_size(m, n, grp.E, xr_t.fmt), dev)
    _check(L.averis_linear_bwd_dw_grouped(_ptr(xr_t), _ptr(dr_t), _ptr(mu_x), _ptr(mu_d), grp.d.data_ptr(), grp.h,
                                          grp.E, dw.data_ptr() if dw.numel() else None, dw.stride(1),
                                          ACCUMULATE if accumulate else 0, ws.data_ptr(), ws.numel(),
                                          _stream(stream)))
    return dw
