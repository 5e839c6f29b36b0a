"""C-ABI boundary checks that need no GPU: the library loads, exports every function that
include/averis.h declares, and rejects bad arguments with the documented status before
enqueuing anything (these calls return before any HIP runtime call)."""
import ctypes
import os
import re
import subprocess

import pytest

import fp4_quantized_amd.averis as av

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "averis.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_FORMAT, E_FLAGS, E_WORKSPACE = range(8)
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced by the validation paths


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(averis_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 9
    nm = subprocess.run(["nm", "-D", "--defined-only", av.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (averis_\w+)", nm))
    assert set(names) <= exported, set(names) - exported
    assert set(names) == set(av.EXPORTS)
    L = av.lib()
    for n in names:
        assert hasattr(L, n)


def test_abi_version_and_status_strings():
    L = av.lib()
    assert L.averis_abi_version() == 1
    for s in range(9):
        assert L.averis_status_string(s)
    assert L.averis_status_string(0) == b"ok"


def q(outer, k, fmt=av.NVFP4, flags=0, codes=FAKE, scales=FAKE, ts=FAKE):
    kp = (k + 255) // 256 * 256
    return av.CQTensor(codes, scales, ts, outer, k, kp, fmt, flags)


def split(x=FAKE, xdt=av.BF16, rows=256, cols=128, ldx=128, fmt=av.NVFP4, flags=av.SPLIT, mean=FAKE,
          q_row="auto", q_col="auto", q_mean="auto", ws=FAKE, ws_bytes=1 << 30):
    L = av.lib()
    if q_row == "auto":
        q_row = q(rows, cols, fmt, flags & av.HADAMARD16)
    if q_col == "auto":
        q_col = q(cols, rows, fmt, flags & av.HADAMARD16)
    if q_mean == "auto":
        q_mean = q(1, cols, fmt, flags & av.HADAMARD16) if flags & av.SPLIT else None
    ref = lambda t: ctypes.byref(t) if t is not None else None
    return L.averis_split_quant(x, xdt, rows, cols, ldx, fmt, flags, mean, ref(q_row), ref(q_col), ref(q_mean),
                                ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(xdt=7), E_DTYPE),
    (dict(fmt=3), E_FORMAT),
    (dict(flags=1 << 9), E_FLAGS),
    (dict(flags=av.MEAN_GIVEN), E_FLAGS),
    (dict(cols=100, ldx=100), E_SHAPE),
    (dict(cols=48, ldx=48), E_SHAPE),
    (dict(ldx=64), E_SHAPE),
    (dict(rows=-1), E_SHAPE),
    (dict(x=None), E_NULL),
    (dict(x=FAKE + 4), E_ALIGN),
    (dict(ldx=130), E_ALIGN),
    (dict(q_row=None, q_col=None), E_NULL),
    (dict(mean=None), E_NULL),
    (dict(q_mean=None), E_NULL),
    (dict(flags=0, q_mean=q(1, 128)), E_FLAGS),
    (dict(ws=None), E_WORKSPACE),
    (dict(ws_bytes=16), E_WORKSPACE),
    (dict(q_row=q(255, 128)), E_SHAPE),
    (dict(q_col=q(128, 256, av.MXFP4)), E_FORMAT),
    (dict(q_row=q(256, 128, av.NVFP4, av.HADAMARD16)), E_FLAGS),
    (dict(q_row=q(256, 128, ts=None)), E_NULL),
    (dict(q_row=q(256, 128, codes=FAKE + 8)), E_ALIGN),
])
def test_split_quant_rejects(kw, status):
    assert split(**kw) == status


def test_split_quant_workspace_size():
    # column statistics of 512-row slabs: psum fp64 + min, max fp32 per slab and column, plus
    # one arrival counter and two partial maxima per 64-column strip
    L = av.lib()
    assert L.averis_split_quant_workspace_size(8192, 1024, av.NVFP4, av.SPLIT) >= 16 * 1024 * 16 + 16 * 12
    assert L.averis_split_quant_workspace_size(0, 1024, av.NVFP4, av.SPLIT) > 0
    assert L.averis_split_quant_workspace_size(-1, 1024, av.NVFP4, av.SPLIT) == 0


def lin(fn, a, mu, w, out=FAKE, odt=av.F32, ldo=None, ws=FAKE, wsb=1 << 30):
    ref = lambda t: ctypes.byref(t) if t is not None else None
    ldo = w.outer if ldo is None else ldo
    return fn(ref(a), ref(mu), ref(w), out, odt, ldo, ws, wsb, None)


@pytest.mark.parametrize("case,status", [
    ("mixed_fmt", E_FORMAT), ("k_mismatch", E_SHAPE), ("rot_mismatch", E_FLAGS), ("mu_shape", E_SHAPE),
    ("bad_dtype", E_DTYPE), ("small_ld", E_SHAPE), ("huge_ld", E_SHAPE), ("null_out", E_NULL),
    ("no_ws", E_WORKSPACE), ("bad_kpad", E_SHAPE),
])
def test_linear_rejects(case, status):
    L = av.lib()
    a, mu, w = q(256, 512), q(1, 512), q(384, 512)
    kw = {}
    if case == "mixed_fmt":
        w = q(384, 512, av.MXFP4)
    elif case == "k_mismatch":
        w = q(384, 256)
    elif case == "rot_mismatch":
        w = q(384, 512, flags=av.HADAMARD16)
    elif case == "mu_shape":
        mu = q(2, 512)
    elif case == "bad_dtype":
        kw["odt"] = 9
    elif case == "small_ld":
        kw["ldo"] = 100
    elif case == "huge_ld":
        kw["ldo"] = 1 << 23  # output offsets of a wave's 64 rows must stay below 2^31 bytes
    elif case == "null_out":
        kw["out"] = None
    elif case == "no_ws":
        kw["ws"] = None
    elif case == "bad_kpad":
        a = av.CQTensor(FAKE, FAKE, FAKE, 256, 512, 640, av.NVFP4, 0)
    for fn in (L.averis_linear_fwd, L.averis_linear_bwd_dx):
        assert lin(fn, a, mu, w, **kw) == status


def test_bwd_dw_rejects():
    L = av.lib()
    ref = ctypes.byref
    xr, dr, mx, md = q(512, 300), q(384, 300), q(1, 512), q(1, 384)
    call = lambda xr=xr, dr=dr, mx=mx, md=md, l=300, dw=FAKE, ld=384, fl=0, ws=FAKE, wsb=1 << 30: \
        L.averis_linear_bwd_dw(ref(xr), ref(dr), ref(mx) if mx else None, ref(md) if md else None, l, dw, ld, fl, ws,
                               wsb, None)
    assert call(fl=1 << 3) == E_FLAGS
    assert call(l=299) == E_SHAPE
    assert call(md=None) == E_NULL
    assert call(mx=q(1, 500)) == E_SHAPE
    assert call(ld=100) == E_SHAPE
    assert call(ld=1 << 23) == E_SHAPE
    assert call(dw=None) == E_NULL
    assert call(wsb=100) == E_WORKSPACE
    assert call(dr=q(384, 300, av.MXFP4)) == E_FORMAT
    assert L.averis_linear_bwd_dw_workspace_size(512, 384, 300, av.NVFP4) > 0


def offs(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_split_quant_grouped_rejects():
    L = av.lib()
    ref = ctypes.byref
    h = offs(0, 37, 37, 100)  # E = 3, row layout 64 + 0 + 64 rows, tokens 256 + 0 + 256
    E, cols = 3, 128

    def call(x=FAKE, h=h, E=E, d=FAKE, q_row="auto", q_col="auto", q_mean="auto", flags=av.SPLIT, means=FAKE,
             ws=FAKE, wsb=1 << 30):
        if q_row == "auto":
            q_row = q(128, cols)
        if q_col == "auto":
            q_col = av.CQTensor(FAKE, FAKE, FAKE, cols, 100, 512, av.NVFP4, 0)
        if q_mean == "auto":
            q_mean = q(E, cols)
        r = lambda t: ref(t) if t is not None else None
        return L.averis_split_quant_grouped(x, av.BF16, cols, cols, d, h, E, av.NVFP4, flags, means, r(q_row),
                                            r(q_col), r(q_mean), ws, wsb, None)

    assert call(E=0) == E_SHAPE
    assert call(d=None) == E_NULL
    assert call(h=offs(1, 37, 37, 100)) == E_SHAPE          # offsets must start at 0
    assert call(h=offs(0, 37, 30, 100)) == E_SHAPE          # and never decrease
    assert call(q_row=q(100, cols)) == E_SHAPE              # rows are padded per group to 32
    assert call(q_col=q(cols, 100)) == E_SHAPE              # tokens are padded per group to 256
    assert call(q_mean=q(1, cols)) == E_SHAPE               # one mean row per group
    assert call(means=None) == E_NULL
    assert call(wsb=16) == E_WORKSPACE
    assert L.averis_split_quant_grouped_workspace_size(100, cols, E, av.NVFP4, av.SPLIT) > 0
    assert L.averis_split_quant_grouped_workspace_size(100, cols, 0, av.NVFP4, av.SPLIT) == 0


def test_linear_grouped_rejects():
    L = av.lib()
    ref = ctypes.byref
    h = offs(0, 37, 37, 100)
    E, m, n = 3, 256, 128
    a, mu, w = q(128, m), q(E, m), q(E * n, m)

    def call(a=a, mu=mu, w=w, h=h, d=FAKE, out=FAKE, ldo=n, wsb=1 << 30):
        r = lambda t: ref(t) if t is not None else None
        return L.averis_linear_fwd_grouped(r(a), r(mu), r(w), d, h, E, out, av.F32, ldo, FAKE, wsb, None)

    assert call(a=q(100, m)) == E_SHAPE        # grouped row layout has 32-row padded groups
    assert call(w=q(E * n + 32, m)) == E_SHAPE  # weights stack E equal groups
    assert call(w=q(E * 80, m)) == E_SHAPE      # each group a multiple of 32 rows
    assert call(mu=q(1, m)) == E_SHAPE
    assert call(d=None) == E_NULL
    assert call(out=None) == E_NULL
    assert call(ldo=64) == E_SHAPE
    assert call(wsb=16) == E_WORKSPACE
    xt = av.CQTensor(FAKE, FAKE, FAKE, m, 100, 512, av.NVFP4, 0)
    dt = av.CQTensor(FAKE, FAKE, FAKE, n, 100, 512, av.NVFP4, 0)
    dw = lambda xt=xt, dt=dt, mx=q(E, m), md=q(E, n), fl=0: L.averis_linear_bwd_dw_grouped(
        ref(xt), ref(dt), ref(mx) if mx else None, ref(md) if md else None, FAKE, h, E, FAKE, n, fl, FAKE, 1 << 30, None)
    assert dw(fl=1 << 3) == E_FLAGS
    assert dw(dt=av.CQTensor(FAKE, FAKE, FAKE, n, 100, 256, av.NVFP4, 0)) == E_SHAPE
    assert dw(md=None) == E_NULL
    assert dw(mx=q(1, m)) == E_SHAPE


def test_check_finite_flag_rules():
    L = av.lib()
    # unknown flag bits are still refused; the allocation-free variant refuses CHECK_FINITE (its
    # status word would sit in the library's hidden array), before touching any device
    assert split(flags=av.SPLIT | (1 << 6)) == E_FLAGS
    q = lambda o, k: av.CQTensor(FAKE, FAKE, FAKE, o, k, (k + 255) // 256 * 256, av.NVFP4, 0)
    r = ctypes.byref
    st = L.averis_split_quant_noalloc(FAKE, av.BF16, 256, 128, 128, av.NVFP4, av.SPLIT | av.CHECK_FINITE, FAKE,
                                      r(q(256, 128)), r(q(128, 256)), r(q(1, 128)), None)
    assert st == E_FLAGS


def colstats(rows=256, cols=128, parts=4, part_rows=64, minmax=True, capacity=None):
    cap = parts * cols if capacity is None else capacity
    return av.CColStats(FAKE, FAKE if minmax else None, FAKE if minmax else None, cap, rows, cols, parts, part_rows)


def split_stats(st, rows=256, cols=128, fmt=av.NVFP4, flags=av.SPLIT, mean=FAKE):
    L = av.lib()
    h = flags & av.HADAMARD16
    return L.averis_split_quant_stats(FAKE, av.BF16, rows, cols, cols, fmt, flags,
                                      ctypes.byref(st) if st is not None else None, mean,
                                      ctypes.byref(q(rows, cols, fmt, h)), ctypes.byref(q(cols, rows, fmt, h)),
                                      ctypes.byref(q(1, cols, fmt, h)), FAKE, 1 << 30, None)


@pytest.mark.parametrize("case,status", [
    ("no_stats", E_NULL), ("no_split", E_FLAGS), ("mean_given", E_FLAGS), ("no_sum", E_NULL),
    ("half_minmax", E_NULL), ("nvfp4_needs_minmax", E_NULL), ("rows", E_SHAPE), ("cols", E_SHAPE),
    ("parts", E_SHAPE), ("capacity", E_SHAPE), ("part_rows", E_SHAPE),
])
def test_split_quant_stats_rejects(case, status):
    st, kw = colstats(), {}
    if case == "no_stats":
        st = None
    elif case == "no_split":
        kw["flags"] = 0
    elif case == "mean_given":
        kw["flags"] = av.SPLIT | av.MEAN_GIVEN
    elif case == "no_sum":
        st.sum = None
    elif case == "half_minmax":
        st.max = None
    elif case == "nvfp4_needs_minmax":
        st = colstats(minmax=False)
    elif case == "rows":
        st.rows = 255
    elif case == "cols":
        st.cols = 96
    elif case == "parts":
        st.parts = 3
    elif case == "capacity":
        st.capacity = 3 * 128
    elif case == "part_rows":
        st = colstats(part_rows=0, parts=0)
    assert split_stats(st, **kw) == status


def test_split_quant_stats_minmax_rules():
    # minima and maxima are required only for NVFP4 without the Hadamard: with sums alone, MXFP4
    # and NVFP4 with the Hadamard pass that check and are refused on the mismatched row count
    assert split_stats(colstats(minmax=False), fmt=av.NVFP4, flags=av.SPLIT) == E_NULL
    assert split_stats(colstats(minmax=False, rows=255), fmt=av.MXFP4) == E_SHAPE
    assert split_stats(colstats(minmax=False, rows=255), fmt=av.NVFP4, flags=av.SPLIT | av.HADAMARD16) == E_SHAPE


def test_linear_stats_rejects():
    L = av.lib()
    a, mu, w = q(256, 512), q(1, 512), q(384, 512)
    r = ctypes.byref
    assert L.averis_colstats_capacity(256, 384) == 4 * 384
    assert L.averis_colstats_capacity(257, 384) == 5 * 384
    assert L.averis_colstats_capacity(-1, 384) == 0
    for fn in (L.averis_linear_fwd_stats, L.averis_linear_bwd_dx_stats):
        assert fn(r(a), r(mu), r(w), FAKE, av.BF16, 384, None, FAKE, 1 << 30, None) == E_NULL
        small = colstats(rows=256, cols=384, parts=3)
        assert fn(r(a), r(mu), r(w), FAKE, av.BF16, 384, r(small), FAKE, 1 << 30, None) == E_SHAPE
        half = colstats(rows=256, cols=384)
        half.min = None
        assert fn(r(a), r(mu), r(w), FAKE, av.BF16, 384, r(half), FAKE, 1 << 30, None) == E_NULL
        # the plain checks come first
        assert fn(r(a), r(mu), r(q(384, 256)), FAKE, av.BF16, 384, r(colstats(cols=384)), FAKE, 1 << 30,
                  None) == E_SHAPE


def batch_items(n, ws_step=1 << 30, bad=None, fmt=av.NVFP4, flags=av.SPLIT):
    """n valid items on distinct fake workspaces; item `bad` gets cols = 48 (not a multiple of 32)."""
    items = (av.CSplitQuantItem * n)()
    keep = []
    for i in range(n):
        rows, cols = 256, (48 if i == bad else 128)
        qs = [q(rows, cols, fmt), q(cols, rows, fmt), q(1, cols, fmt) if flags & av.SPLIT else None]
        keep.append(qs)
        ptr = [ctypes.pointer(t) if t is not None else None for t in qs]
        items[i] = av.CSplitQuantItem(FAKE, rows, cols, cols, FAKE, ptr[0], ptr[1], ptr[2], FAKE + i * ws_step, 1 << 30)
    return items, keep


@pytest.mark.parametrize("case,status", [
    ("n0", E_SHAPE), ("n9", E_SHAPE), ("null", E_NULL), ("check_finite", E_FLAGS), ("bad_item", E_SHAPE),
    ("shared_ws", E_WORKSPACE), ("mean_given_without_split", E_FLAGS),
])
def test_split_quant_batch_rejects(case, status):
    # every case fails validation before anything is enqueued (the pointers are never used)
    L = av.lib()
    n = 9 if case == "n9" else 3
    items, keep = batch_items(n, ws_step=(0 if case == "shared_ws" else 1 << 32), bad=(1 if case == "bad_item" else None))
    flags = {"check_finite": av.SPLIT | av.CHECK_FINITE, "mean_given_without_split": av.MEAN_GIVEN}.get(case, av.SPLIT)
    arg_n = 0 if case == "n0" else n
    arg_items = None if case == "null" else items
    assert L.averis_split_quant_batch(arg_n, arg_items, av.BF16, av.NVFP4, flags, None) == status
