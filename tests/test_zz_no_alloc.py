"""averis_split_quant_noalloc (the library's own device scratch array, no workspace argument)
against averis_split_quant with a caller workspace: the same kernels, so means, codes, block
scales and tensor scales must be identical.  Two calls in a row, the second on a smaller input
(the array keeps the first call's contents), then a size beyond the array is refused."""
import numpy as np
import pytest
import torch

import fp4_quantized_amd.averis as av
from fp4_quantized_amd import workloads
from tests.gpu_util import device

pytestmark = pytest.mark.gpu


def same(a, b, what):
    for k in ("row", "col", "mean_q"):
        if a[k] is None:
            assert b[k] is None, what
            continue
        assert torch.equal(a[k].codes, b[k].codes), f"{what}: {k} codes"
        assert torch.equal(a[k].scales, b[k].scales), f"{what}: {k} scales"
        if a[k].tensor_scale is not None:
            assert torch.equal(a[k].tensor_scale, b[k].tensor_scale), f"{what}: {k} tensor scale"
    if a["mean"] is not None:
        assert torch.equal(a["mean"], b["mean"]), f"{what}: mean"


def test_noalloc_matches_workspace_entry_point_two_calls():
    dev = device()
    cases = [(workloads.up_proj_like(81, 8192, 1024, 8).x, av.MXFP4, True, False, "8192x1024-mxfp4"),
             (workloads.up_proj_like(82, 300, 256, 8).x, av.NVFP4, True, True, "300x256-nvfp4-h16"),
             (workloads.up_proj_like(83, 77, 96, 8).x, av.NVFP4, False, False, "77x96-nvfp4-vanilla")]
    for x_np, fmt, split, h16, tag in cases:
        print(f"case noalloc {tag}", flush=True)
        x = workloads.to_torch(x_np, "bf16", dev)
        got = av.split_quant_noalloc(x, fmt, split, h16)
        ref = av.split_quant(x, fmt, split, h16)
        torch.cuda.synchronize()
        same(got, ref, tag)


def test_noalloc_refuses_sizes_beyond_its_array():
    dev = device()
    L = av.lib()
    limit = L.averis_split_quant_noalloc_max_bytes()
    rows, cols = 1 << 20, 8192
    assert L.averis_split_quant_workspace_size(rows, cols, av.MXFP4, av.SPLIT) > limit
    x = torch.empty((1, cols), dtype=torch.bfloat16, device=dev)  # never read: the call is refused first
    out = av.split_quant_outputs(1, cols, av.MXFP4, True, device=dev)
    st = L.averis_split_quant_noalloc(x.data_ptr(), av.BF16, rows, cols, cols, av.MXFP4, av.SPLIT,
                                      out["mean"].data_ptr(), av._ptr(out["row"]), av._ptr(out["col"]),
                                      av._ptr(out["mean_q"]), av._stream())
    assert st == 7, f"status {st}"  # AVERIS_E_WORKSPACE
