"""MI355X (gfx950) implementation of the Averis mean-residual split before FP4 quantization.

The compute path is the HIP library libaveris.so (C ABI declared in include/averis.h).
`fp4_quantized_amd.averis` is the thin ctypes binding; importing this package loads nothing.
"""
__all__ = ["averis", "workloads"]
