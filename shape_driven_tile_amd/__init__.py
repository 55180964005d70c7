"""sdt: fp16 GEMM (C = A.B, fp32 accumulate, fp16 out) and M=1 decode GEMV
for AMD Instinct MI355X (gfx950), behind a small C ABI (``include/sdt.h``).

The compute entry points live in :mod:`shape_driven_tile_amd.binding`, a thin
ctypes layer over ``libsdt.so``; importing this package does not load the
library, so host-only tools (the input generators) work without it.
"""
__all__ = ["binding", "inputs"]
