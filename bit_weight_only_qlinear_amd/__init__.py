"""Group-wise weight-only quantized linear layer for MI355X (gfx950).

The compute path is the C-ABI library ``libqlinear.so`` (HIP kernels);
this package only marshals torch tensors into it.  See ``include/qlinear.h``.
"""
