"""The quantized linear layer's result, by its plain definition:

    y[m, n] = sum_k x[m, k] * w[n, k]  (+ bias[n])

with w the exact (fp64) dequantized weight, x the exact value of the
activations, and the sum taken in fp64 by a library matmul.  W is [N, K]
and the product is x @ W^T (the "_t" of the Metal page's affine_qmm_t).
"""
import numpy as np

from .dequant import dequant_f64
from .formats import QFormat


def linear_f64(x64, qz, f: QFormat, bias64=None, w64=None):
    """x64: [M, K] fp64; returns y [M, N] fp64."""
    if w64 is None:
        w64 = dequant_f64(qz, f)
    y = np.matmul(np.asarray(x64, np.float64), w64.T)
    if bias64 is not None:
        y = y + np.asarray(bias64, np.float64)[None, :]
    return y

