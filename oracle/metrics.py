"""Error measures used to compare a result against the oracle.

Tolerance of the linear layer's output: relative L2 error <= 2e-3, and per
element |y - y_ref| <= 1e-2 * ||x_m||_2 * max|w| / sqrt(K), where ||x_m|| is
the L2 norm of the row of activations the element belongs to and max|w| is
taken over the layer's dequantized weights.
"""
import numpy as np


def rel_l2(y, y_ref):
    y = np.asarray(y, np.float64)
    r = np.asarray(y_ref, np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(y - r) / den) if den > 0 else float(
        np.linalg.norm(y - r))


def maxabs_bound(x64, wmax, K):
    """Per-row bound [M, 1]."""
    xn = np.linalg.norm(np.asarray(x64, np.float64), axis=1, keepdims=True)
    return 1e-2 * xn * float(wmax) / np.sqrt(K)


def snr_db(w_ref, w):
    w_ref = np.asarray(w_ref, np.float64)
    e = w_ref - np.asarray(w, np.float64)
    return float(10.0 * np.log10(np.sum(w_ref ** 2) / np.sum(e ** 2)))
