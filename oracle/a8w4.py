"""a8w4: int8 activations times symmetric int4 weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ExecuTorch PR #16577, "Arm backend: Support a8w4 for convolution and
linear", description: 4-bit weights carried in an int8 container with
qmin = -7 and qmax = 7 ("w4"), with 8-bit activations ("a8").  The weight
side is the sym4 format of this oracle (per output channel scale).

The page does not state how the activations are quantized.  Reading taken
here (the plainest one consistent with the symmetric weight rule): per
token, i.e. per row m of x, symmetric int8 with the full range 127:
    s_m = fl32(max_k |x[m, k]| / 127)
    q[m, k] = 0 if s_m == 0 else clamp(rint(fl32(x[m, k] / s_m)), -127, 127)
one IEEE fp32 operation per step, ties to even.  The layer is then
    y[m, n] = s_m * s_n * sum_k q[m, k] * qw[n, k]   (+ bias[n])
with the integer sum exact (int64) and the two scalings in fp64 (relative
error below 2^-52).
"""
import numpy as np

F32 = np.float32


def quantize_activations(x):
    """x: [M, K] values exactly representable in fp32 (bf16 / fp16 inputs).
    Returns (q int8 [M, K], s fp32 [M])."""
    x = np.asarray(x, dtype=F32)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    amax = np.max(np.abs(x), axis=1)
    s = (amax / F32(127)).astype(F32)          # one fp32 division per row
    safe = np.where(s == 0, F32(1), s)
    t = (x / safe[:, None]).astype(F32)          # one fp32 division per element
    q = np.clip(np.rint(t), -127, 127)
    q = np.where(s[:, None] == 0, 0, q)
    return q.astype(np.int8), s


def dequantize_activations(q, s):
    """Exact fp64 value of the quantized activations."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[:, None]


def linear_a8w4(xq, xs, wq, ws, bias64=None):
    """y[m, n] = xs[m] * ws[n] * sum_k xq[m, k] * wq[n, k] (+ bias) in fp64.
    xq int8 [M, K], xs fp32 [M]; wq int8 codes in [-7, 7] [N, K], ws fp32 [N]
    (one scale per output channel)."""
    acc = np.asarray(xq, np.int64) @ np.asarray(wq, np.int64).T      # exact
    y = acc.astype(np.float64) * np.asarray(xs, np.float64)[:, None] \
        * np.asarray(ws, np.float64)[None, :]
    if bias64 is not None:
        y = y + np.asarray(bias64, np.float64)[None, :]
    return y
