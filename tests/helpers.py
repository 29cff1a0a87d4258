"""Shared test plumbing: host<->device marshalling and the output tolerance.

Only the tests import this.  Reference values come from the oracle package.
"""
import numpy as np

import oracle
from oracle import QFormat
from oracle.packing import to_buffers


def qformat_of(desc):
    if desc.fmt == "affine":
        return QFormat.affine(desc.bits, desc.group_size, desc.meta)
    if desc.fmt == "q4k":
        return QFormat.q4k()
    if desc.fmt == "q6k":
        return QFormat.q6k()
    return QFormat.sym4(desc.group_size)


def to_dev_bits(bits, xdtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if xdtype == "bf16" else torch.float16).cuda()


def buf_to_np(t):
    """Device buffer -> uint8 numpy bytes (layout-agnostic comparison)."""
    import torch
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def oracle_buffers(W_rows, f):
    """Oracle quantization of some rows -> dict of byte arrays [rows, bytes]."""
    buf = to_buffers(oracle.quantize(W_rows, f), f)
    out = {}
    for k, v in buf.items():
        if v is not None:
            a = np.ascontiguousarray(v)
            out[k] = a.view(np.uint8).reshape(W_rows.shape[0], -1)
    return out


def gpu_rows(buf_dev, N, rows):
    """Rows of a device buffer laid out [N, ...] -> uint8 numpy [len(rows), bytes]."""
    b = buf_to_np(buf_dev).reshape(N, -1)
    return b[rows]


def y_to_f64(y):
    import torch
    return y.detach().float().cpu().numpy().astype(np.float64)


def ulp(v, ydt):
    """Spacing of the output type at |v| (normal range)."""
    a = np.abs(np.asarray(v, np.float64))
    if ydt == "f32":
        return np.spacing(a.astype(np.float32)).astype(np.float64)
    if ydt == "f16":
        return np.spacing(a.astype(np.float16)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def round_out(y_ref, ydt):
    y32 = np.asarray(y_ref, np.float64).astype(np.float32)
    if ydt == "f16":
        return y32.astype(np.float16).astype(np.float64)
    if ydt == "bf16":
        return oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(y32)).astype(np.float64)
    return y32.astype(np.float64)


def check_linear(y_dev, y_ref, x64, wmax, K, ydt, rel=2e-3):
    """The layer's tolerance: rel-L2 <= 2e-3 and per element
    |y - y_ref| <= 1e-2 * ||x_m|| * max|w| / sqrt(K) (+ half an output ulp
    for fp16 / bf16 outputs, the rounding of the result itself).

    rel-L2 <= 2e-3 is required of fp32 outputs and of fp16/bf16 outputs with
    at least 4096 elements (bf16 rounding alone costs ~1.7e-3 on average).
    A smaller fp16/bf16 output may also carry the rel-L2 that rounding the
    exact result to its type costs (up to 2^-8 per element for bf16)."""
    y = y_to_f64(y_dev)
    assert y.shape == y_ref.shape
    assert np.all(np.isfinite(y))
    r = oracle.rel_l2(y, y_ref)
    if ydt != "f32" and y.size < 4096:
        rel = rel + oracle.rel_l2(round_out(y_ref, ydt), y_ref)
    bound = oracle.maxabs_bound(x64, wmax, K)
    if ydt != "f32":
        bound = bound + 0.5 * ulp(y_ref, ydt)
    err = np.abs(y - y_ref)
    bound = np.broadcast_to(bound, err.shape)
    # a zero bound (all-zero weights) demands an exact result
    ratio = np.divide(err, bound, out=np.where(err == 0, 0.0, np.inf), where=bound > 0)
    worst = float(np.max(ratio))
    assert r <= rel, f"rel-L2 {r:.3e} > {rel}"
    assert worst <= 1.0, f"max-abs error is {worst:.3f}x the bound"
    return r, worst

