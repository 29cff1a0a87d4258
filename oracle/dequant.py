"""Dequantization: codes + metadata -> weights.

dequant_f64 is the exact value of each format's closed form (every form is
exact in fp64: products of at most 8-bit codes with 8..11-bit metadata):
  affine : w = q * scale + bias          ("Metal" page, per-group scale/bias)
  q4k    : w = (q - zc*zstep) * (sc*sstep)  (superscale page: w = (q - zero)
           * scale, zero and scale each a uint8 code times an fp16 step)
  q6k    : w = q * (sc*step)             (superscale page, int6: no zero)
  sym4   : w = q * scale                 (a8w4 page: symmetric, qmin=-7..7)

dequant_f32 is the fp32 evaluation of the same closed form in the pages'
operation order, one IEEE fp32 operation per step:
  affine : fl32(fl32(q*scale) + bias)          (q*scale exact)
  q4k    : fl32(fl32(q - fl32(zc*zstep)) * fl32(sc*sstep))  (products exact)
  q6k    : fl32(q * fl32(sc*step))             (exact)
  sym4   : fl32(q * scale)
For affine, q6k and sym4 this equals the fp64 value rounded once to fp32;
for q4k it can differ from that in the last place when q - zero is inexact.
"""
import numpy as np

from .formats import QFormat
from .numerics import meta_to_f32, f32_to_bf16_bits

F32 = np.float32


def _expand(meta, gs):
    return np.repeat(meta, gs, axis=1)


def dequant_f64(qz, f: QFormat):
    q = qz["codes"].astype(np.float64)
    if f.fmt == "affine":
        s = meta_to_f32(qz["scales"], f.meta).astype(np.float64)
        b = meta_to_f32(qz["biases"], f.meta).astype(np.float64)
        return q * _expand(s, f.group_size) + _expand(b, f.group_size)
    if f.fmt == "q4k":
        S = qz["sc"].astype(np.float64) * _expand(
            qz["sstep"].astype(np.float64), 8)
        Z = qz["zc"].astype(np.float64) * _expand(
            qz["zstep"].astype(np.float64), 8)
        return (q - _expand(Z, 32)) * _expand(S, 32)
    if f.fmt == "q6k":
        S = qz["sc"].astype(np.float64) * _expand(
            qz["step"].astype(np.float64), 16)
        return q * _expand(S, 16)
    s = qz["scales"].astype(np.float64)
    return q * _expand(s, f.group_size)


def dequant_f32(qz, f: QFormat):
    q = qz["codes"].astype(np.float32)
    if f.fmt == "affine":
        s = _expand(meta_to_f32(qz["scales"], f.meta), f.group_size)
        b = _expand(meta_to_f32(qz["biases"], f.meta), f.group_size)
        return (q * s) + b
    if f.fmt == "q4k":
        S = qz["sc"].astype(F32) * _expand(qz["sstep"].astype(F32), 8)
        Z = qz["zc"].astype(F32) * _expand(qz["zstep"].astype(F32), 8)
        return (q - _expand(Z, 32)) * _expand(S, 32)
    if f.fmt == "q6k":
        S = qz["sc"].astype(F32) * _expand(qz["step"].astype(F32), 16)
        return q * _expand(S, 16)
    return q * _expand(qz["scales"].astype(F32), f.group_size)


def dequant_out(qz, f: QFormat, out):
    """Dequantized weights in an output type: 'f32' is dequant_f32; 'f16'
    and 'bf16' round that fp32 value once more (to nearest, ties to even).
    f16/bf16 results are returned as uint16 bit patterns."""
    w = dequant_f32(qz, f)
    if out == "f32":
        return w
    if out == "f16":
        return w.astype(np.float16).view(np.uint16)
    if out == "bf16":
        return f32_to_bf16_bits(w)
    raise ValueError(out)
