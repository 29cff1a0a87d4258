"""Scalar-type helpers of the oracle: fp32 / fp16 / bf16 encodings.

bf16 is the upper half of an IEEE fp32 word; rounding to it is written out
on the bits (round to nearest, ties to even).  fp16 rounding uses NumPy's
float32 -> float16 conversion, which rounds to nearest-even and produces
subnormals (the nested steps of the superscale formats are mostly fp16
subnormals at ordinary weight scales, so flushing them would be wrong).
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16, ties to even.  Returns uint16 bit patterns.

    Inputs must be finite (the quantized formats never carry NaN/Inf)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns to fp32."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_bits_to_f32(b):
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return b.view(np.float16).astype(np.float32)


def f32_to_f16(x):
    """Round fp32 to fp16 (nearest-even, subnormals kept)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def to_meta(x32, meta):
    """Round fp32 metadata to its storage type; returns uint16 bit patterns."""
    if meta == "f16":
        return f32_to_f16(x32).view(np.uint16)
    if meta == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown metadata dtype {meta!r}")


def meta_to_f32(bits, meta):
    if meta == "f16":
        return f16_bits_to_f32(bits)
    if meta == "bf16":
        return bf16_bits_to_f32(bits)
    raise ValueError(f"unknown metadata dtype {meta!r}")


def decode_activations(bits, dtype):
    """Activation bit patterns (uint16, 'f16' or 'bf16') -> exact fp64."""
    if dtype == "f16":
        return f16_bits_to_f32(bits).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown activation dtype {dtype!r}")
