"""Metadata encodings of the superscale ablation: alternative ways to store
the per-group scale and zero point of Q4_K-style int4 weights.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ExecuTorch PR #20571, "[cuda] Nested Superscale Quantization for
CUDA Weights (int4 / int6)", section "Ablation study" (a table of scale code,
scale step, zero code and zero step choices with their SNR and bits per
weight) and section "Analysis" (step granularity matters more than step
dtype; narrower codes lose accuracy; codes stay the source values).

An encoding names, for the scale and for the zero point of each group of 32:
  code: "bf16" (the value itself in bf16, no step), "u8" (uint8 code, levels
        255) or "u6" (6-bit code, levels 63);
  step: "256" (one step per 256 weights, i.e. per 8 groups) or "row" (one
        step per output row), stored as "f16" or "bf16".
Reading (the page gives the table, not the rule): every code is computed
with the rule of the nested quantizer -- step = dtype(fl32(max / levels))
over the step's span, code = clamp(rint(fl32(v / step)), 0, levels), 0
where the step is 0 -- and the int4 codes and the plain per-group (s, z)
are those of the nested quantizer's first stage, so only the metadata
differs between encodings.

Bits per weight: 4 for the codes, the code bits / 32 for each of scale and
zero, and 16 bits per step over its span (256 weights, or K per row).  The
table prints the per-256 rows exactly and the per-row rows without the
16/K term (4.5625, 4.500), except its last row (4.441), which matches
4.4375 + 32/K at K near 9000; `bits_per_weight` gives both terms.
"""
import numpy as np

from .numerics import f32_to_bf16_bits, bf16_bits_to_f32

F32 = np.float32

LEVELS = {"u8": 255, "u6": 63}
CODE_BITS = {"bf16": 16, "u8": 8, "u6": 6}


def _round_step(x32, dtype):
    x32 = np.asarray(x32, F32)
    if dtype == "f16":
        return x32.astype(np.float16).astype(F32)
    return bf16_bits_to_f32(f32_to_bf16_bits(x32)).astype(F32)


def encode_value(v, code, step, step_dtype):
    """Re-quantize non-negative per-group values v [N, G] (G groups of 32
    per row).  Returns the decoded fp64 values the encoding stores."""
    v = np.asarray(v, F32)
    if np.any(v < 0):
        raise ValueError("metadata encodings need non-negative values")
    if code == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(v)).astype(np.float64)
    levels = LEVELS[code]
    N, G = v.shape
    span = 8 if step == "256" else G
    vb = v.reshape(N, G // span, span)
    st = _round_step(vb.max(axis=2) / F32(levels), step_dtype)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (vb / st).astype(F32)
    c = np.where(st != 0, np.clip(np.rint(t), 0, levels), 0)
    return (c.astype(np.float64) * st.astype(np.float64)).reshape(N, G)


def dequant_f64(codes, s, z, enc):
    """Weights of an int4 layer (codes [N, K] in [0, 15], plain s, z [N, K/32])
    under encoding enc = (scale_code, scale_step, scale_step_dtype, zero_code,
    zero_step, zero_step_dtype): w = (u - Z) * S."""
    sc, ss, sd, zc, zs, zd = enc
    S = encode_value(s, sc, ss, sd)
    Z = encode_value(z, zc, zs, zd)
    u = np.asarray(codes, np.float64)
    return (u - np.repeat(Z, 32, axis=1)) * np.repeat(S, 32, axis=1)


def bits_per_weight(enc, K):
    """(bits per weight without the per-row step terms, with them)."""
    sc, ss, _, zc, zs, _ = enc
    base = 4.0 + CODE_BITS[sc] / 32.0 + CODE_BITS[zc] / 32.0
    row = 0.0
    for code, step in ((sc, ss), (zc, zs)):
        if code == "bf16":
            continue
        if step == "256":
            base += 16.0 / 256.0
        else:
            row += 16.0 / K
    return base, base + row
