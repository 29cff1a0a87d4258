"""Re-encoding plain per-group int4 / int6 weights into the nested
superscale formats.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ExecuTorch PR #20571, "[cuda] Nested Superscale Quantization for
CUDA Weights (int4 / int6)": in the review thread the authors convert the
original int4 and int6 tensors into Q4_K / Q6_K form and reuse the k-quant
pipeline (a loss of about 0.7 dB from the conversion); section "Analysis":
the weight codes stay identical to the source 4-bit / 6-bit values and only
the metadata is re-quantized; section "Quant schema update": the nested
encodings (uint8 scale and zero codes times per-256 fp16 steps for int4, an
int8 scale code times a per-256 fp16 step for int6).

Reading of the source forms (the pages name them but do not print them):
  plain int4: codes u in [0, 15], groups of 32 along K, an fp32 scale s >= 0
              and zero point z >= 0 in code units per group; w = (u - z) * s.
  plain int6: codes q in [-32, 31], groups of 16, an fp32 scale s >= 0 per
              group; w = q * s.
The metadata is re-quantized with exactly the rule of the nested quantizers
(`quantize_q4k` / `quantize_q6k` stage 2): per super-block of 256 weights,
step = fp16(fl32(max / levels)) and code = clamp(rint(fl32(v / step)), 0,
code_max), 0 where the step is 0.  The plain forms are what the nested
quantizers hold after their stage 1 (their "s", "z" outputs), so quantizing
W directly and converting W's plain form give the same bytes.
"""
import numpy as np

from .quantize import _encode_per_super

F32 = np.float32


def to_q4k(codes, s, z):
    """codes uint8 [N, K] in [0, 15]; s, z fp32 [N, K/32] (non-negative).
    Returns the q4k dict of `quantize` (codes unchanged)."""
    codes = np.asarray(codes)
    s = np.asarray(s, F32)
    z = np.asarray(z, F32)
    N, K = codes.shape
    if K % 256 or s.shape != (N, K // 32) or z.shape != s.shape:
        raise ValueError("q4k conversion needs K % 256 == 0 and [N, K/32] scales and zeros")
    if codes.min() < 0 or codes.max() > 15:
        raise ValueError("int4 codes must lie in [0, 15]")
    sc, sstep = _encode_per_super(s, 8, 255, 255)
    zc, zstep = _encode_per_super(z, 8, 255, 255)
    return {"codes": codes.astype(np.uint8), "sc": sc.astype(np.uint8),
            "zc": zc.astype(np.uint8), "sstep": sstep, "zstep": zstep, "s": s, "z": z}


def to_q6k(codes, s):
    """codes int8 [N, K] in [-32, 31]; s fp32 [N, K/16] (non-negative).
    Returns the q6k dict of `quantize` (codes unchanged)."""
    codes = np.asarray(codes)
    s = np.asarray(s, F32)
    N, K = codes.shape
    if K % 256 or s.shape != (N, K // 16):
        raise ValueError("q6k conversion needs K % 256 == 0 and [N, K/16] scales")
    if codes.min() < -32 or codes.max() > 31:
        raise ValueError("int6 codes must lie in [-32, 31]")
    sc, step = _encode_per_super(s, 16, 127, 127)
    return {"codes": codes.astype(np.int8), "sc": sc.astype(np.int8), "step": step, "s": s}


def plain_int4_f64(codes, s, z):
    """Exact fp64 value of a plain int4 weight: (u - z) * s per group."""
    u = np.asarray(codes, np.float64)
    N, K = u.shape
    S = np.repeat(np.asarray(s, np.float64), 32, axis=1)
    Z = np.repeat(np.asarray(z, np.float64), 32, axis=1)
    return (u - Z) * S


def plain_int6_f64(codes, s):
    """Exact fp64 value of a plain int6 weight: q * s per group."""
    q = np.asarray(codes, np.float64)
    return q * np.repeat(np.asarray(s, np.float64), 16, axis=1)
