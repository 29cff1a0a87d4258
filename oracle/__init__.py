"""CPU oracle for the group-wise weight-only quantized linear layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
NumPy statement of what the quantized linear computes.  It exists to check the
HIP implementation, and only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import it.  The product path never calls it
and shares no code with it.

Sources (the pages this follows):
  * "Metal" quantization page of the HF Transformers docs, introduction and
    "load a pre-quantized model" sections: weights packed into uint32 tensors
    with per-group scales and biases (``qbiases``), bits 2/4/8, group size
    default 64, a fused dequantize + matmul ``affine_qmm_t``.
  * ExecuTorch PR #20571 "Nested Superscale Quantization for CUDA Weights
    (int4 / int6)", section "Quant schema update": dequant is affine,
    w = (q - zero) * scale; int4 Q4_K-style with gs=32, a 256-weight
    super-block, uint8 scale and zero codes times per-256 fp16 steps packed in
    one 32-bit word (4.625 bpw); int6 Q6_K-style symmetric with gs=16, int8
    scale code times a per-256 fp16 step (6.5625 bpw).  Section "Analysis":
    codes stay identical to the source values, only metadata is re-quantized.
    Review comment 1: max-based step, codes clamped to [0, 255], zero >= 0.
  * ExecuTorch PR #16577 "Arm backend: Support a8w4", description: int4
    carried in an int8 with qmin=-7, qmax=7; int8 activations (a8w4.py, with
    the per-token activation rule it states as a reading).

Every floating-point operation that the format fixes is done in IEEE fp32
(NumPy float32 arithmetic is correctly rounded), ties round half to even,
fp16 conversion keeps subnormals, and the linear layer's result is the fp64
matmul of the exactly dequantized weights.  Points the pages leave open are
taken at their plainest reading; each is listed in the module that uses it.

  * The same superscale page, review thread: the original int4 / int6
    tensors are converted into Q4_K / Q6_K with the codes kept
    (convert.py: to_q4k, to_q6k).
  * The same page, "Ablation study": alternative scale / zero encodings
    (ablation.py: encode_value, dequant_f64, bits_per_weight).
  * ExecuTorch PR #17235 (Metal int4 for Parakeet), review thread: the
    "hqq" choice of quantization parameters for the affine int4 weights,
    i.e. Half-Quadratic Quantization's zero-point optimisation
    (hqq.py: quantize_affine_hqq, with the readings it lists).

Parity status per function:
  quantize_* / pack_* / unpack_* / dequant_* / linear : pinned by the tests in
  tests/test_oracle_*.py (closed-form fixtures, lattice exactness, brute-force
  optimal rounding, exhaustive pack round trip, bpw accounting, scalar-loop
  equality).  a8w4 (quantize_activations, linear_a8w4): hand-worked tokens
  and dots, rounding invariants, exact rational brute force.  convert
  (to_q4k, to_q6k): hand-worked super-blocks, the lossless lattice case,
  the half-step bound.  hqq (quantize_affine_hqq, shrink_lp,
  hqq_zero_step): hand-worked thresholds and zero updates, the
  least-squares property of the update, no-iteration equality with the
  pinned min/max quantizer, lattice losslessness, lower l_p error than
  min/max.  ablation: the table's bpw column, the uint8 case
  against the pinned conversion, hand-worked lattice and rounding cases;
  its SNR values are parity unpinned (GGUF tensors), only the orderings.  snr_db: pinned by hand-worked closed forms; the
  pages' own SNR figures (GGUF tensors, not available) are not reproduced,
  only their ordering.
"""
from .numerics import (bf16_bits_to_f32, f32_to_bf16_bits, f16_bits_to_f32,
                       decode_activations)
from .formats import FORMATS, QFormat, check_shape
from .quantize import quantize
from .packing import pack_codes, unpack_codes, pack_bits, unpack_bits
from .dequant import dequant_f64, dequant_f32, dequant_out
from .linear import linear_f64
from .sizes import buffer_bytes, bits_per_weight
from .metrics import snr_db, rel_l2, maxabs_bound
from .a8w4 import quantize_activations, dequantize_activations, linear_a8w4
from .hqq import quantize_affine_hqq

__all__ = [
    "bf16_bits_to_f32", "f32_to_bf16_bits", "f16_bits_to_f32",
    "decode_activations", "FORMATS", "QFormat", "check_shape", "quantize",
    "pack_codes", "unpack_codes", "pack_bits", "unpack_bits", "dequant_f64",
    "dequant_f32", "dequant_out", "linear_f64", "buffer_bytes",
    "bits_per_weight", "snr_db", "rel_l2", "maxabs_bound",
    "quantize_activations", "dequantize_activations", "linear_a8w4",
    "quantize_affine_hqq",
]
