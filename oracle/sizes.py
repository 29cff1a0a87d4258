"""Storage accounting: bytes of each packed buffer and bits per weight.

Buffers (row-major, N leading):
  qweight     codes, [N, K*b/32] uint32 (q6k: low-nibble plane [N, K/8])
  qweight_hi  q6k only: high 2-bit plane [N, K/16] uint32
  scales      affine: [N, K/gs] fp16|bf16; q4k: [N, K/32] uint8;
              q6k: [N, K/16] int8; sym4: [N, K/gs] fp32
  zeros       affine biases [N, K/gs] fp16|bf16; q4k zero codes [N, K/32]
  steps       q4k: [N, K/256] uint32 (two fp16 steps); q6k: [N, K/256] fp16

The superscale page states 4.625 bpw for its int4 form (4 + 8/32 + 8/32 +
32/256) and 6.5625 for int6 (6 + 8/16 + 16/256).
"""
from .formats import QFormat


def buffer_bytes(f: QFormat, N, K):
    nb = {"qweight": 0, "qweight_hi": 0, "scales": 0, "zeros": 0, "steps": 0}
    if f.fmt == "affine":
        nb["qweight"] = N * K * f.bits // 8
        nb["scales"] = N * (K // f.group_size) * 2
        nb["zeros"] = N * (K // f.group_size) * 2
    elif f.fmt == "q4k":
        nb["qweight"] = N * K // 2
        nb["scales"] = N * K // 32
        nb["zeros"] = N * K // 32
        nb["steps"] = N * (K // 256) * 4
    elif f.fmt == "q6k":
        nb["qweight"] = N * K // 2
        nb["qweight_hi"] = N * K // 4
        nb["scales"] = N * K // 16
        nb["steps"] = N * (K // 256) * 2
    else:
        nb["qweight"] = N * K // 2
        nb["scales"] = N * (K // f.group_size) * 4
    return nb


def bits_per_weight(f: QFormat, N, K):
    return 8.0 * sum(buffer_bytes(f, N, K).values()) / (N * K)
