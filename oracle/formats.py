"""The four weight formats, as the oracle understands them.

affine  (HF Transformers "Metal" page): unsigned b-bit codes, b in {2, 4, 8},
        per-group scale and bias in fp16 or bf16, w = q * scale + bias.
q4k     (ExecuTorch PR #20571, "Quant schema update", int4 bullet):
        unsigned 4-bit codes, group 32, super-block 256;
        scale = uint8 code * fp16 step, zero = uint8 code * fp16 step,
        w = (q - zero) * scale.
q6k     (same page, int6 bullet): symmetric signed 6-bit codes, group 16,
        super-block 256, scale = int8 code * fp16 step, no zero, w = q * scale.
sym4    (ExecuTorch PR #16577, description): symmetric int4 codes in
        [-7, 7] carried in int8, fp32 scale per output channel (group = K)
        or per group, w = q * scale.

Readings taken where the pages are silent (each one is listed in the design
notes):
  * bit order inside a uint32: code k sits at bits [b*(k % (32/b)), +b) of
    word k // (32/b), i.e. least-significant first along K;
  * int6 storage: two planes, the low nibble of u = q + 32 packed 8 per u32
    and its high 2 bits packed 16 per u32, both least-significant first;
  * sym4 kernel form: nibble u = q + 8 (zero pinned to 8);
  * q4k step word: low 16 bits = fp16 scale step, high 16 bits = fp16 zero
    step.
"""
from dataclasses import dataclass

FORMATS = ("affine", "q4k", "q6k", "sym4")


@dataclass(frozen=True)
class QFormat:
    fmt: str
    bits: int
    group_size: int
    meta: str = "bf16"          # affine only: 'f16' or 'bf16'
    super_block: int = 0        # 256 for the nested formats

    @staticmethod
    def affine(bits, group_size=64, meta="bf16"):
        return QFormat("affine", bits, group_size, meta, 0)

    @staticmethod
    def q4k():
        return QFormat("q4k", 4, 32, "f16", 256)

    @staticmethod
    def q6k():
        return QFormat("q6k", 6, 16, "f16", 256)

    @staticmethod
    def sym4(group_size):
        return QFormat("sym4", 4, group_size, "f32", 0)

    @property
    def signed(self):
        return self.fmt in ("q6k", "sym4")

    @property
    def qmin(self):
        return {"affine": 0, "q4k": 0, "q6k": -32, "sym4": -7}[self.fmt]

    @property
    def qmax(self):
        if self.fmt == "affine":
            return (1 << self.bits) - 1
        return {"q4k": 15, "q6k": 31, "sym4": 7}[self.fmt]


def check_shape(f: QFormat, N: int, K: int):
    """Shape rules the oracle assumes (the layer must tile into groups,
    packed words and, for nested formats, 256-weight super-blocks)."""
    if N <= 0 or K <= 0:
        raise ValueError("N and K must be positive")
    if K % f.group_size:
        raise ValueError("K must be a multiple of group_size")
    if f.fmt == "affine" and f.bits not in (2, 4, 8):
        raise ValueError("affine bits must be 2, 4 or 8")
    if K % (32 // (f.bits if f.bits != 6 else 2)):
        raise ValueError("K must fill whole uint32 words")
    if f.super_block:
        if K % f.super_block or f.super_block % f.group_size:
            raise ValueError("nested formats need K % 256 == 0")
