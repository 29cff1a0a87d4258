"""Bit-packing of integer codes into uint32 words.

The "Metal" page says only that weights are packed into uint32 tensors.  The
reading taken: code k of a row lands in word k // (32/b), at bits
[b * (k % (32/b)), b * (k % (32/b)) + b) -- least-significant first along K
-- and rows are laid out one after another ([N, K*b/32] row-major).

Formats map their codes to unsigned fields before packing:
  affine, q4k : the code itself (already unsigned)
  sym4        : u = q + 8 in [1, 15]
  q6k         : u = q + 32 in [0, 63]; low nibble plane (8 per word) and a
                high 2-bit plane (16 per word), both packed as above.
"""
import numpy as np

from .formats import QFormat


def pack_bits(u, b):
    """u: [N, K] unsigned fields (< 2**b) -> [N, K*b/32] uint32."""
    u = np.asarray(u).astype(np.uint64)
    N, K = u.shape
    per = 32 // b
    if K % per:
        raise ValueError("K must fill whole words")
    if np.any(u >> np.uint64(b)):
        raise ValueError("field does not fit in b bits")
    u = u.reshape(N, K // per, per)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(b))
    words = (u << shifts).sum(axis=2)       # disjoint bit fields: sum == or
    return words.astype(np.uint32)


def unpack_bits(words, b, K):
    """Inverse of pack_bits: [N, K*b/32] uint32 -> [N, K] uint8 fields."""
    w = np.asarray(words, dtype=np.uint32).astype(np.uint64)
    N = w.shape[0]
    per = 32 // b
    shifts = np.arange(per, dtype=np.uint64) * np.uint64(b)
    mask = np.uint64((1 << b) - 1)
    u = (w[:, :, None] >> shifts) & mask
    return u.reshape(N, K).astype(np.uint8)


def pack_codes(codes, f: QFormat):
    """Codes [N, K] -> dict of packed planes: {'qweight'} (+ 'qweight_hi')."""
    c = np.asarray(codes).astype(np.int64)
    if np.any(c < f.qmin) or np.any(c > f.qmax):
        raise ValueError("code outside the format's range")
    if f.fmt in ("affine", "q4k"):
        return {"qweight": pack_bits(c, f.bits)}
    if f.fmt == "sym4":
        return {"qweight": pack_bits(c + 8, 4)}
    u = c + 32                                   # q6k
    return {"qweight": pack_bits(u & 15, 4), "qweight_hi": pack_bits(u >> 4, 2)}


def unpack_codes(planes, f: QFormat, K):
    """Packed planes -> codes [N, K] (uint8 for affine/q4k, int8 otherwise)."""
    if f.fmt in ("affine", "q4k"):
        return unpack_bits(planes["qweight"], f.bits, K)
    if f.fmt == "sym4":
        return (unpack_bits(planes["qweight"], 4, K).astype(np.int16)
                - 8).astype(np.int8)
    lo = unpack_bits(planes["qweight"], 4, K).astype(np.int16)
    hi = unpack_bits(planes["qweight_hi"], 2, K).astype(np.int16)
    return ((lo | (hi << 4)) - 32).astype(np.int8)


def q4k_step_words(sstep, zstep):
    """Two fp16 steps in one 32-bit word: low half = scale step, high half =
    zero step (the page says only that both are packed in one word)."""
    s = np.asarray(sstep, dtype=np.float16).view(np.uint16).astype(np.uint32)
    z = np.asarray(zstep, dtype=np.float16).view(np.uint16).astype(np.uint32)
    return (s | (z << np.uint32(16))).astype(np.uint32)


def q4k_split_step_words(words):
    w = np.asarray(words, dtype=np.uint32)
    s = (w & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z = (w >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return s, z


def to_buffers(qz, f: QFormat):
    """Quantizer output -> the five buffers of the packed layout:
    qweight, qweight_hi, scales, zeros, steps (None where unused)."""
    planes = pack_codes(qz["codes"], f)
    out = {"qweight": planes["qweight"], "qweight_hi": planes.get("qweight_hi"),
           "scales": None, "zeros": None, "steps": None}
    if f.fmt == "affine":
        out["scales"] = qz["scales"]
        out["zeros"] = qz["biases"]
    elif f.fmt == "q4k":
        out["scales"] = qz["sc"]
        out["zeros"] = qz["zc"]
        out["steps"] = q4k_step_words(qz["sstep"], qz["zstep"])
    elif f.fmt == "q6k":
        out["scales"] = qz["sc"]
        out["steps"] = qz["step"].view(np.uint16)
    else:
        out["scales"] = qz["scales"]
    return out


def from_buffers(buf, f: QFormat, K):
    """The five buffers -> codes + metadata in the quantizer's dict form."""
    codes = unpack_codes(buf, f, K)
    if f.fmt == "affine":
        return {"codes": codes, "scales": np.asarray(buf["scales"], np.uint16),
                "biases": np.asarray(buf["zeros"], np.uint16)}
    if f.fmt == "q4k":
        s, z = q4k_split_step_words(buf["steps"])
        return {"codes": codes, "sc": np.asarray(buf["scales"], np.uint8),
                "zc": np.asarray(buf["zeros"], np.uint8), "sstep": s, "zstep": z}
    if f.fmt == "q6k":
        return {"codes": codes, "sc": np.asarray(buf["scales"], np.int8),
                "step": np.asarray(buf["steps"], np.uint16).view(np.float16)}
    return {"codes": codes, "scales": np.asarray(buf["scales"], np.float32)}
