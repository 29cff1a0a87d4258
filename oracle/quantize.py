"""Quantization of an fp32 weight matrix W [N, K] into codes + metadata.

Each function follows the steps of its format in the order the pages give
them; every arithmetic step is one IEEE fp32 operation (NumPy float32),
rounding of codes is np.rint (half to even), and codes are clamped to the
format's range.  Groups run along K (the input dimension) of each output row.

Signed zeros: a zero extreme or zero point is taken as +0.0 (IEEE x + 0.0
turns -0.0 into +0.0), so a group whose minimum is +-0 stores bias +0 and an
all-non-negative q4k group stores zero point +0 (the superscale review notes
that zero points are non-negative; the sign of a zero carries no value).

Returned dict (all NumPy arrays, row-major with N leading):
  codes   [N, K]      uint8 (affine, q4k) or int8 (q6k, sym4)
  affine: scales, biases  [N, K/gs]  uint16 bit patterns (fp16 or bf16)
  q4k:    sc, zc [N, K/32] uint8; sstep, zstep [N, K/256] float16;
          plus s, z [N, K/32] float32 (the group scale / zero before their
          re-quantization, kept for the pins)
  q6k:    sc [N, K/16] int8 in [0, 127]; step [N, K/256] float16; s fp32
  sym4:   scales [N, K/gs] float32
"""
import numpy as np

from .formats import QFormat, check_shape
from .numerics import to_meta, meta_to_f32

F32 = np.float32


def _groups(W, gs):
    N, K = W.shape
    return W.reshape(N, K // gs, gs)


def quantize_affine(W, f: QFormat):
    """MLX-style group affine quantization (HF Transformers "Metal" page:
    uint32-packed weights with per-group scales and biases, bits 2/4/8).

    The page does not print the rule; the plainest one it supports is used:
    per group lo = min(w), hi = max(w); scale = meta(fl32(fl32(hi - lo) /
    (2^b - 1))); bias = meta(lo); codes are rounded against the stored
    (meta-rounded) scale and bias so that pack-time and kernel-time
    reconstruction agree (the superscale page's review notes the same
    principle for its steps); a zero scale gives code 0."""
    G = _groups(W, f.group_size)
    # "+ 0" turns a -0.0 extreme into +0.0 (signed zeros are canonical +0
    # in the metadata; see the module notes)
    lo = G.min(axis=2) + F32(0)
    hi = G.max(axis=2) + F32(0)
    s32 = (hi - lo) / F32(f.qmax)
    s_bits = to_meta(s32, f.meta)
    b_bits = to_meta(lo, f.meta)
    s = meta_to_f32(s_bits, f.meta)[..., None]
    b = meta_to_f32(b_bits, f.meta)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (G - b) / s
    q = np.where(s != 0, np.clip(np.rint(t), 0, f.qmax), 0)
    N, K = W.shape
    return {"codes": q.reshape(N, K).astype(np.uint8),
            "scales": s_bits, "biases": b_bits}


def _encode_per_super(v, per_super, levels, code_max):
    """Re-quantize non-negative per-group values v [N, G] to integer codes
    times one fp16 step per super-block (superscale page: max-based step,
    rounding against the fp16-rounded step, codes clamped).

    step = fp16(fl32(max over the super-block / levels));
    code = 0 if step == 0 else clamp(rint(fl32(v / fp32(step))), 0, code_max)
    """
    if np.any(v < 0):
        # The pages' encoder would silently clamp a negative value; the
        # review asks for a loud failure instead.
        raise ValueError("superscale encoder needs non-negative inputs")
    N, Gn = v.shape
    vb = v.reshape(N, Gn // per_super, per_super)
    step = (vb.max(axis=2) / F32(levels)).astype(np.float16)
    st = step.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = vb / st
    code = np.where(st != 0, np.clip(np.rint(t), 0, code_max), 0)
    return code.reshape(N, Gn), step


def quantize_q4k(W, f: QFormat):
    """Q4_K-style nested superscale int4 (superscale page, int4 bullet).

    1. Per group of 32: lo = min(min w, 0), hi = max(max w, 0) (the range is
       widened to contain 0 so that the zero point lies in [0, 15], the
       invariant the page's review relies on);
       s = fl32(fl32(hi - lo) / 15); z = fl32(-lo / s);
       q = clamp(rint(fl32(fl32(w - lo) / s)), 0, 15); s == 0 gives q = z = 0.
       Codes are fixed here and never recomputed ("Analysis": codes stay
       identical to the source 4-bit values, only metadata is re-quantized).
    2. Per super-block of 256 (8 groups): scale and zero are each encoded as
       a uint8 code times an fp16 step (step = max / 255)."""
    G = _groups(W, 32)
    lo = np.minimum(G.min(axis=2), F32(0)) + F32(0)
    hi = np.maximum(G.max(axis=2), F32(0)) + F32(0)
    s = (hi - lo) / F32(15)
    with np.errstate(divide="ignore", invalid="ignore"):
        z = (np.where(s != 0, (-lo) / s, F32(0)) + F32(0)).astype(np.float32)
        t = (G - lo[..., None]) / s[..., None]
    q = np.where(s[..., None] != 0, np.clip(np.rint(t), 0, 15), 0)
    sc, sstep = _encode_per_super(s, 8, 255, 255)
    zc, zstep = _encode_per_super(z, 8, 255, 255)
    N, K = W.shape
    return {"codes": q.reshape(N, K).astype(np.uint8),
            "sc": sc.astype(np.uint8), "zc": zc.astype(np.uint8),
            "sstep": sstep, "zstep": zstep, "s": s, "z": z}


def quantize_q6k(W, f: QFormat):
    """Q6_K-style symmetric int6 (superscale page, int6 bullet).

    1. Per group of 16: s = fl32(max|w| / 31);
       q = clamp(rint(fl32(w / s)), -32, 31) (the int6 storage range;
       |q| <= 31 in practice); s == 0 gives q = 0.
    2. Per super-block of 256 (16 groups): s is encoded as a non-negative
       int8 code times an fp16 step (step = max / 127, code in [0, 127])."""
    G = _groups(W, 16)
    s = np.abs(G).max(axis=2) / F32(31)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = G / s[..., None]
    q = np.where(s[..., None] != 0, np.clip(np.rint(t), -32, 31), 0)
    sc, step = _encode_per_super(s, 16, 127, 127)
    N, K = W.shape
    return {"codes": q.reshape(N, K).astype(np.int8),
            "sc": sc.astype(np.int8), "step": step, "s": s}


def quantize_sym4(W, f: QFormat):
    """Symmetric int4 in an int8 carrier, qmin = -7, qmax = 7 (a8w4 page).

    s = fl32(max|w| / 7) per group (group = K: one scale per output
    channel), stored as fp32; q = clamp(rint(fl32(w / s)), -7, 7)."""
    G = _groups(W, f.group_size)
    s = np.abs(G).max(axis=2) / F32(7)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = G / s[..., None]
    q = np.where(s[..., None] != 0, np.clip(np.rint(t), -7, 7), 0)
    N, K = W.shape
    return {"codes": q.reshape(N, K).astype(np.int8),
            "scales": s.astype(np.float32)}


def quantize(W, f: QFormat):
    W = np.ascontiguousarray(np.asarray(W, dtype=np.float32))
    N, K = W.shape
    check_shape(f, N, K)
    if not np.all(np.isfinite(W)):
        raise ValueError("weights must be finite")
    return {"affine": quantize_affine, "q4k": quantize_q4k,
            "q6k": quantize_q6k, "sym4": quantize_sym4}[f.fmt](W, f)
