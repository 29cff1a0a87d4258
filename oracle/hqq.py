"""HQQ choice of the affine zero point for the Metal-style affine format.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ExecuTorch PR #17235, "Metal backend: Add Metal int4 quantization
support to Parakeet", review thread on `quantize.py`: the Metal int4 affine
weights (torchao's UIntxWeightOnlyConfig, bitwidth 4, group size) are to
choose their quantization parameters with the "hqq" algorithm.  The page
only names the option; the method is Half-Quadratic Quantization (H. Badri
and A. Shaji, 2023): the min/max scale s is kept and the zero point z (in
code units, w ~ (q - z) * s) is chosen to minimise an l_p error, p < 1, of
the group's reconstruction, by half-quadratic splitting.  An auxiliary
error variable W_e is introduced and the method alternates

  1. W_e <- shrink_p(W - dq(q(W; z)), beta), the generalised soft threshold
     shrink_p(e, beta) = sign(e) * max(|e| - |e|^(p - 1) / beta, 0)
     (the proximal step of the l_p term);
  2. z   <- mean over the group of (q(W; z) - (W - W_e) / s), the exact
     minimiser of the quadratic term for fixed codes;
  3. beta <- kappa * beta,

with q(W; z) = clamp(rint(W / s + z), 0, 2^b - 1) and dq(q) = (q - z) * s.

Readings (where the method leaves a choice open; the GPU quantizer takes the
same ones):
  H1  The scale is the AFFINE min/max scale as stored (meta-rounded); only
      the zero point moves.  The start is z0 = fl32(-bias0 / s) with bias0
      the stored min/max bias, so the start reproduces the plain quantizer.
  H2  Every step is one IEEE fp32 operation in the order written above;
      |e|^(p-1) is evaluated in fp64 (library pow) and rounded once to fp32;
      the group sums run sequentially in ascending k (fp32).
  H3  Hyper-parameters: p = 0.7, beta0 = 10, kappa = 1.01, 20 iterations
      (the method's published defaults), each given to the function as fp32.
  H4  Per group, the iterate (z0 .. z_T) with the smallest l1 error
      sum |W - dq(q(W; z))| (fp32, sequential) is kept; ties keep the
      earlier one, so the result is never worse than the start in that
      measure.
  H5  The kept zero becomes the stored bias meta(fl32(-z * s)) (+0 for a
      zero), and the codes are then rounded against the stored scale and
      bias exactly as the plain affine quantizer does, so the kernels'
      dequantization w = q * scale + bias is unchanged.  A group with
      scale 0 is left as the plain quantizer leaves it.
"""
import numpy as np

from .formats import QFormat, check_shape
from .numerics import to_meta, meta_to_f32
from .quantize import quantize_affine

F32 = np.float32


def shrink_lp(e, beta, p):
    """Generalised soft threshold (reading H2): sign(e) * max(|e| -
    fl32(fl32(|e|^(p-1)) / beta), 0), with the power in fp64 rounded once
    to fp32, and 0 for e == 0."""
    e = np.asarray(e, F32)
    a = np.abs(e)
    live = a > 0
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        g = np.power(a.astype(np.float64), np.float64(F32(p)) - 1.0).astype(F32)
        h = g / F32(beta)
        t = a - h
    return np.where(live & (t > 0), np.copysign(t, e), F32(0)).astype(F32)


def _seq_sum(v):
    """fp32 sum along the last axis, in ascending order."""
    acc = np.zeros(v.shape[:-1], F32)
    for k in range(v.shape[-1]):
        acc = acc + v[..., k]
    return acc


def _codes(G, s, z, qmax):
    return np.clip(np.rint(G / s + z), 0, qmax).astype(F32)


def hqq_zero_step(G, s, z, beta, p, qmax):
    """One half-quadratic update of the zero points.

    G [..., gs] fp32 group values, s [..., 1] fp32 scales (non-zero), z
    [..., 1] fp32 zero points.  Returns (new z [..., 1], l1 error of the
    given z [...]) following steps 1 and 2 of the module docstring."""
    q = _codes(G, s, z, qmax)
    e = G - (q - z) * s
    err = _seq_sum(np.abs(e))
    we = shrink_lp(e, beta, p)
    v = q - (G - we) / s
    znew = (_seq_sum(v) / F32(G.shape[-1]))[..., None]
    return znew.astype(F32), err


def quantize_affine_hqq(W, f: QFormat, iters=20, p=0.7, beta=10.0, kappa=1.01):
    """AFFINE quantization with the HQQ zero point (readings H1-H5).

    Returns the same dict as `quantize` for the affine format: codes uint8
    [N, K], scales and biases [N, K/gs] as fp16 / bf16 bit patterns."""
    if f.fmt != "affine":
        raise ValueError("HQQ applies to the affine format")
    W = np.ascontiguousarray(np.asarray(W, dtype=np.float32))
    N, K = W.shape
    check_shape(f, N, K)
    if not np.all(np.isfinite(W)):
        raise ValueError("weights must be finite")
    if iters < 0:
        raise ValueError("iters must be >= 0")
    plain = quantize_affine(W, f)            # H1: the start and its scale
    gs, qmax = f.group_size, F32(f.qmax)
    G = W.reshape(N, K // gs, gs)
    s = meta_to_f32(plain["scales"], f.meta)[..., None]
    b0 = meta_to_f32(plain["biases"], f.meta)[..., None]
    live = s != 0
    sd = np.where(live, s, F32(1)).astype(F32)   # scale-0 groups: ignored
    z = ((-b0) / sd).astype(F32)
    best_z = z.copy()
    best_err = np.full(z.shape[:-1], np.inf, F32)
    bt = F32(beta)
    for t in range(iters + 1):
        if t < iters:
            znew, err = hqq_zero_step(G, sd, z, bt, p, qmax)
        else:
            q = _codes(G, sd, z, qmax)
            err = _seq_sum(np.abs(G - (q - z) * sd))
        better = err < best_err                  # H4: strict, earlier wins ties
        best_z = np.where(better[..., None], z, best_z)
        best_err = np.where(better, err, best_err)
        if t < iters:
            z = znew
            bt = F32(bt * F32(kappa))
    bias = (-best_z) * s + F32(0)                # H5 (+0 canonical zero)
    b_bits = np.where(live[..., 0], to_meta(bias[..., 0], f.meta), plain["biases"])
    b = meta_to_f32(b_bits, f.meta)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        tq = (G - b) / s
    q = np.where(live, np.clip(np.rint(tq), 0, qmax), 0)
    return {"codes": q.reshape(N, K).astype(np.uint8),
            "scales": plain["scales"].copy(), "biases": b_bits.astype(np.uint16)}
