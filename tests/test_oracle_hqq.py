"""Pins of the oracle's HQQ zero-point choice (oracle/hqq.py).

HQQ (Half-Quadratic Quantization, Badri and Shaji 2023) is the
quantization-parameter option that ExecuTorch PR #17235's review asks for
on the Metal int4 affine weights.  What pins it, without trusting it:

  * hand-worked generalised soft thresholds and zero-point updates
    (tests/golden/closed_forms.json, "hqq"): a wrong sign, a p in place of
    p - 1, a missing division by beta or a sum in place of the mean fails;
  * the zero update is the least-squares zero of the quadratic term,
    checked against an fp64 evaluation of that minimiser;
  * with no iterations the result is the plain min/max affine quantizer,
    byte for byte (pins the final encode against the pinned quantizer);
  * weights on the quantization lattice stay lossless;
  * the method's purpose: the l_p reconstruction error (p = 0.7) of the
    whole layer drops below the min/max quantizer's, and so does the l1
    error of every group (the kept iterate is never worse than the start).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import QFormat
from oracle.hqq import hqq_zero_step, quantize_affine_hqq, shrink_lp

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "closed_forms.json")))["hqq"]
F32 = np.float32


def _f(v):
    return float(Fraction(v))


@pytest.mark.parametrize("case", GOLD["shrink"], ids=lambda c: f"p{c['p']}_b{c['beta']}_e{c['e']}")
def test_shrink_golden(case):
    out = shrink_lp(np.array([_f(case["e"])], F32), case["beta"], case["p"])
    assert out.dtype == F32
    assert float(out[0]) == _f(case["out"])


@pytest.mark.parametrize("case", GOLD["zero_step"], ids=range(len(GOLD["zero_step"])))
def test_zero_step_golden(case):
    G = np.array([[_f(v) for v in case["G"]]], F32)
    s = np.array([[_f(case["s"])]], F32)
    z = np.array([[_f(case["z"])]], F32)
    znew, err = hqq_zero_step(G, s, z, F32(case["beta"]), case["p"], F32(case["qmax"]))
    assert float(znew[0, 0]) == _f(case["z_new"])
    assert float(err[0]) == _f(case["err"])


def test_zero_step_is_least_squares_zero():
    """z' minimises sum (q - (G - W_e)/s - z')^2: it is the group mean of
    u = q - (G - W_e)/s, up to fp32 rounding of the sequential sum."""
    rng = np.random.default_rng(3)
    G = rng.laplace(0, 0.015, (64, 64)).astype(F32)
    lo, hi = G.min(1, keepdims=True), G.max(1, keepdims=True)
    s = ((hi - lo) / F32(15)).astype(F32)
    z = (-lo / s + F32(0.3)).astype(F32)
    for beta in (1e-3, 10.0, 1e3):
        znew, _ = hqq_zero_step(G, s, z, F32(beta), 0.7, F32(15))
        q = np.clip(np.rint(G / s + z), 0, 15).astype(np.float64)
        e = G - ((q.astype(F32) - z) * s)
        we = shrink_lp(e, F32(beta), 0.7).astype(np.float64)
        u = q - (G.astype(np.float64) - we) / s.astype(np.float64)
        mean = u.mean(1, keepdims=True)
        tol = 64 * 4 * np.finfo(F32).eps * (np.abs(u).max(1, keepdims=True) + 1)
        assert np.all(np.abs(znew - mean) <= tol), beta


@pytest.mark.parametrize("bits,gs,meta", [(2, 64, "bf16"), (4, 64, "bf16"), (4, 32, "f16"),
                                          (8, 128, "bf16"), (4, 128, "f16")])
def test_no_iterations_is_plain_minmax(bits, gs, meta):
    rng = np.random.default_rng(bits * 100 + gs)
    W = rng.normal(0, 0.02, (48, 512)).astype(F32)
    W[3, 64:128] = 0.25          # a constant group: scale 0
    W[5, :64] = -0.0             # negative zeros
    f = QFormat.affine(bits, gs, meta)
    h = quantize_affine_hqq(W, f, iters=0)
    p = oracle.quantize(W, f)
    for k in ("codes", "scales", "biases"):
        assert np.array_equal(h[k], p[k]), k


@pytest.mark.parametrize("bits,meta", [(2, "bf16"), (4, "f16"), (8, "bf16")])
def test_lattice_weights_stay_lossless(bits, meta):
    """Groups holding only lattice levels q*s + b with both extreme codes
    present: the start reconstructs them exactly (zero error), so no later
    iterate can be strictly better and the result stays lossless."""
    rng = np.random.default_rng(bits)
    qmax = (1 << bits) - 1
    N, K, gs = 8, 256, 64
    s = F32(2.0 ** -7)
    b = (rng.integers(-64, 0, (N, K // gs)) * F32(2.0 ** -7)).astype(F32)
    q = rng.integers(0, qmax + 1, (N, K)).astype(F32)
    q[:, ::gs] = 0
    q[:, 1::gs] = qmax
    W = (q * s + np.repeat(b, gs, axis=1)).astype(F32)
    f = QFormat.affine(bits, gs, meta)
    h = quantize_affine_hqq(W, f)
    assert np.array_equal(oracle.dequant_f64(h, f), W.astype(np.float64))


@pytest.mark.parametrize("dist", ["normal", "laplace"])
@pytest.mark.parametrize("bits", [2, 4])
def test_lp_error_below_minmax(dist, bits):
    rng = np.random.default_rng(7)
    W = (rng.normal(0, 0.02, (64, 1024)) if dist == "normal"
         else rng.laplace(0, 0.015, (64, 1024))).astype(F32)
    f = QFormat.affine(bits, 64, "bf16")
    h = quantize_affine_hqq(W, f)
    p = oracle.quantize(W, f)
    dh = np.abs(W - oracle.dequant_f64(h, f))
    dp = np.abs(W - oracle.dequant_f64(p, f))
    assert np.sum(dh ** 0.7) < 0.99 * np.sum(dp ** 0.7)
    # per group, l1: the kept iterate is never worse than the start (the
    # final meta rounding of the bias can cost a little: allow half a bias
    # ulp times the group size)
    gh = dh.reshape(64, -1, 64).sum(2)
    gp = dp.reshape(64, -1, 64).sum(2)
    bias = oracle.bf16_bits_to_f32(h["biases"]).astype(np.float64)
    slack = 64 * np.abs(bias) * 2.0 ** -8
    assert np.all(gh <= gp + slack)
    assert np.mean(gh < gp) > 0.5


def test_rejects_bad_input():
    W = np.zeros((4, 64), F32)
    with pytest.raises(ValueError):
        quantize_affine_hqq(W, QFormat.q4k())
    with pytest.raises(ValueError):
        quantize_affine_hqq(W, QFormat.affine(4, 64), iters=-1)
    W[0, 0] = np.inf
    with pytest.raises(ValueError):
        quantize_affine_hqq(W, QFormat.affine(4, 64))
