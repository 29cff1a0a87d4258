"""Pins of the oracle's a8w4 path (int8 activations x symmetric int4
weights): hand-worked tokens and dots, the rounding invariants of the
per-token activation rule, and an exact rational brute force.

Source: ExecuTorch PR #16577, "Arm backend: Support a8w4 for convolution and
linear", description (int4 weights in an int8 container, qmin = -7, qmax = 7;
int8 activations).  The per-token activation rule is a reading (see
oracle/a8w4.py)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import QFormat

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


@pytest.mark.parametrize("case", GOLD["a8w4_activations"], ids=lambda c: c["name"][:24])
def test_activation_quant_golden(case):
    x = np.array([case["x"]], np.float32)
    q, s = oracle.quantize_activations(x)
    assert s.tolist() == [case["s"]]
    assert q.astype(int).tolist() == [case["q"]]
    assert q.dtype == np.int8


@pytest.mark.parametrize("case", GOLD["a8w4_linear"], ids=lambda c: c["name"][:24])
def test_a8w4_linear_golden(case):
    y = oracle.linear_a8w4(np.array(case["xq"], np.int8), np.array(case["xs"], np.float32),
                           np.array(case["wq"], np.int8), np.array(case["ws"], np.float32))
    assert [[Fraction(float(v)) for v in row] for row in y] == \
        [[Fraction(v) for v in row] for row in case["y"]]


def test_activation_quant_invariants():
    """Per token: codes in [-127, 127]; the largest magnitude maps to +-127;
    every element is within half a step of its reconstruction; ties go to
    the even code."""
    rng = np.random.default_rng(4)
    x = rng.normal(size=(64, 512)).astype(np.float32)
    x[3] *= 1e-30                         # tiny token
    x[5] *= 1e20                          # huge token
    x[7, :] = 0.0                         # all-zero token
    x[9, ::3] = 0.0
    q, s = oracle.quantize_activations(x)
    assert s.dtype == np.float32 and q.dtype == np.int8
    assert q.min() >= -127 and q.max() <= 127
    assert s[7] == 0 and not q[7].any()
    rows = [m for m in range(64) if s[m] > 0]
    amax = np.abs(x).argmax(axis=1)
    for m in rows:
        assert abs(int(q[m, amax[m]])) == 127
    xd = oracle.dequantize_activations(q, s)
    err = np.abs(x.astype(np.float64) - xd)
    assert np.all(err[rows] <= 0.5 * s[rows, None].astype(np.float64) * (1 + 2.0 ** -20))
    # the fp32 quotient decides the code: exact ties (x / s == k + 1/2 in
    # fp32) went to the even neighbour
    t = (x / np.where(s == 0, 1, s)[:, None]).astype(np.float32)
    tie = (t - np.floor(t) == 0.5)
    assert np.all(q[tie].astype(int) % 2 == 0)


def test_a8w4_linear_brute_force():
    """The vectorised oracle against exact rational arithmetic, element by
    element, on a tiny shape with the sym4 weights of the oracle's own
    quantizer."""
    rng = np.random.default_rng(8)
    M, N, K = 3, 5, 64
    W = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    qz = oracle.quantize(W, QFormat.sym4(K))
    x = rng.normal(size=(M, K)).astype(np.float32)
    xq, xs = oracle.quantize_activations(x)
    y = oracle.linear_a8w4(xq, xs, qz["codes"], qz["scales"][:, 0])
    for m in range(M):
        for n in range(N):
            acc = sum(int(xq[m, k]) * int(qz["codes"][n, k]) for k in range(K))
            exact = Fraction(acc) * Fraction(float(xs[m])) * Fraction(float(qz["scales"][n, 0]))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_a8w4_approximates_the_float_layer():
    """End to end: quantizing the activations moves each output by at most
    sum_k |w'[n, k]| * s_m / 2 from the layer on the exact activations."""
    rng = np.random.default_rng(9)
    M, N, K = 4, 32, 1024
    W = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    f = QFormat.sym4(K)
    qz = oracle.quantize(W, f)
    x = rng.normal(size=(M, K)).astype(np.float32)
    xq, xs = oracle.quantize_activations(x)
    y = oracle.linear_a8w4(xq, xs, qz["codes"], qz["scales"][:, 0])
    w64 = oracle.dequant_f64(qz, f)
    y_float = oracle.linear_f64(x.astype(np.float64), qz, f, w64=w64)
    bound = 0.5 * xs.astype(np.float64)[:, None] * np.abs(w64).sum(axis=1)[None, :]
    assert np.all(np.abs(y - y_float) <= bound * (1 + 1e-12))
