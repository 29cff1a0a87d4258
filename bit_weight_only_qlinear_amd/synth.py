"""Seeded synthetic workloads (weights and activations), shared by the tests,
the benchmark and the smoke check.  Random draws and dtype casts only: no
quantization arithmetic lives here.

Recipe (every workload): ``numpy.random.default_rng(seed)``, draws in the
order W (fp64 -> fp32), outlier column indices (if any), x (fp64 -> fp32 ->
the activation dtype, round to nearest even via torch's cast).

Workloads, named for what they are:
  tiny_w4a16        M=1,    K=512,  N=256,   W ~ N(0, 0.02),   x fp16
  decode_affine     M=1,    K=4096, N=14336, W ~ N(0, 0.02) with 0.1% of
                    the input columns (4 of 4096) scaled x20, x bf16
  decode_q4k        M=1,    K=5120, N=25600, W ~ Laplace(0, 0.015), x bf16
  decode_8k         M in {1,4,8}, K=8192, N=8192, W ~ N(0, 0.02), x bf16
  prefill_affine    M=2048, K=4096, N=14336, W ~ N(0, 0.02), x bf16
"""
from dataclasses import dataclass

import numpy as np

WORKLOADS = {
    "tiny_w4a16": dict(M=1, K=512, N=256, dist="normal", outliers=0.0,
                       xdtype="f16"),
    "decode_affine": dict(M=1, K=4096, N=14336, dist="normal", outliers=1e-3,
                          xdtype="bf16"),
    "decode_q4k": dict(M=1, K=5120, N=25600, dist="laplace", outliers=0.0,
                       xdtype="bf16"),
    "decode_8k": dict(M=1, K=8192, N=8192, dist="normal", outliers=0.0,
                      xdtype="bf16"),
    "prefill_affine": dict(M=2048, K=4096, N=14336, dist="normal",
                           outliers=0.0, xdtype="bf16"),
}


@dataclass
class Workload:
    W: np.ndarray          # [N, K] float32
    x_bits: np.ndarray     # [M, K] uint16 bit patterns (fp16 or bf16)
    xdtype: str            # 'f16' | 'bf16'
    outlier_cols: np.ndarray


def _cast_bits(x32, xdtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    tt = t.to(torch.float16 if xdtype == "f16" else torch.bfloat16)
    return tt.view(torch.int16).numpy().view(np.uint16).copy()


def draw_weights(rng, N, K, dist="normal", outliers=0.0):
    if dist == "normal":
        W = rng.normal(0.0, 0.02, size=(N, K))
    elif dist == "laplace":
        W = rng.laplace(0.0, 0.015, size=(N, K))
    else:
        raise ValueError(dist)
    W = W.astype(np.float32)
    cols = np.zeros(0, np.int64)
    if outliers > 0:
        cols = rng.choice(K, size=int(round(outliers * K)), replace=False)
        W[:, cols] *= np.float32(20.0)
    return W, cols


def draw_activations(rng, M, K, xdtype="bf16"):
    x = rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    return _cast_bits(x, xdtype)


def make(name, seed=0, M=None, N=None, K=None):
    """Build a named workload (optionally overriding M, N or K, e.g. to
    draw a smaller instance with the same distributions)."""
    p = dict(WORKLOADS[name])
    M = p["M"] if M is None else M
    N = p["N"] if N is None else N
    K = p["K"] if K is None else K
    rng = np.random.default_rng(seed)
    W, cols = draw_weights(rng, N, K, p["dist"], p["outliers"])
    x = draw_activations(rng, M, K, p["xdtype"])
    return Workload(W, x, p["xdtype"], cols)


def random_bias_bits(seed, N, xdtype):
    rng = np.random.default_rng(seed + 1000)
    return _cast_bits(rng.normal(0.0, 0.5, size=(N,)).astype(np.float32),
                      xdtype)
