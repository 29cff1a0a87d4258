"""GPU parity of the HQQ quantizer (qpack_quantize_hqq) against the oracle
(oracle/hqq.py): packed codes, scales and biases byte for byte, on small
layers of every affine width, group size and metadata type, on sampled rows
of the full int4 decode layer, and a forward over HQQ weights against the
oracle's fp64 product.

HQQ (Half-Quadratic Quantization) is the quantization-parameter option that
ExecuTorch PR #17235's review asks for on the Metal int4 affine weights.
Both sides evaluate |e|^(p-1) in fp64 with their own library pow and round
it to fp32; the two pows may differ in the last fp64 bit, which moves an
fp32 result only if it falls within that bit of an fp32 rounding boundary
(about 2^-29 per evaluation), and a moved W_e must further change a stored
bias or code to show; the byte comparison below holds on every case here."""
import numpy as np
import pytest

import oracle
from oracle import QFormat
from oracle.hqq import quantize_affine_hqq
from oracle.packing import to_buffers
from helpers import gpu_rows, check_linear, to_dev_bits
from bit_weight_only_qlinear_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_weight_only_qlinear_amd import qlinear
    return qlinear


def _expected(W, f, **kw):
    buf = to_buffers(quantize_affine_hqq(W, f, **kw), f)
    return {k: np.ascontiguousarray(v).view(np.uint8).reshape(W.shape[0], -1)
            for k, v in buf.items() if v is not None}


def _weights(rng, N, K, dist):
    W = (rng.normal(0, 0.02, (N, K)) if dist == "normal"
         else rng.laplace(0, 0.015, (N, K))).astype(np.float32)
    W[0, :128] = 0.03125          # constant groups: scale 0
    W[1, :64] = -0.0              # negative zeros
    W[2, 5] = 0.4                 # an outlier
    return W


@pytest.mark.parametrize("bits,gs,meta", [(2, 64, "bf16"), (4, 64, "bf16"), (8, 64, "bf16"),
                                          (4, 32, "f16"), (4, 128, "bf16"), (2, 32, "f16"),
                                          (8, 128, "f16")])
@pytest.mark.parametrize("dist", ["normal", "laplace"])
def test_hqq_bit_exact(q, bits, gs, meta, dist):
    N, K = 97, 1024
    rng = np.random.default_rng(bits * 1000 + gs + (dist == "laplace"))
    W = _weights(rng, N, K, dist)
    f = QFormat.affine(bits, gs, meta)
    d = q.QDesc.affine(N, K, bits, gs, meta)
    buf = q.qpack_quantize_hqq(d, torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    for name, e in _expected(W, f).items():
        assert np.array_equal(gpu_rows(buf[name], N, np.arange(N)), e), name


@pytest.mark.parametrize("iters,p,beta,kappa", [(0, 0.7, 10.0, 1.01), (1, 0.7, 10.0, 1.01),
                                                (5, 0.5, 1.0, 1.1), (50, 0.9, 100.0, 1.0)])
def test_hqq_parameters(q, iters, p, beta, kappa):
    N, K = 64, 512
    rng = np.random.default_rng(iters + 17)
    W = _weights(rng, N, K, "laplace")
    f = QFormat.affine(4, 64, "bf16")
    d = q.QDesc.affine(N, K, 4, 64, "bf16")
    buf = q.qpack_quantize_hqq(d, torch.from_numpy(W).cuda(), iters=iters, lp_norm=p,
                               beta=beta, kappa=kappa)
    torch.cuda.synchronize()
    for name, e in _expected(W, f, iters=iters, p=p, beta=beta, kappa=kappa).items():
        assert np.array_equal(gpu_rows(buf[name], N, np.arange(N)), e), name
    if iters == 0:   # no iteration: the plain min/max quantizer
        plain = q.qpack_quantize(d, torch.from_numpy(W).cuda())
        torch.cuda.synchronize()
        for name in ("qweight", "scales", "zeros"):
            assert torch.equal(plain[name], buf[name]), name


def test_hqq_full_decode_layer(q):
    """The int4 decode layer (K = 4096, N = 14336, outlier columns): the
    whole layer on the GPU, 256 sampled rows against the oracle, then one
    forward of the HQQ layer against the oracle's product on those rows."""
    wl = synth.make("decode_affine", seed=0)
    N, K = wl.W.shape
    f = QFormat.affine(4, 64, "bf16")
    d = q.QDesc.affine(N, K, 4, 64, "bf16")
    buf = q.qpack_quantize_hqq(d, torch.from_numpy(wl.W).cuda())
    x = to_dev_bits(wl.x_bits, "bf16")
    y = q.qlinear_forward(d, x, buf, y_dtype="f32")
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(N, 256, replace=False))
    rows[0] = 0
    rows[-1] = N - 1
    Wr = np.ascontiguousarray(wl.W[rows])
    for name, e in _expected(Wr, f).items():
        assert np.array_equal(gpu_rows(buf[name], N, rows), e), name
    qz = quantize_affine_hqq(Wr, f)
    x64 = oracle.decode_activations(wl.x_bits, "bf16")
    w64 = oracle.dequant_f64(qz, f)
    y_ref = oracle.linear_f64(x64, qz, f, w64=w64)
    yr = y[:, torch.from_numpy(rows).cuda()]
    # max |w'| over the sampled rows only: at most the layer's, so the bound
    # is at most the tolerance's own (stricter, and no GPU value enters it)
    wmax = float(np.abs(w64).max())
    check_linear(yr, y_ref, x64, wmax, K, "f32")
