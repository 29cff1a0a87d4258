"""GPU parity of the plain int4 / int6 -> nested Q4K / Q6K conversion
(qpack_pack_codes + qpack_encode_nested) against the oracle: every metadata
and code byte bit-exact, the converted layer's output against the oracle's
fp64 product, and the invalid-input flag; and of the fused-N concatenation
(qpack_concat_n): the stacked buffers against the oracle's packing of the
stacked W, and one forward over them."""
import numpy as np
import pytest

import oracle
from oracle import QFormat
from oracle.convert import to_q4k, to_q6k
from helpers import oracle_buffers, gpu_rows, check_linear, to_dev_bits
from bit_weight_only_qlinear_amd import synth
from oracle.packing import to_buffers

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_weight_only_qlinear_amd import qlinear
    return qlinear


def _bytes(buf):
    out = {}
    for k, v in buf.items():
        if v is not None:
            out[k] = np.ascontiguousarray(v).view(np.uint8).reshape(v.shape[0], -1)
    return out


def _plain4(rng, N, K):
    s = rng.uniform(0, 0.01, size=(N, K // 32)).astype(np.float32)
    z = rng.uniform(0, 15, size=(N, K // 32)).astype(np.float32)
    s[0, :8] = 0.0                         # an all-zero super-block: step 0
    z[0, 8:16] = 0.0
    if N > 1:
        s[1, :8] = np.float32(2.0 ** -20)  # equal tiny values: the fp16 step underflows to 0
    z[min(2, N - 1), 8:16] = 15.0
    u = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    return u, s, z


@pytest.mark.parametrize("N,K", [(1, 256), (37, 768), (300, 5120)])
def test_convert_q4k_bit_exact(q, N, K):
    rng = np.random.default_rng(N + K)
    u, s, z = _plain4(rng, N, K)
    d = q.QDesc.q4k(N, K)
    buf, bad = q.convert_to_nested(d, torch.from_numpy(u).cuda(), torch.from_numpy(s).cuda(),
                                   torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    assert int(bad[0]) == 0
    exp = _bytes(to_buffers(to_q4k(u, s, z), QFormat.q4k()))
    for name, e in exp.items():
        assert np.array_equal(gpu_rows(buf[name], N, np.arange(N)), e), name


@pytest.mark.parametrize("N,K", [(1, 256), (37, 768), (300, 5120)])
def test_convert_q6k_bit_exact(q, N, K):
    rng = np.random.default_rng(N * K)
    s = rng.uniform(0, 0.02, size=(N, K // 16)).astype(np.float32)
    s[0, :16] = 0.0
    qc = rng.integers(-32, 32, size=(N, K)).astype(np.int8)
    d = q.QDesc.q6k(N, K)
    buf, bad = q.convert_to_nested(d, torch.from_numpy(qc).cuda(), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    assert int(bad[0]) == 0
    exp = _bytes(to_buffers(to_q6k(qc, s), QFormat.q6k()))
    for name, e in exp.items():
        assert np.array_equal(gpu_rows(buf[name], N, np.arange(N)), e), name


def test_converted_layer_forward(q):
    """The plain form of a Laplace layer, converted on the GPU, then run: the
    output against the oracle's product of the converted weights."""
    N, K, M = 512, 4096, 4
    rng = np.random.default_rng(7)
    W = rng.laplace(0, 0.015, size=(N, K)).astype(np.float32)
    plain = oracle.quantize(W, QFormat.q4k())          # holds the plain (codes, s, z)
    d = q.QDesc.q4k(N, K)
    buf, bad = q.convert_to_nested(d, torch.from_numpy(plain["codes"]).cuda(),
                                   torch.from_numpy(plain["s"]).cuda(),
                                   torch.from_numpy(plain["z"]).cuda())
    xb = synth.draw_activations(rng, M, K, "bf16")
    y = q.qlinear_forward(d, to_dev_bits(xb, "bf16"), buf, y_dtype="f32")
    torch.cuda.synchronize()
    assert int(bad[0]) == 0
    qz = to_q4k(plain["codes"], plain["s"], plain["z"])
    x64 = oracle.decode_activations(xb, "bf16")
    w64 = oracle.dequant_f64(qz, QFormat.q4k())
    check_linear(y, oracle.linear_f64(x64, qz, QFormat.q4k(), w64=w64), x64, np.abs(w64).max(),
                 K, "f32")


def test_convert_flags_invalid_inputs(q):
    N, K = 4, 256
    rng = np.random.default_rng(9)
    u, s, z = _plain4(rng, N, K)
    s[3, 2] = -1e-3
    z[2, 5] = np.nan
    buf, bad = q.convert_to_nested(q.QDesc.q4k(N, K), torch.from_numpy(u).cuda(),
                                   torch.from_numpy(s).cuda(), torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    assert int(bad[0]) == 1
    # the invalid values were encoded as 0; the rest as the oracle does
    s2, z2 = s.copy(), z.copy()
    s2[3, 2] = 0.0
    z2[2, 5] = 0.0
    exp = _bytes(to_buffers(to_q4k(u, s2, z2), QFormat.q4k()))
    for name, e in exp.items():
        assert np.array_equal(gpu_rows(buf[name], N, np.arange(N)), e), name
    with pytest.raises(q.QLinearError):
        q.convert_to_nested(q.QDesc.affine(N, K), torch.from_numpy(u).cuda(),
                            torch.from_numpy(s).cuda(), torch.from_numpy(z).cuda())


@pytest.mark.parametrize("fmt", ["affine", "q4k", "q6k", "sym4"])
def test_concat_n(q, fmt):
    K = 1024
    Ns = (100, 37, 256)
    rng = np.random.default_rng(11)
    Ws = [rng.normal(0, 0.02, size=(n, K)).astype(np.float32) for n in Ns]
    mk = {"affine": lambda n: q.QDesc.affine(n, K, 4, 64, "bf16"), "q4k": lambda n: q.QDesc.q4k(n, K),
          "q6k": lambda n: q.QDesc.q6k(n, K), "sym4": lambda n: q.QDesc.sym4(n, K)}[fmt]
    descs = [mk(n) for n in Ns]
    bufs = [q.qpack_quantize(d, torch.from_numpy(W).cuda()) for d, W in zip(descs, Ws)]
    dout, out = q.concat_n(descs, bufs)
    W = np.vstack(Ws)
    N = W.shape[0]
    assert dout.N == N
    f = {"affine": QFormat.affine(4, 64, "bf16"), "q4k": QFormat.q4k(), "q6k": QFormat.q6k(),
         "sym4": QFormat.sym4(K)}[fmt]
    for name, e in oracle_buffers(W, f).items():
        assert np.array_equal(gpu_rows(out[name], N, np.arange(N)), e), name
    M = 3
    xb = synth.draw_activations(rng, M, K, "bf16")
    y = q.qlinear_forward(dout, to_dev_bits(xb, "bf16"), out, y_dtype="f32")
    torch.cuda.synchronize()
    qz = oracle.quantize(W, f)
    x64 = oracle.decode_activations(xb, "bf16")
    w64 = oracle.dequant_f64(qz, f)
    check_linear(y, oracle.linear_f64(x64, qz, f, w64=w64), x64, np.abs(w64).max(), K, "f32")
