"""GPU parity of the a8w4 path (int8 activations x symmetric int4 weights):
the activation quantizer and the integer forward through the C ABI against
the oracle, bit for bit.

Both sides compute the same thing exactly: the per-token scale and codes
are single IEEE fp32 operations, the dot product is exact in integers and
the two scalings are fp64 in the same order, so the fp32 result rounds the
same fp64 value and the fp16 / bf16 results round that fp32 value (ties to
even) on both sides.
"""
import numpy as np
import pytest

import oracle
from oracle import QFormat
from bit_weight_only_qlinear_amd import synth
from helpers import to_dev_bits, round_out

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_weight_only_qlinear_amd import qlinear
    return qlinear


def _acts(M, K, xdtype, seed):
    """Activations of the workloads' distribution plus edge rows: an all-zero
    token, a token with one large outlier, tiny and large magnitudes."""
    rng = np.random.default_rng(seed)
    xb = synth.draw_activations(rng, M, K, xdtype)
    x = oracle.decode_activations(xb, xdtype).astype(np.float32)
    if M > 1:
        x[1] = 0.0
    if M > 2:
        x[2, K // 3] = 60.0
    if M > 3:
        x[3] *= 2.0 ** -12 if xdtype == "bf16" else 2.0 ** -4
    if M > 4:
        x[4] *= 2.0 ** 20 if xdtype == "bf16" else 2.0 ** 4
    if xdtype == "bf16":
        bits = oracle.f32_to_bf16_bits(x)
    else:
        bits = x.astype(np.float16).view(np.uint16)
    return bits, oracle.decode_activations(bits, xdtype).astype(np.float32)


@pytest.mark.parametrize("xdtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,K", [(1, 128), (7, 1000), (33, 4096), (5, 14336)])
def test_quantize_activations_bit_exact(q, M, K, xdtype):
    bits, x = _acts(M, K, xdtype, seed=M + K)
    xq, xs = q.quantize_activations(to_dev_bits(bits, xdtype))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_activations(x)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), rq)


def _forward(q, N, K, M, ydt, with_bias, seed):
    rng = np.random.default_rng(seed)
    W, _ = synth.draw_weights(rng, N, K, "laplace", 0.0)
    W[0] = 0.0                               # an all-zero channel: scale 0
    d = q.QDesc.sym4(N, K)                   # one scale per output channel
    buf = q.qpack_quantize(d, torch.from_numpy(W).cuda())
    bits, x = _acts(M, K, "bf16", seed + 1)
    xq, xs = q.quantize_activations(to_dev_bits(bits, "bf16"))
    bias = rng.normal(0, 0.1, size=N).astype(np.float32) if with_bias else None
    bd = torch.from_numpy(bias).cuda() if with_bias else None
    y = q.qlinear_forward_a8w4(d, xq, xs, buf, bias=bd, y_dtype=ydt)
    torch.cuda.synchronize()
    qz = oracle.quantize(W, QFormat.sym4(K))
    rq, rs = oracle.quantize_activations(x)
    ref = oracle.linear_a8w4(rq, rs, qz["codes"], qz["scales"][:, 0],
                             None if bias is None else bias.astype(np.float64))
    want = round_out(ref, ydt)
    got = y.float().cpu().numpy().astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (len(bad), bad[:4].tolist())


@pytest.mark.parametrize("ydt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N,K,M", [(1, 128, 1), (33, 384, 3), (130, 1024, 17),
                                   (257, 4096, 40), (64, 14336, 5)])
def test_a8w4_forward_bit_exact(q, N, K, M, ydt):
    _forward(q, N, K, M, ydt, with_bias=(N % 2 == 1), seed=N + M)


def test_a8w4_full_decode(q):
    """The decode layer's shape, 14336 x 4096, at M = 1 and a 16-token tile
    plus a ragged one, every output element."""
    for M in (1, 19):
        _forward(q, 14336, 4096, M, "bf16", with_bias=True, seed=M)


def test_a8w4_rejects(q):
    d = q.QDesc.sym4(64, 256, 64)            # group-wise scales: not a8w4
    buf = q.alloc_weights(d)
    xq = torch.zeros((2, 256), dtype=torch.int8, device="cuda")
    xs = torch.ones(2, dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="one scale per output channel"):
        q.qlinear_forward_a8w4(d, xq, xs, buf)
    d = q.QDesc.sym4(64, 192)                # K % 128 != 0
    buf = q.alloc_weights(d)
    xq = torch.zeros((2, 192), dtype=torch.int8, device="cuda")
    with pytest.raises(RuntimeError, match="K % 128"):
        q.qlinear_forward_a8w4(d, xq, xs, buf)
