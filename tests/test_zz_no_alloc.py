"""The allocation-free forward (qlinear_forward_static) against the
workspace forward (qlinear_forward_ws) on the same inputs: two calls in a
row, the second smaller, both bit-identical to the workspace call (same
kernels, same staging); and the size limit of the static scratch."""
import numpy as np
import pytest

from bit_weight_only_qlinear_amd import synth
from helpers import to_dev_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_weight_only_qlinear_amd import qlinear
    return qlinear


def _case(q, d, M, seed, ydt=torch.bfloat16, kernel=0, with_bias=True):
    rng = np.random.default_rng(seed)
    W, _ = synth.draw_weights(rng, d.N, d.K, "normal", 1e-3)
    buf = q.qpack_quantize(d, torch.from_numpy(W).cuda())
    x = to_dev_bits(synth.draw_activations(rng, M, d.K, "bf16"), "bf16")
    bias = to_dev_bits(synth.random_bias_bits(seed, d.N, "bf16"), "bf16") if with_bias else None
    return buf, x, bias


def test_static_matches_workspace_twice(q):
    """A staged qGEMM call, then a smaller one reusing the scratch."""
    cases = [(q.QDesc.affine(1792, 4096, 4, 64, "bf16"), 2048),
             (q.QDesc.q4k(1000, 1024), 300)]
    for i, (d, M) in enumerate(cases):
        assert q.workspace_bytes(d, M, "bf16", q.QP_KERNEL_AUTO) > 0   # staged path
        print("static vs ws", d.fmt, d.N, d.K, M, flush=True)
        buf, x, bias = _case(q, d, M, seed=11 + i)
        ref = q.qlinear_forward(d, x, buf, bias=bias, y_dtype="bf16", workspace="auto")
        out = torch.full((M, d.N), float("nan"), dtype=torch.bfloat16, device="cuda")
        q.qlinear_forward_static(d, x, buf, out, bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_static_other_kernels_and_limit(q):
    """The other kernel choices (qGEMV, MFMA qGEMV, a small qGEMM) give the
    workspace call's result; a staging need past the scratch is refused
    before anything is enqueued."""
    d = q.QDesc.affine(512, 2048, 4, 64, "bf16")
    for M, kernel in ((1, q.QP_KERNEL_AUTO), (12, q.QP_KERNEL_AUTO), (64, q.QP_KERNEL_GEMM)):
        print("static other kernels", M, kernel, flush=True)
        buf, x, bias = _case(q, d, M, seed=M)
        ref = q.qlinear_forward(d, x, buf, bias=bias, y_dtype="f32", kernel=kernel,
                                workspace="auto")
        out = torch.empty((M, d.N), dtype=torch.float32, device="cuda")
        q.qlinear_forward_static(d, x, buf, out, bias=bias, kernel=kernel)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    big = q.QDesc.affine(14336, 8192, 4, 64, "bf16")
    M = 4096
    assert q.workspace_bytes(big, M, "bf16", q.QP_KERNEL_AUTO) > 40 << 20
    w = q.alloc_weights(big)
    x = torch.zeros((M, big.K), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, big.N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q.QLinearError) as e:
        q.qlinear_forward_static(big, x, w, out)
    assert e.value.status == q.QP_EUNSUPPORTED and "static scratch" in str(e.value)
