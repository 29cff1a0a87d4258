"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact for quantize / pack / unpack / dequantize; the linear layer's
output within its tolerance (rel-L2 <= 2e-3, per element
|y - y_ref| <= 1e-2 * ||x_m|| * max|w| / sqrt(K), plus half an output ulp
for fp16/bf16 outputs).  Small shapes span several waves, blocks and ragged
tails; the full workload shapes are checked on sampled rows, which the
oracle can quantize and evaluate on their own (rows are independent).
"""
import numpy as np
import pytest

import oracle
from bit_weight_only_qlinear_amd import synth
from helpers import (f16_weight_bound, qformat_of, to_dev_bits, oracle_buffers, gpu_rows, check_linear,
                     buf_to_np, y_to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_weight_only_qlinear_amd import qlinear
    return qlinear


def _descs(q, N, K):
    D = q.QDesc
    out = [D.affine(N, K, 4, 64, "bf16"), D.affine(N, K, 4, 64, "f16"),
           D.affine(N, K, 2, 64), D.affine(N, K, 8, 64), D.affine(N, K, 4, 32),
           D.affine(N, K, 2, 32, "f16"), D.affine(N, K, 4, 128), D.affine(N, K, 8, 128, "f16"),
           D.sym4(N, K), D.sym4(N, K, 64)]
    if K % 256 == 0:
        out += [D.q4k(N, K), D.q6k(N, K)]
    return out


def _id(d):
    return f"{d.fmt}-b{d.bits}-g{d.group_size}-{d.meta}-N{d.N}-K{d.K}"


def _weights(N, K, seed, dist="laplace"):
    rng = np.random.default_rng(seed)
    W, _ = synth.draw_weights(rng, N, K, dist, 0.0)
    # edge cases inside the matrix: a zero group, a constant group, an
    # all-positive row and an all-negative row
    W[0, :256] = 0.0
    if N > 1:
        W[1, : min(K, 64)] = 0.03125
    if N > 2:
        W[2] = np.abs(W[2])
    if N > 3:
        W[3] = -np.abs(W[3])
    return W


SMALL = [(1, 256), (3, 512), (37, 768), (130, 1280), (300, 5120)]


# ------------------------------------------------------------ quantization
@pytest.mark.parametrize("N,K", SMALL)
def test_quantize_bit_exact(q, N, K):
    W = _weights(N, K, N + K)
    Wd = torch.from_numpy(W).cuda()
    for d in _descs(q, N, K):
        print("quantize", _id(d), flush=True)
        buf = q.qpack_quantize(d, Wd)
        torch.cuda.synchronize()
        ref = oracle_buffers(W, qformat_of(d))
        for name, exp in ref.items():
            got = gpu_rows(buf[name], N, np.arange(N))
            assert np.array_equal(got, exp), f"{_id(d)} {name} differs"


@pytest.mark.parametrize("N,K", [(64, 512), (9, 1536)])
def test_unpack_pack_dequant_bit_exact(q, N, K):
    W = _weights(N, K, 7)
    Wd = torch.from_numpy(W).cuda()
    for d in _descs(q, N, K):
        print("unpack/dequant", _id(d), flush=True)
        f = qformat_of(d)
        qz = oracle.quantize(W, f)
        buf = q.qpack_quantize(d, Wd)
        codes = q.qpack_unpack_codes(d, buf)
        exp = qz["codes"]
        assert np.array_equal(codes.cpu().numpy().view(exp.dtype), exp), _id(d)
        # pack(unpack(words)) == words
        packed = q.qpack_pack_codes(d, codes)
        for name in ("qweight", "qweight_hi"):
            if buf[name] is not None:
                assert torch.equal(packed[name], buf[name]), (_id(d), name)
        for out in ("f32", "f16", "bf16"):
            w = q.qpack_dequantize(d, buf, out)
            e = oracle.dequant_out(qz, f, out)
            got = buf_to_np(w).view(np.float32 if out == "f32" else np.uint16).reshape(N, K)
            assert np.array_equal(got.view(np.uint32 if out == "f32" else np.uint16),
                                  np.ascontiguousarray(e).view(np.uint32 if out == "f32" else np.uint16)), \
                (_id(d), out)


def test_quantize_exhaustive_codes_roundtrip(q):
    """Every code value at every position of a word survives pack -> unpack
    on the GPU (codes generated on the host, oracle-free)."""
    N, K = 16, 512
    for d in _descs(q, N, K):
        f = qformat_of(d)
        vals = np.arange(f.qmin, f.qmax + 1)
        c = np.stack([np.roll(np.resize(vals, K), s) for s in range(N)])
        dt = torch.int8 if f.signed else torch.uint8
        cd = torch.from_numpy(c.astype(np.int8 if f.signed else np.uint8)).cuda()
        packed = q.qpack_pack_codes(d, cd)
        back = q.qpack_unpack_codes(d, packed)
        assert torch.equal(back, cd.to(dt)), _id(d)
        words = oracle.pack_codes(c, f)
        assert np.array_equal(buf_to_np(packed["qweight"]).reshape(N, -1),
                              words["qweight"].view(np.uint8).reshape(N, -1)), _id(d)


# --------------------------------------------------------------- forward
def _forward_case(q, d, M, xdtype, ydt, kernel, seed, with_bias, rows=None, f16_weights=False,
                  workspace="auto"):
    W = _weights(d.N, d.K, seed)
    rng = np.random.default_rng(seed + 1)
    xb = synth.draw_activations(rng, M, d.K, xdtype)
    x64 = oracle.decode_activations(xb, xdtype)
    f = qformat_of(d)
    buf = q.qpack_quantize(d, torch.from_numpy(W).cuda())
    xd = to_dev_bits(xb, xdtype)
    bias_bits = synth.random_bias_bits(seed, d.N, xdtype) if with_bias else None
    bd = to_dev_bits(bias_bits, xdtype) if with_bias else None
    y = q.qlinear_forward(d, xd, buf, bias=bd, y_dtype=ydt, kernel=kernel, workspace=workspace)
    torch.cuda.synchronize()
    qz = oracle.quantize(W, f)
    w64 = oracle.dequant_f64(qz, f)
    b64 = oracle.decode_activations(bias_bits, xdtype) if with_bias else None
    y_ref = oracle.linear_f64(x64, qz, f, b64, w64=w64)
    extra = f16_weight_bound(x64, w64) if f16_weights else None
    return check_linear(y, y_ref, x64, np.abs(w64).max(), d.K, ydt, extra=extra)


GEMV_SHAPES = [(1, 256), (3, 512), (77, 1024), (300, 4096), (513, 5120), (64, 8192)]


@pytest.mark.parametrize("N,K", GEMV_SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8])
def test_gemv_forward(q, N, K, M):
    for i, d in enumerate(_descs(q, N, K)):
        for xdt, ydt in [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16")]:
            print("gemv", _id(d), M, xdt, ydt, flush=True)
            _forward_case(q, d, M, xdt, ydt, q.QP_KERNEL_GEMV, seed=N * 31 + K + M + i,
                          with_bias=(i % 2 == 0))


@pytest.mark.parametrize("N,K", [(1, 256), (31, 384), (77, 1024), (300, 4096), (513, 5120)])
@pytest.mark.parametrize("M", [1, 3, 4, 5, 8, 11, 16])
def test_gemv_mfma_forward(q, N, K, M):
    """The skinny MFMA decode kernel on every format, ragged N, M up to 16."""
    for i, d in enumerate(_descs(q, N, K)):
        if K % 256 and d.fmt in ("q4k", "q6k"):
            continue
        for xdt, ydt in [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16")]:
            print("gemv_mfma", _id(d), M, xdt, ydt, flush=True)
            _forward_case(q, d, M, xdt, ydt, q.QP_KERNEL_GEMV_MFMA, seed=N * 37 + K + M + i,
                          with_bias=(i % 2 == 1))


@pytest.mark.parametrize("fmt", ["affine32", "q4k", "q6k", "sym4g32"])
def test_gemv_mfma_large_k(q, fmt):
    """K = 32768: a block's metadata no longer fits LDS, so the MFMA qGEMV
    reads it per step from HBM (the other code path of the kernel).  At this
    K the fp16 rounding of the weights can exceed the layer's element bound,
    so the MFMA kernels are held to it plus the fp16-weight bound.  The
    exact-code qGEMV's register plan stops short of this K, so AUTO picks an
    fp16-weight kernel here as well."""
    N, K = 40, 32768
    d = {"affine32": q.QDesc.affine(N, K, 4, 32, "bf16"), "q4k": q.QDesc.q4k(N, K),
         "q6k": q.QDesc.q6k(N, K), "sym4g32": q.QDesc.sym4(N, K, 32)}[fmt]
    for M in (4, 9):
        print("gemv_mfma large K", _id(d), M, flush=True)
        _forward_case(q, d, M, "bf16", "f32", q.QP_KERNEL_GEMV_MFMA, seed=M + 7, with_bias=True,
                      f16_weights=True)
        _forward_case(q, d, M, "bf16", "bf16", q.QP_KERNEL_AUTO, seed=M + 8, with_bias=False,
                      f16_weights=True)


@pytest.mark.parametrize("gs", [32, 128])
@pytest.mark.parametrize("N,K,M", [(130, 512, 9), (257, 1536, 300)])
def test_gemm_sym4_group_sizes(q, gs, N, K, M):
    """Group-wise SYM4 group sizes outside the common descriptor list."""
    d = q.QDesc.sym4(N, K, gs)
    for ws in ("auto", None):
        print("gemm sym4", _id(d), M, ws, flush=True)
        _forward_case(q, d, M, "bf16", "f32", q.QP_KERNEL_GEMM, seed=gs + M, with_bias=True,
                      workspace=ws)


@pytest.mark.parametrize("fmt", ["affine64", "affine32", "affine128", "q4k", "q6k", "sym4",
                                 "sym4g32", "sym4g128"])
def test_gemm_large_k(q, fmt):
    """K = 32768 (512 steps): the qGEMM's metadata chunk rings and staged
    activation offsets cycle many times; both tilings, fp16-weight bound."""
    N, K, M = 300, 32768, 40
    d = {"affine64": q.QDesc.affine(N, K, 4, 64, "bf16"), "affine32": q.QDesc.affine(N, K, 4, 32),
         "affine128": q.QDesc.affine(N, K, 8, 128, "f16"),
         "q4k": q.QDesc.q4k(N, K), "q6k": q.QDesc.q6k(N, K), "sym4": q.QDesc.sym4(N, K),
         "sym4g32": q.QDesc.sym4(N, K, 32), "sym4g128": q.QDesc.sym4(N, K, 128)}[fmt]
    for ws in ("auto", None):
        print("gemm large K", _id(d), M, ws, flush=True)
        _forward_case(q, d, M, "bf16", "f32", q.QP_KERNEL_GEMM, seed=3, with_bias=True,
                      f16_weights=True, workspace=ws)


@pytest.mark.parametrize("N,K", [(1, 256), (130, 512), (257, 1280), (64, 4096), (520, 768),
                                 (72, 1536)])
@pytest.mark.parametrize("M", [1, 9, 64, 130, 300])
def test_gemm_forward(q, N, K, M):
    for i, d in enumerate(_descs(q, N, K)):
        if K % 64:
            continue
        for xdt, ydt in [("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16")]:
            for ws in ("auto", None):   # 224-row tiles where they pay, 256-row tiles
                print("gemm", _id(d), M, xdt, ydt, ws, flush=True)
                _forward_case(q, d, M, xdt, ydt, q.QP_KERNEL_GEMM, seed=N * 17 + K + M + i,
                              with_bias=(i % 2 == 1), workspace=ws)


@pytest.mark.parametrize("N,K,M", [(130, 512, 1), (257, 1280, 33), (520, 768, 300),
                                   (64, 4096, 257)])
def test_gemm_workspace_tilings_agree(q, N, K, M):
    """224-row tiles (staged activations) and 256-row tiles: same fp16
    operands, fp32 sums in another order; a workspace full of NaN bytes
    checks that the staging writes every byte the kernel reads."""
    for i, d in enumerate(_descs(q, N, K)):
        for xdt in ("bf16", "f16"):
            print("gemm workspace", _id(d), M, xdt, flush=True)
            W = _weights(N, K, 5 + i)
            xb = synth.draw_activations(np.random.default_rng(M + i), M, K, xdt)
            buf = q.qpack_quantize(d, torch.from_numpy(W).cuda())
            xd = to_dev_bits(xb, xdt)
            nb = q.workspace_bytes(d, M, xdt, q.QP_KERNEL_GEMM)
            assert nb == (M + 15) // 16 * 16 * K * 2
            ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
            y0 = q.qlinear_forward(d, xd, buf, y_dtype="f32", kernel=q.QP_KERNEL_GEMM,
                                   workspace=None)
            y1 = q.qlinear_forward(d, xd, buf, y_dtype="f32", kernel=q.QP_KERNEL_GEMM,
                                   workspace=ws)
            y2 = q.qlinear_forward(d, xd, buf, y_dtype="f32", kernel=q.QP_KERNEL_GEMM)
            torch.cuda.synchronize()
            assert torch.isfinite(y1).all()
            assert torch.equal(y1, y2)
            # |difference| <= K * 2^-23 * sum |w x| bounds two fp32 summation orders
            wd = q.qpack_dequantize(d, buf, "f16").float()
            xf = xd.float()
            bound = K * 2.0 ** -23 * (xf.abs() @ wd.abs().T) + 1e-30
            assert ((y0 - y1).abs() <= bound).all()


@pytest.mark.parametrize("M,kernel,ws", [(1, 0, "auto"), (8, 3, "auto"), (300, 2, "auto"),
                                          (300, 2, None)])
def test_graph_replay_matches_eager(q, M, kernel, ws):
    """A captured forward (the qGEMM's workspace is allocated inside the
    capture, from the graph's pool) replayed several times, with eager work
    and synchronizations in between, gives the eager result bit for bit."""
    d = q.QDesc.affine(520, 1024, 4, 64, "bf16")
    W = _weights(d.N, d.K, 11)
    buf = q.qpack_quantize(d, torch.from_numpy(W).cuda())
    xd = to_dev_bits(synth.draw_activations(np.random.default_rng(M), M, d.K, "bf16"), "bf16")
    ref = q.qlinear_forward(d, xd, buf, kernel=kernel, workspace=ws)
    torch.cuda.synchronize()
    y = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.qlinear_forward(d, xd, buf, kernel=kernel, out=y, workspace=ws)   # warm-up
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qlinear_forward(d, xd, buf, kernel=kernel, out=y, workspace=ws)
    other = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        y.fill_(float("nan"))
        other.add_(1.0)                      # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep


def test_auto_dispatch_matches(q):
    d = q.QDesc.affine(200, 1024)
    for M in (1, 8, 9, 33):
        _forward_case(q, d, M, "bf16", "f32", q.QP_KERNEL_AUTO, seed=M, with_bias=True)


# ------------------------------------------------- full workload shapes
def _full(q, name, d, M, kernel, ydt, xdtype, nsample=384):
    print("full", name, _id(d), M, flush=True)
    wl = synth.make(name, seed=0, M=M)
    W = wl.W
    N, K = W.shape
    f = qformat_of(d)
    Wd = torch.from_numpy(W).cuda()
    buf = q.qpack_quantize(d, Wd)
    xd = to_dev_bits(wl.x_bits, xdtype)
    y = q.qlinear_forward(d, xd, buf, y_dtype=ydt, kernel=kernel)
    torch.cuda.synchronize()
    rng = np.random.default_rng(123)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, nsample, replace=False)]))
    # bit-exact packed buffers on the sampled rows
    ref = oracle_buffers(W[rows], f)
    for bname, exp in ref.items():
        assert np.array_equal(gpu_rows(buf[bname], N, rows), exp), (name, bname)
    # output on the sampled rows (columns n of y)
    qz = oracle.quantize(W[rows], f)
    x64 = oracle.decode_activations(wl.x_bits, xdtype)
    w64 = oracle.dequant_f64(qz, f)
    y_ref = oracle.linear_f64(x64, qz, f, w64=w64)
    ys = y[:, torch.from_numpy(rows).cuda()]
    # max|w| over the whole layer: sampled rows give a lower bound, so use
    # the GPU dequantized layer's exact maximum
    wmax = float(q.qpack_dequantize(d, buf, "f32").abs().max())
    return check_linear(ys, y_ref, x64, wmax, K, ydt)


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_full_decode_affine(q, bits):
    d = q.QDesc.affine(14336, 4096, bits, 64, "bf16")
    _full(q, "decode_affine", d, 1, q.QP_KERNEL_AUTO, "bf16", "bf16")
    _full(q, "decode_affine", d, 1, q.QP_KERNEL_AUTO, "f32", "bf16")


def test_full_tiny(q):
    d = q.QDesc.affine(256, 512, 4, 64, "f16")
    _full(q, "tiny_w4a16", d, 1, q.QP_KERNEL_AUTO, "f16", "f16", nsample=254)


def test_full_decode_q4k(q):
    d = q.QDesc.q4k(25600, 5120)
    _full(q, "decode_q4k", d, 1, q.QP_KERNEL_AUTO, "bf16", "bf16")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_full_decode_8k(q, M):
    _full(q, "decode_8k", q.QDesc.q6k(8192, 8192), M, q.QP_KERNEL_AUTO, "bf16", "bf16")
    _full(q, "decode_8k", q.QDesc.sym4(8192, 8192), M, q.QP_KERNEL_AUTO, "bf16", "bf16")


def test_full_prefill(q):
    d = q.QDesc.affine(14336, 4096, 4, 64, "bf16")
    _full(q, "prefill_affine", d, 2048, q.QP_KERNEL_AUTO, "bf16", "bf16", nsample=128)
