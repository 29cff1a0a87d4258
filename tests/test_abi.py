"""C-ABI checks that need no GPU: the library loads, exports every entry
point declared in include/qlinear.h, and validates arguments on the host
(every error path returns a status and a message before any launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q():
    from bit_weight_only_qlinear_amd import qlinear
    return qlinear


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qlinear.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(q):
    names = declared_functions()
    assert set(names) == set(q.EXPORTED)
    for n in names:
        assert hasattr(q.lib, n)
    assert q.lib.qpack_abi_version() == 1


def test_sizes_and_bpw(q):
    D = q.QDesc
    cases = [(D.q4k(256, 4096), 4.625), (D.q6k(256, 4096), 6.5625),
             (D.affine(256, 4096, 4, 64), 4.5), (D.affine(256, 4096, 2, 64), 2.5),
             (D.affine(256, 4096, 8, 64), 8.5), (D.sym4(256, 4096), 4 + 32 / 4096)]
    for d, bpw in cases:
        s = q.qpack_sizes(d)
        assert 8 * sum(s.values()) / (d.N * d.K) == bpw


def test_sizes_match_oracle(q):
    import oracle
    from helpers import qformat_of
    D = q.QDesc
    for d in [D.q4k(7, 512), D.q6k(3, 768), D.affine(5, 640, 2, 32, "f16"),
              D.affine(9, 384, 8, 128), D.sym4(4, 96), D.sym4(4, 256, 64)]:
        assert q.qpack_sizes(d) == oracle.buffer_bytes(qformat_of(d), d.N, d.K)


FAKE = 1 << 20   # an aligned, never-dereferenced address (validation fails first)


def _call_forward(q, desc, x=FAKE, xdt=1, M=1, w=None, bias=None, y=FAKE, ydt=1, kernel=0):
    d = desc.c() if hasattr(desc, "c") else desc
    if w is None:
        w = q._Weights(FAKE, FAKE, FAKE, FAKE, FAKE)
    return q.lib.qlinear_forward_kernel(ctypes.byref(d), ctypes.c_void_p(x), xdt, M,
                                        ctypes.byref(w), ctypes.c_void_p(bias),
                                        ctypes.c_void_p(y), ydt, kernel, None)


def _err(q):
    return q.lib.qpack_last_error().decode()


@pytest.mark.parametrize("desc,status,msg", [
    (dict(fmt=0, bits=3, group_size=64, N=8, K=512), 3, "bits"),
    (dict(fmt=0, bits=4, group_size=48, N=8, K=480), 3, "group_size"),
    (dict(fmt=0, bits=4, group_size=64, N=8, K=500), 2, "multiple"),
    (dict(fmt=0, bits=2, group_size=32, N=8, K=96), 2, "16-byte"),
    (dict(fmt=0, bits=4, group_size=64, N=0, K=512), 2, "positive"),
    (dict(fmt=0, bits=4, group_size=64, N=8, K=512, meta=2), 3, "meta_dtype"),
    (dict(fmt=0, bits=4, group_size=64, N=8, K=512, sb=256), 1, "super"),
    (dict(fmt=1, bits=4, group_size=32, N=8, K=384, sb=256), 2, "256"),
    (dict(fmt=1, bits=4, group_size=64, N=8, K=512, sb=256), 3, "Q4K"),
    (dict(fmt=2, bits=6, group_size=32, N=8, K=512, sb=256), 3, "Q6K"),
    (dict(fmt=2, bits=6, group_size=16, N=8, K=272, sb=256), 2, "256"),
    (dict(fmt=3, bits=4, group_size=48, N=8, K=96), 3, "SYM4"),
    (dict(fmt=3, bits=4, group_size=96, N=8, K=100), 2, "32"),
    (dict(fmt=7, bits=4, group_size=64, N=8, K=512), 1, "format"),
    (dict(fmt=0, bits=4, group_size=64, N=8, K=512, reserved=1), 1, "reserved"),
])
def test_descriptor_validation(q, desc, status, msg):
    d = q._Desc(desc["fmt"], desc["bits"], desc["group_size"], desc.get("sb", 0),
                desc.get("meta", 1), desc.get("reserved", 0), desc["N"], desc["K"])
    out = (ctypes.c_size_t * 5)()
    st = q.lib.qpack_sizes(ctypes.byref(d), out)
    assert st == status, _err(q)
    assert msg.lower() in _err(q).lower()
    # the same check guards every entry point that takes a descriptor
    assert _call_forward(q, d) == status


def test_forward_argument_validation(q):
    d = q.QDesc.affine(64, 512)
    assert _call_forward(q, d, M=0) == q.QP_ESHAPE and "M" in _err(q)
    assert _call_forward(q, d, xdt=2) == q.QP_EINVAL and "x_dtype" in _err(q)
    assert _call_forward(q, d, ydt=5) == q.QP_EINVAL and "y_dtype" in _err(q)
    assert _call_forward(q, d, x=0) == q.QP_EINVAL and "x is NULL" in _err(q)
    assert _call_forward(q, d, y=0) == q.QP_EINVAL and "y is NULL" in _err(q)
    assert _call_forward(q, d, x=FAKE + 2) == q.QP_EALIGN and "aligned" in _err(q)
    assert _call_forward(q, d, bias=FAKE + 8) == q.QP_EALIGN
    assert _call_forward(q, d, kernel=9) == q.QP_EINVAL and "kernel" in _err(q)
    w = q._Weights(FAKE, None, None, FAKE, None)
    assert _call_forward(q, d, w=w) == q.QP_EINVAL and "scales" in _err(q)
    w = q._Weights(FAKE + 4, None, FAKE, FAKE, None)
    assert _call_forward(q, d, w=w) == q.QP_EALIGN and "qweight" in _err(q)
    # the nested formats need their step buffer
    w = q._Weights(FAKE, None, FAKE, FAKE, None)
    assert _call_forward(q, q.QDesc.q4k(64, 512), w=w) == q.QP_EINVAL and "steps" in _err(q)
    w = q._Weights(FAKE, None, FAKE, None, FAKE)
    assert _call_forward(q, q.QDesc.q6k(64, 512), w=w) == q.QP_EINVAL and "qweight_hi" in _err(q)
    # the qGEMM (fp16-rounded weights) needs K % 64 == 0 and K <= 8192, where
    # it meets the output bound
    assert _call_forward(q, q.QDesc.affine(8, 96, 4, 32), kernel=2) == q.QP_EUNSUPPORTED
    assert _call_forward(q, q.QDesc.affine(8, 16384, 4, 64), M=64,
                         kernel=2) == q.QP_EUNSUPPORTED and "8192" in _err(q)
    # the MFMA qGEMV needs K % 128 == 0 (any M: tiles of 16 activation rows)
    assert _call_forward(q, q.QDesc.affine(8, 192, 4, 64), M=4,
                         kernel=q.QP_KERNEL_GEMV_MFMA) == q.QP_EUNSUPPORTED
    assert "K % 128" in _err(q)


def test_other_entry_points_validate(q):
    d = q.QDesc.affine(64, 512).c()
    w = q._Weights(FAKE, None, FAKE, FAKE, None)
    assert q.lib.qpack_quantize(ctypes.byref(d), None, ctypes.byref(w), None) == q.QP_EINVAL
    assert q.lib.qpack_quantize(ctypes.byref(d), ctypes.c_void_p(FAKE + 4), ctypes.byref(w),
                                None) == q.QP_EALIGN
    assert q.lib.qpack_unpack_codes(ctypes.byref(d), ctypes.byref(w), None, None) == q.QP_EINVAL
    assert q.lib.qpack_pack_codes(ctypes.byref(d), None, ctypes.byref(w), None) == q.QP_EINVAL
    assert q.lib.qpack_dequantize(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(FAKE), 7,
                                  None) == q.QP_EINVAL
    assert "out_dtype" in _err(q)
    assert q.lib.qpack_sizes(None, None) == q.QP_EINVAL
    assert q.lib.qpack_sizes(ctypes.byref(d), None) == q.QP_EINVAL


def test_concat_and_encode_validate(q):
    """Host-side checks of qpack_concat_n and qpack_encode_nested (no
    device access: validation fails first)."""
    w = q._Weights(FAKE, None, FAKE, FAKE, None)
    parts = [q.QDesc.affine(64, 512), q.QDesc.affine(32, 512)]
    dins = (q._Desc * 2)(*[p.c() for p in parts])
    wins = (q._Weights * 2)(w, w)
    good = q.QDesc.affine(96, 512).c()
    assert q.lib.qpack_concat_n(ctypes.byref(good), 0, dins, wins, ctypes.byref(w),
                                None) == q.QP_EINVAL
    bad_n = q.QDesc.affine(100, 512).c()
    assert q.lib.qpack_concat_n(ctypes.byref(bad_n), 2, dins, wins, ctypes.byref(w),
                                None) == q.QP_ESHAPE and "add up" in _err(q)
    other_k = (q._Desc * 2)(parts[0].c(), q.QDesc.affine(32, 1024).c())
    assert q.lib.qpack_concat_n(ctypes.byref(good), 2, other_k, wins, ctypes.byref(w),
                                None) == q.QP_EINVAL and "differs" in _err(q)
    d4 = q.QDesc.q4k(64, 512).c()
    w4 = q._Weights(FAKE, None, FAKE, FAKE, FAKE)
    S = ctypes.c_void_p(FAKE)
    assert q.lib.qpack_encode_nested(ctypes.byref(d4), S, None, ctypes.byref(w4), None,
                                     None) == q.QP_EINVAL and "zero points" in _err(q)
    assert q.lib.qpack_encode_nested(ctypes.byref(q.QDesc.affine(64, 512).c()), S, S,
                                     ctypes.byref(w4), None, None) == q.QP_EUNSUPPORTED
    d6 = q.QDesc.q6k(64, 512).c()
    assert q.lib.qpack_encode_nested(ctypes.byref(d6), S, S, ctypes.byref(w4), None,
                                     None) == q.QP_EINVAL
    assert q.lib.qpack_encode_nested(ctypes.byref(d4), ctypes.c_void_p(FAKE + 4), S,
                                     ctypes.byref(w4), None, None) == q.QP_EALIGN


def test_quantize_hqq_validates(q):
    """Host-side checks of qpack_quantize_hqq (no device access)."""
    w = q._Weights(FAKE, None, FAKE, FAKE, None)
    W = ctypes.c_void_p(FAKE)
    d = q.QDesc.affine(64, 512).c()

    def call(desc=d, Wp=W, iters=20, p=0.7, beta=10.0, kappa=1.01):
        return q.lib.qpack_quantize_hqq(ctypes.byref(desc), Wp, ctypes.byref(w), iters, p, beta,
                                        kappa, None)
    assert call(desc=q.QDesc.q4k(64, 512).c()) == q.QP_EUNSUPPORTED and "AFFINE" in _err(q)
    assert call(iters=-1) == q.QP_EINVAL and "iters" in _err(q)
    assert call(iters=10001) == q.QP_EINVAL
    assert call(p=0.0) == q.QP_EINVAL and "lp_norm" in _err(q)
    assert call(p=1.5) == q.QP_EINVAL
    assert call(beta=0.0) == q.QP_EINVAL and "beta" in _err(q)
    assert call(beta=float("inf")) == q.QP_EINVAL
    assert call(kappa=float("nan")) == q.QP_EINVAL and "kappa" in _err(q)
    assert call(Wp=None) == q.QP_EINVAL
    assert call(Wp=ctypes.c_void_p(FAKE + 4)) == q.QP_EALIGN
    bad = q.QDesc.affine(64, 500).c()
    assert call(desc=bad) != q.QP_OK


def test_workspace_query_and_checks(q):
    n = ctypes.c_size_t(7)
    d = q.QDesc.affine(64, 512).c()
    # qGEMM: M rounded up to 16 rows of K fp16; other kernels take none
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(d), 1, 300, 2, ctypes.byref(n)) == q.QP_OK
    assert n.value == 304 * 512 * 2 + 304 * 4
    # 8192 rows at M = 2048: 256 blocks of 256 rows (one wave) beat 296
    # blocks of 224 rows (two waves): no workspace
    d8 = q.QDesc.affine(8192, 512).c()
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(d8), 1, 2048, 0, ctypes.byref(n)) == q.QP_OK
    assert n.value == 0
    # 14336 rows at M = 2048: 512 blocks of 224 rows beat 448 of 256
    d14 = q.QDesc.affine(14336, 4096).c()
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(d14), 1, 2048, 0, ctypes.byref(n)) == q.QP_OK
    assert n.value == 2048 * 4096 * 2 + 2048 * 4
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(d), 1, 1, 0, ctypes.byref(n)) == q.QP_OK
    assert n.value == 0
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(d), 1, 4, 1, ctypes.byref(n)) == q.QP_OK
    assert n.value == 0
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(d), 1, 0, 2, ctypes.byref(n)) == q.QP_ESHAPE
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(d), 1, 64, 2, None) == q.QP_EINVAL
    # past 2^31 staged bytes the qGEMM runs without a workspace
    big = q.QDesc.affine(64, 8192).c()
    assert q.lib.qlinear_workspace_bytes(ctypes.byref(big), 1, 1 << 18, 2,
                                         ctypes.byref(n)) == q.QP_OK
    assert n.value == 0
    w = q._Weights(FAKE, None, FAKE, FAKE, None)

    def fwd(ws, nbytes, M=64, kernel=2):
        return q.lib.qlinear_forward_ws(ctypes.byref(d), ctypes.c_void_p(FAKE), 1, M,
                                        ctypes.byref(w), None, ctypes.c_void_p(FAKE), 1,
                                        kernel, ctypes.c_void_p(ws), nbytes, None)
    assert fwd(FAKE, 16) == q.QP_EINVAL and "workspace too small" in _err(q)
    assert fwd(FAKE + 8, 1 << 20) == q.QP_EALIGN and "workspace" in _err(q)
    assert fwd(FAKE, 16, M=0) == q.QP_ESHAPE


def test_binding_fails_loudly_without_the_library():
    """No fallback: with libqlinear.so absent, importing the binding raises
    (checked in a child process that hides the built file)."""
    import subprocess
    import sys
    code = ("import os\n"
            "real = os.path.exists\n"
            "os.path.exists = lambda p: False if str(p).endswith('libqlinear.so') else real(p)\n"
            "try:\n"
            "    import bit_weight_only_qlinear_amd.qlinear\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n"
            "    raise SystemExit(3)\n"
            "raise SystemExit(0)\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root,
                       timeout=120)
    assert r.returncode == 3, r.stdout + r.stderr
    assert "missing" in r.stdout
