"""Thin ctypes binding of libqlinear (include/qlinear.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
The library must be built (``python -m bit_weight_only_qlinear_amd.build``
or ``__graft_entry__.build()``); importing this module without it raises.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlinear.so")

QP_OK, QP_EINVAL, QP_ESHAPE, QP_EUNSUPPORTED, QP_EALIGN, QP_EHIP = range(6)
QP_FMT_AFFINE, QP_FMT_Q4K, QP_FMT_Q6K, QP_FMT_SYM4 = range(4)
QP_F16, QP_BF16, QP_F32 = range(3)
QP_KERNEL_AUTO, QP_KERNEL_GEMV, QP_KERNEL_GEMM, QP_KERNEL_GEMV_MFMA = range(4)

FMT_IDS = {"affine": QP_FMT_AFFINE, "q4k": QP_FMT_Q4K, "q6k": QP_FMT_Q6K,
           "sym4": QP_FMT_SYM4}
DTYPE_IDS = {"f16": QP_F16, "bf16": QP_BF16, "f32": QP_F32}
BUFFERS = ("qweight", "qweight_hi", "scales", "zeros", "steps")


class QLinearError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"qlinear status {status}: {message}")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("super_block", ctypes.c_int32),
                ("meta_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _Weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in BUFFERS]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m bit_weight_only_qlinear_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    D, W = ctypes.POINTER(_Desc), ctypes.POINTER(_Weights)
    sig = {
        "qpack_abi_version": (I32, []),
        "qpack_last_error": (ctypes.c_char_p, []),
        "qpack_sizes": (I32, [D, ctypes.POINTER(ctypes.c_size_t)]),
        "qpack_quantize": (I32, [D, P, W, P]),
        "qpack_quantize_hqq": (I32, [D, P, W, I32, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_float, P]),
        "qpack_unpack_codes": (I32, [D, W, P, P]),
        "qpack_pack_codes": (I32, [D, P, W, P]),
        "qpack_dequantize": (I32, [D, W, P, I32, P]),
        "qlinear_forward": (I32, [D, P, I32, I64, W, P, P, I32, P]),
        "qlinear_forward_kernel": (I32, [D, P, I32, I64, W, P, P, I32, I32, P]),
        "qlinear_workspace_bytes": (I32, [D, I32, I64, I32, ctypes.POINTER(ctypes.c_size_t)]),
        "qlinear_forward_ws": (I32, [D, P, I32, I64, W, P, P, I32, I32, P, ctypes.c_size_t, P]),
        "qlinear_forward_static": (I32, [D, P, I32, I64, W, P, P, I32, I32, P]),
        "qpack_encode_nested": (I32, [D, P, P, W, P, P]),
        "qpack_concat_n": (I32, [D, I32, D, W, W, P]),
        "qpack_quantize_activations": (I32, [P, I32, I64, I64, P, P, P]),
        "qlinear_forward_a8w4": (I32, [D, P, P, I64, W, P, P, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = ("qpack_abi_version", "qpack_last_error", "qpack_sizes", "qpack_quantize",
            "qpack_quantize_hqq",
            "qpack_unpack_codes", "qpack_pack_codes", "qpack_dequantize",
            "qlinear_forward", "qlinear_forward_kernel", "qlinear_workspace_bytes",
            "qlinear_forward_ws", "qlinear_forward_static", "qpack_encode_nested",
            "qpack_concat_n",
            "qpack_quantize_activations",
            "qlinear_forward_a8w4")


@dataclass(frozen=True)
class QDesc:
    """Python form of qp_desc."""
    fmt: str
    bits: int
    group_size: int
    N: int
    K: int
    meta: str = "bf16"          # affine metadata dtype
    super_block: int = 0

    @staticmethod
    def affine(N, K, bits=4, group_size=64, meta="bf16"):
        return QDesc("affine", bits, group_size, N, K, meta, 0)

    @staticmethod
    def q4k(N, K):
        return QDesc("q4k", 4, 32, N, K, "f16", 256)

    @staticmethod
    def q6k(N, K):
        return QDesc("q6k", 6, 16, N, K, "f16", 256)

    @staticmethod
    def sym4(N, K, group_size=None):
        return QDesc("sym4", 4, K if group_size is None else group_size, N, K, "f32", 0)

    def c(self):
        return _Desc(FMT_IDS[self.fmt], self.bits, self.group_size, self.super_block,
                     DTYPE_IDS[self.meta], 0, self.N, self.K)


def _check(status):
    if status != QP_OK:
        raise QLinearError(status, lib.qpack_last_error().decode())


def _stream(device=None):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def qpack_sizes(desc: QDesc):
    out = (ctypes.c_size_t * 5)()
    d = desc.c()
    _check(lib.qpack_sizes(ctypes.byref(d), out))
    return dict(zip(BUFFERS, [int(v) for v in out]))


def _buf_dtypes(desc):
    import torch
    meta = {"f16": torch.float16, "bf16": torch.bfloat16}.get(desc.meta, torch.float16)
    if desc.fmt == "affine":
        return dict(qweight=torch.int32, scales=meta, zeros=meta)
    if desc.fmt == "q4k":
        return dict(qweight=torch.int32, scales=torch.uint8, zeros=torch.uint8,
                    steps=torch.int32)
    if desc.fmt == "q6k":
        return dict(qweight=torch.int32, qweight_hi=torch.int32, scales=torch.int8,
                    steps=torch.float16)
    return dict(qweight=torch.int32, scales=torch.float32)


def alloc_weights(desc: QDesc, device="cuda"):
    """Empty device buffers of the sizes qpack_sizes gives (torch memory)."""
    import torch
    sizes = qpack_sizes(desc)
    dts = _buf_dtypes(desc)
    out = {}
    for name in BUFFERS:
        if sizes[name]:
            dt = dts[name]
            itemsize = torch.empty(0, dtype=dt).element_size()
            # allocated to the next multiple of 16 bytes (the library reads
            # its buffers in 16-byte units); the view has the exact size
            padded = (sizes[name] + 15) // 16 * 16
            out[name] = torch.empty(padded // itemsize, dtype=dt,
                                    device=device)[: sizes[name] // itemsize]
        else:
            out[name] = None
    return out


def _wstruct(w):
    return _Weights(*[None if w.get(n) is None else w[n].data_ptr() for n in BUFFERS])


def qpack_quantize(desc: QDesc, W, out=None):
    """W: device fp32 [N, K] -> dict of packed buffers (torch tensors)."""
    if out is None:
        out = alloc_weights(desc, W.device)
    d, ws = desc.c(), _wstruct(out)
    _check(lib.qpack_quantize(ctypes.byref(d), _ptr(W), ctypes.byref(ws), _stream(W.device)))
    return out


def qpack_quantize_hqq(desc: QDesc, W, out=None, iters=20, lp_norm=0.7, beta=10.0,
                       kappa=1.01):
    """AFFINE only: W device fp32 [N, K] -> packed buffers, with the HQQ zero
    point per group (see qpack_quantize_hqq in include/qlinear.h)."""
    if out is None:
        out = alloc_weights(desc, W.device)
    d, ws = desc.c(), _wstruct(out)
    _check(lib.qpack_quantize_hqq(ctypes.byref(d), _ptr(W), ctypes.byref(ws), int(iters),
                                  float(lp_norm), float(beta), float(kappa),
                                  _stream(W.device)))
    return out


def qpack_unpack_codes(desc: QDesc, w, codes=None):
    import torch
    if codes is None:
        dt = torch.int8 if desc.fmt in ("q6k", "sym4") else torch.uint8
        codes = torch.empty((desc.N, desc.K), dtype=dt, device=w["qweight"].device)
    d, ws = desc.c(), _wstruct(w)
    _check(lib.qpack_unpack_codes(ctypes.byref(d), ctypes.byref(ws), _ptr(codes),
                                  _stream(codes.device)))
    return codes


def qpack_pack_codes(desc: QDesc, codes, out=None):
    if out is None:
        out = alloc_weights(desc, codes.device)
    d, ws = desc.c(), _wstruct(out)
    _check(lib.qpack_pack_codes(ctypes.byref(d), _ptr(codes), ctypes.byref(ws),
                                _stream(codes.device)))
    return out


def qpack_dequantize(desc: QDesc, w, out_dtype="f32", out=None):
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_dtype]
    if out is None:
        out = torch.empty((desc.N, desc.K), dtype=tdt, device=w["qweight"].device)
    d, ws = desc.c(), _wstruct(w)
    _check(lib.qpack_dequantize(ctypes.byref(d), ctypes.byref(ws), _ptr(out),
                                DTYPE_IDS[out_dtype], _stream(out.device)))
    return out


def _xdtype(t):
    import torch
    if t.dtype == torch.float16:
        return "f16"
    if t.dtype == torch.bfloat16:
        return "bf16"
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def workspace_bytes(desc: QDesc, M: int, x_dtype: str = "bf16",
                    kernel: int = QP_KERNEL_AUTO) -> int:
    """Device workspace bytes qlinear_forward can use (qlinear_workspace_bytes)."""
    d, n = desc.c(), ctypes.c_size_t(0)
    _check(lib.qlinear_workspace_bytes(ctypes.byref(d), DTYPE_IDS[x_dtype], M, kernel,
                                       ctypes.byref(n)))
    return n.value


def qlinear_forward(desc: QDesc, x, w, bias=None, y_dtype: Optional[str] = None,
                    kernel: int = QP_KERNEL_AUTO, out=None, workspace="auto"):
    """y [M, N] = x [M, K] W^T (+ bias).  x: fp16/bf16 device tensor.

    workspace: "auto" allocates what the call can use from torch's caching
    allocator on the current stream; None runs without one; or a device
    tensor (its bytes are the workspace)."""
    import torch
    xd = _xdtype(x)
    yd = y_dtype or xd
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[yd]
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, desc.N), dtype=tdt, device=x.device)
    buf, nbytes = None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a tensor, got {workspace!r}")
        nbytes = workspace_bytes(desc, M, xd, kernel)
        if nbytes:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    elif workspace is not None:
        buf, nbytes = workspace, workspace.numel() * workspace.element_size()
    d, ws = desc.c(), _wstruct(w)
    _check(lib.qlinear_forward_ws(ctypes.byref(d), _ptr(x), DTYPE_IDS[xd], M,
                                  ctypes.byref(ws), _ptr(bias), _ptr(out), DTYPE_IDS[yd],
                                  kernel, _ptr(buf), nbytes, _stream(x.device)))
    return out


def qlinear_forward_static(desc: QDesc, x, w, out, bias=None, kernel: int = QP_KERNEL_AUTO):
    """qlinear_forward_static: the forward into the caller's `out` (its dtype
    is the output dtype) with the library's static scratch in place of a
    workspace; the C call allocates nothing."""
    import torch
    yd = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[out.dtype]
    d, ws = desc.c(), _wstruct(w)
    _check(lib.qlinear_forward_static(ctypes.byref(d), _ptr(x), DTYPE_IDS[_xdtype(x)], x.shape[0],
                                      ctypes.byref(ws), _ptr(bias), _ptr(out), DTYPE_IDS[yd],
                                      kernel, _stream(x.device)))
    return out


def concat_n(descs, weights):
    """Stack layers of one format and K along N (qpack_concat_n): returns
    (QDesc of the stacked layer, its buffers)."""
    import dataclasses
    d0 = descs[0]
    dout = dataclasses.replace(d0, N=sum(d.N for d in descs))
    out = alloc_weights(dout, device=weights[0]["qweight"].device)
    n = len(descs)
    dins = (_Desc * n)(*[d.c() for d in descs])
    wins = (_Weights * n)(*[_wstruct(w) for w in weights])
    _check(lib.qpack_concat_n(ctypes.byref(dout.c()), n, dins, wins, ctypes.byref(_wstruct(out)),
                              _stream(weights[0]["qweight"].device)))
    return dout, out


def convert_to_nested(desc: QDesc, codes, s, z=None):
    """Plain int4 (codes uint8 [N, K], s, z fp32 [N, K/32]) or int6 (codes
    int8 [N, K], s fp32 [N, K/16]) -> nested Q4K / Q6K buffers with the codes
    unchanged (qpack_pack_codes + qpack_encode_nested).  Returns (buffers,
    bad) with bad a device int32 that is 1 if any input was invalid."""
    import torch
    w = alloc_weights(desc, device=codes.device)
    _check(lib.qpack_pack_codes(ctypes.byref(desc.c()), _ptr(codes), ctypes.byref(_wstruct(w)),
                                _stream(codes.device)))
    bad = torch.zeros(4, dtype=torch.int32, device=codes.device)
    _check(lib.qpack_encode_nested(ctypes.byref(desc.c()), _ptr(s), _ptr(z),
                                   ctypes.byref(_wstruct(w)), _ptr(bad), _stream(codes.device)))
    return w, bad


def quantize_activations(x):
    """Per-token symmetric int8 activations (qpack_quantize_activations):
    x fp16/bf16 [M, K] -> (xq int8 [M, K], xs fp32 [M])."""
    import torch
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib.qpack_quantize_activations(_ptr(x), DTYPE_IDS[_xdtype(x)], M, K, _ptr(xq),
                                          _ptr(xs), _stream(x.device)))
    return xq, xs


def qlinear_forward_a8w4(desc: QDesc, xq, xs, w, bias=None, y_dtype: str = "bf16", out=None):
    """y [M, N] = xs[m] * s_n * sum_k xq[m, k] q[n, k] (+ bias fp32 [N]) for
    SYM4 weights with one scale per output channel."""
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[y_dtype]
    M = xq.shape[0]
    if out is None:
        out = torch.empty((M, desc.N), dtype=tdt, device=xq.device)
    d, ws = desc.c(), _wstruct(w)
    _check(lib.qlinear_forward_a8w4(ctypes.byref(d), _ptr(xq), _ptr(xs), M, ctypes.byref(ws),
                                    _ptr(bias), _ptr(out), DTYPE_IDS[y_dtype],
                                    _stream(xq.device)))
    return out
