"""Scalar-loop restatement of the oracle, for tiny shapes only.

Each group is handled by explicit Python loops over its elements with
np.float32 scalar arithmetic, so that the vectorized oracle's reshapes,
axes and broadcasts can be checked against a version with none of them.
Same steps and same sources as quantize.py / dequant.py / linear.py.
"""
import math

import numpy as np

from .formats import QFormat
from .numerics import to_meta, meta_to_f32

F32 = np.float32


def _rint(v):
    return float(np.rint(F32(v)))


def _clamp(v, lo, hi):
    return lo if v < lo else hi if v > hi else v


def _step_and_codes(vals, levels, code_max):
    m = F32(0)
    for v in vals:
        m = v if v > m else m
    step = np.float16(F32(m) / F32(levels))
    st = F32(step)
    codes = [0 if st == 0 else int(_clamp(_rint(F32(v) / st), 0, code_max))
             for v in vals]
    return step, codes


def quantize_scalar(W, f: QFormat):
    W = np.asarray(W, np.float32)
    N, K = W.shape
    gs = f.group_size
    ng = K // gs
    codes = np.zeros((N, K), np.int64)
    out = {}
    if f.fmt == "affine":
        sb = np.zeros((N, ng), np.uint16)
        bb = np.zeros((N, ng), np.uint16)
        for n in range(N):
            for g in range(ng):
                grp = [W[n, g * gs + i] for i in range(gs)]
                lo = F32(min(grp) + F32(0))
                hi = F32(max(grp) + F32(0))
                s32 = F32(F32(hi - lo) / F32(f.qmax))
                sb[n, g] = to_meta(np.array([s32]), f.meta)[0]
                bb[n, g] = to_meta(np.array([lo]), f.meta)[0]
                s = meta_to_f32(sb[n, g:g + 1], f.meta)[0]
                b = meta_to_f32(bb[n, g:g + 1], f.meta)[0]
                for i, w in enumerate(grp):
                    codes[n, g * gs + i] = 0 if s == 0 else int(
                        _clamp(_rint(F32(F32(w - b) / s)), 0, f.qmax))
        out = {"codes": codes.astype(np.uint8), "scales": sb, "biases": bb}
    elif f.fmt == "q4k":
        s_all = np.zeros((N, ng), np.float32)
        z_all = np.zeros((N, ng), np.float32)
        for n in range(N):
            for g in range(ng):
                grp = [W[n, g * 32 + i] for i in range(32)]
                lo = F32(min(min(grp), F32(0)) + F32(0))
                hi = F32(max(max(grp), F32(0)) + F32(0))
                s = F32(F32(hi - lo) / F32(15))
                z = F32(0) if s == 0 else F32(F32(F32(-lo) / s) + F32(0))
                s_all[n, g], z_all[n, g] = s, z
                for i, w in enumerate(grp):
                    codes[n, g * 32 + i] = 0 if s == 0 else int(
                        _clamp(_rint(F32(F32(w - lo) / s)), 0, 15))
        nsb = K // 256
        sc = np.zeros((N, ng), np.uint8)
        zc = np.zeros((N, ng), np.uint8)
        sstep = np.zeros((N, nsb), np.float16)
        zstep = np.zeros((N, nsb), np.float16)
        for n in range(N):
            for j in range(nsb):
                sl = slice(8 * j, 8 * j + 8)
                sstep[n, j], c = _step_and_codes(list(s_all[n, sl]), 255, 255)
                sc[n, sl] = c
                zstep[n, j], c = _step_and_codes(list(z_all[n, sl]), 255, 255)
                zc[n, sl] = c
        out = {"codes": codes.astype(np.uint8), "sc": sc, "zc": zc,
               "sstep": sstep, "zstep": zstep, "s": s_all, "z": z_all}
    elif f.fmt == "q6k":
        s_all = np.zeros((N, ng), np.float32)
        for n in range(N):
            for g in range(ng):
                grp = [W[n, g * 16 + i] for i in range(16)]
                amax = F32(0)
                for w in grp:
                    amax = max(amax, abs(w))
                s = F32(amax / F32(31))
                s_all[n, g] = s
                for i, w in enumerate(grp):
                    codes[n, g * 16 + i] = 0 if s == 0 else int(
                        _clamp(_rint(F32(w / s)), -32, 31))
        nsb = K // 256
        sc = np.zeros((N, ng), np.int8)
        step = np.zeros((N, nsb), np.float16)
        for n in range(N):
            for j in range(nsb):
                sl = slice(16 * j, 16 * j + 16)
                step[n, j], c = _step_and_codes(list(s_all[n, sl]), 127, 127)
                sc[n, sl] = c
        out = {"codes": codes.astype(np.int8), "sc": sc, "step": step,
               "s": s_all}
    else:
        sc = np.zeros((N, ng), np.float32)
        for n in range(N):
            for g in range(ng):
                grp = [W[n, g * gs + i] for i in range(gs)]
                amax = F32(0)
                for w in grp:
                    amax = max(amax, abs(w))
                s = F32(amax / F32(7))
                sc[n, g] = s
                for i, w in enumerate(grp):
                    codes[n, g * gs + i] = 0 if s == 0 else int(
                        _clamp(_rint(F32(w / s)), -7, 7))
        out = {"codes": codes.astype(np.int8), "scales": sc}
    return out


def dequant_scalar_f64(qz, f: QFormat):
    q = qz["codes"]
    N, K = q.shape
    w = np.zeros((N, K), np.float64)
    for n in range(N):
        for k in range(K):
            c = float(q[n, k])
            if f.fmt == "affine":
                g = k // f.group_size
                s = float(meta_to_f32(qz["scales"][n, g:g + 1], f.meta)[0])
                b = float(meta_to_f32(qz["biases"][n, g:g + 1], f.meta)[0])
                w[n, k] = c * s + b
            elif f.fmt == "q4k":
                g, j = k // 32, k // 256
                S = float(qz["sc"][n, g]) * float(qz["sstep"][n, j])
                Z = float(qz["zc"][n, g]) * float(qz["zstep"][n, j])
                w[n, k] = (c - Z) * S
            elif f.fmt == "q6k":
                g, j = k // 16, k // 256
                w[n, k] = c * (float(qz["sc"][n, g]) * float(qz["step"][n, j]))
            else:
                w[n, k] = c * float(qz["scales"][n, k // f.group_size])
    return w


def linear_scalar_f64(x64, qz, f: QFormat, bias64=None):
    w = dequant_scalar_f64(qz, f)
    M, K = x64.shape
    N = w.shape[0]
    y = np.zeros((M, N), np.float64)
    for m in range(M):
        for n in range(N):
            y[m, n] = math.fsum(float(x64[m, k]) * w[n, k] for k in range(K))
            if bias64 is not None:
                y[m, n] += float(bias64[n])
    return y
