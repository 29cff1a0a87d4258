"""Benchmark of the quantized linear layer on one MI355X.

Headline (the JSON line's `value`): decode-shaped qGEMV, int4 affine codes
with bf16 per-group scale/bias (group 64), M=1, K=4096, N=14336, x bf16 ->
y bf16.  One step is one decode pass over a stack of `--layers` layers of
that shape, each with its own weights (32 distinct weight sets, 1.06 GB, so
that no layer's weights are served from the 256 MB Infinity Cache); the pass
is captured once as a HIP graph and replayed.  The metric is effective HBM
GB/s: algorithmic bytes (packed codes + metadata + x + y, each once) per
second.

Also reported on the same line: the prefill qGEMM (M=2048, K=4096, N=14336,
int4 affine gs64) in TFLOP/s against the bf16/fp16 dense MFMA peak, the
other weight formats' qGEMV rates, the dominant kernel's roofline, and the
CPU oracle timed on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16/bf16 MFMA (256 CU x 2.4 GHz x 4096)
METRIC = ("qGEMV effective HBM GB/s (% of peak) at M=1; "
          "qGEMM TFLOP/s (% MFMA peak) at M=2048")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_layer_weights(q, desc, W_np, copies):
    """Quantize W on the GPU once, then make `copies` distinct copies."""
    import torch
    base = q.qpack_quantize(desc, torch.from_numpy(W_np).cuda())
    torch.cuda.synchronize()
    out = [base]
    for _ in range(copies - 1):
        out.append({k: (None if v is None else v.clone()) for k, v in base.items()})
    torch.cuda.synchronize()
    return out


def algorithmic_bytes(q, desc, M):
    s = q.qpack_sizes(desc)
    return sum(s.values()) + M * desc.K * 2 + M * desc.N * 2


def time_graph(fn_list, steps, warmup, warmup_s=0.0):
    """Capture fn_list (one call per layer) as one graph; replay it.
    Untimed warm-up: `warmup` replays, then more until `warmup_s` seconds
    have passed (the chip's clocks take ~0.1 s of sustained MFMA load to
    settle after an idle gap).  Returns (wall seconds for `steps` replays,
    event ms for the same)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fn_list:          # eager warm-up outside capture
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fn_list:
            f()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < warmup_s:
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1)


# Counter summary of the headline kernel: HBM bytes per launch from
# rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a plain copy's reading, and
# the hash of the kernel sources the counters were taken on.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_gemv_int4_affine_m1_k4096_n14336.md")
KERNEL_SOURCES = ("gemv.hip", "device_common.hpp")


def kernel_source_hash():
    """First 16 hex digits of the SHA-256 of the kernel sources with comments
    and whitespace removed: the counters stay valid across comment edits."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_weight_only_qlinear_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:") or line.startswith("kernel_source_sha256:"):
            k, v = line.split(":", 1)
            vals[k] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gemv_case(q, desc, W_np, M, x_bits, layers, steps, warmup):
    import numpy as np
    import torch
    xd = torch.from_numpy(np.ascontiguousarray(x_bits[:M]).view(np.int16)).view(torch.bfloat16).cuda()
    ws = make_layer_weights(q, desc, W_np, layers)
    ys = [torch.empty((M, desc.N), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    fns = [(lambda w=w, y=y: q.qlinear_forward(desc, xd, w, out=y)) for w, y in zip(ws, ys)]
    wall, ev_ms = time_graph(fns, steps, warmup)
    nb = algorithmic_bytes(q, desc, M)
    per_launch_s = ev_ms * 1e-3 / (steps * layers)
    res = dict(bytes_per_call=nb, wall_s=wall, event_ms=ev_ms,
               us_per_call=per_launch_s * 1e6,
               gbs=nb / per_launch_s / 1e9,
               gbs_wall=nb * steps * layers / wall / 1e9,
               tok_s_per_layer=M / per_launch_s)
    del ws, ys
    torch.cuda.empty_cache()
    return res


def copy_floor_case(nbytes, layers, steps, warmup):
    """Calibration, not the target: a plain device-to-device copy moving
    `nbytes` per launch (nbytes/2 read + nbytes/2 written), `layers`
    distinct buffer pairs captured in one graph and timed exactly like the
    qGEMV, so that it carries the same per-launch dispatch and ramp cost."""
    import torch
    n = nbytes // 2 // 4
    src = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(layers)]
    dst = [torch.empty_like(a) for a in src]
    fns = [(lambda a=a, b=b: b.copy_(a)) for a, b in zip(src, dst)]
    wall, ev_ms = time_graph(fns, steps, warmup)
    per_launch_s = ev_ms * 1e-3 / (steps * layers)
    del src, dst
    torch.cuda.empty_cache()
    return dict(us_per_call=per_launch_s * 1e6, gbs=2 * n * 4 / per_launch_s / 1e9)


def concat_case(q, K, Ns, x_bits, layers, steps, warmup):
    """Fused-N projections (e.g. q, k, v of one attention layer): the parts
    as separate forward calls against one forward over their qpack_concat_n
    stack, `layers` distinct weight sets each, M = 1."""
    import numpy as np
    import torch
    rng = np.random.default_rng(3)
    descs = [q.QDesc.affine(n, K, 4, 64, "bf16") for n in Ns]
    xd = torch.from_numpy(np.ascontiguousarray(x_bits[:1]).view(np.int16)).view(torch.bfloat16).cuda()
    parts, fused, ys, yf = [], [], [], []
    for _ in range(layers):
        bufs = [q.qpack_quantize(d, torch.from_numpy(rng.normal(0, 0.02, size=(d.N, K)).astype(np.float32)).cuda())
                for d in descs]
        dout, out = q.concat_n(descs, bufs)
        parts.append(bufs)
        fused.append(out)
        ys.append([torch.empty((1, d.N), dtype=torch.bfloat16, device="cuda") for d in descs])
        yf.append(torch.empty((1, dout.N), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    sep = [(lambda d=d, w=w, y=y: q.qlinear_forward(d, xd, w, out=y))
           for bl, yl in zip(parts, ys) for d, w, y in zip(descs, bl, yl)]
    one = [(lambda w=w, y=y: q.qlinear_forward(dout, xd, w, out=y)) for w, y in zip(fused, yf)]
    _, ms_sep = time_graph(sep, steps, warmup)
    _, ms_one = time_graph(one, steps, warmup)
    del parts, fused
    torch.cuda.empty_cache()
    return dict(us_separate=ms_sep * 1e3 / (steps * layers), us_fused=ms_one * 1e3 / (steps * layers))


def a8w4_case(q, desc, W_np, M, x_bits, layers, steps, warmup):
    """The a8w4 layer: per-token int8 quantization of x, then the int8 MFMA
    forward, per layer (both kernels timed)."""
    import numpy as np
    import torch
    xd = torch.from_numpy(np.ascontiguousarray(x_bits[:M]).view(np.int16)).view(torch.bfloat16).cuda()
    ws = make_layer_weights(q, desc, W_np, layers)
    ys = [torch.empty((M, desc.N), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    xq = torch.empty((M, desc.K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")

    def call(w, y):
        q._check(q.lib.qpack_quantize_activations(q._ptr(xd), q.DTYPE_IDS["bf16"], M, desc.K,
                                                  q._ptr(xq), q._ptr(xs), q._stream(xd.device)))
        q.qlinear_forward_a8w4(desc, xq, xs, w, y_dtype="bf16", out=y)

    fns = [(lambda w=w, y=y: call(w, y)) for w, y in zip(ws, ys)]
    wall, ev_ms = time_graph(fns, steps, warmup)
    s = q.qpack_sizes(desc)
    nb = s["qweight"] + s["scales"] + M * desc.K * 2 + M * desc.N * 2
    per = ev_ms * 1e-3 / (steps * layers)
    del ws, ys
    torch.cuda.empty_cache()
    return dict(bytes_per_call=nb, us_per_call=per * 1e6, gbs=nb / per / 1e9)


def gemm_case(q, desc, W_np, x_bits, steps, warmup, warmup_s=0.3):
    import numpy as np
    import torch
    M = x_bits.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    w = make_layer_weights(q, desc, W_np, 1)[0]
    y = torch.empty((M, desc.N), dtype=torch.bfloat16, device="cuda")
    fns = [lambda: q.qlinear_forward(desc, xd, w, out=y)]
    wall, ev_ms = time_graph(fns, steps, warmup, warmup_s)
    per = ev_ms * 1e-3 / steps
    flops = 2.0 * M * desc.N * desc.K
    tf = flops / per / 1e12
    # the C call with no workspace argument (qlinear_forward), eager: it
    # takes its workspace from the library's pool (not under capture)
    import ctypes
    d, ws = desc.c(), q._wstruct(w)
    yd = q.DTYPE_IDS["bf16"]

    def plain():
        st = q.lib.qlinear_forward(ctypes.byref(d), q._ptr(xd), yd, M, ctypes.byref(ws), None,
                                   q._ptr(y), yd, q._stream(xd.device))
        assert st == q.QP_OK, q.lib.qpack_last_error()
    for _ in range(20):
        plain()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        plain()
    ev1.record()
    torch.cuda.synchronize()
    plain_us = ev0.elapsed_time(ev1) * 1e3 / steps
    return dict(flops_per_call=flops, us_per_call=per * 1e6, tflops=tf,
                frac=tf / MFMA_F16_PEAK_TFLOPS, tok_s_per_layer=M / per, plain_c_us=plain_us)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:
        return 1


def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def cpu_stages(rows=2048):
    """The oracle's stages timed separately for every workload: quantize,
    pack into the device buffers, fp64 dequantize and the fp64 matmul, on
    the first `rows` weight rows of each layer (seed 0), scaled to the whole
    layer; plus one whole-layer decode forward (dequantize + matvec) of the
    int4 affine decode layer on a single core."""
    import numpy as np
    import oracle
    from oracle import QFormat
    from oracle.packing import to_buffers
    from bit_weight_only_qlinear_amd import synth
    cases = [("tiny_w4a16", "int4 affine gs64 fp16 meta", QFormat.affine(4, 64, "f16"), "f16"),
             ("decode_affine", "int4 affine gs64", QFormat.affine(4, 64, "bf16"), "bf16"),
             ("decode_affine", "int2 affine gs64", QFormat.affine(2, 64, "bf16"), "bf16"),
             ("decode_affine", "int8 affine gs64", QFormat.affine(8, 64, "bf16"), "bf16"),
             ("decode_q4k", "Q4_K-style", QFormat.q4k(), "bf16"),
             ("decode_8k", "Q6_K-style", QFormat.q6k(), "bf16"),
             ("decode_8k", "sym int4 per-channel", QFormat.sym4(8192), "bf16"),
             ("prefill_affine", "int4 affine gs64", QFormat.affine(4, 64, "bf16"), "bf16")]
    out = []
    wl_cache = {}
    for name, label, f, xdt in cases:
        if name not in wl_cache:
            wl_cache.clear()
            wl_cache[name] = synth.make(name, seed=0, M=8 if name == "decode_8k" else None)
        wl = wl_cache[name]
        N, K = wl.W.shape
        r = min(rows, N)
        Ws = wl.W[:r]
        x64 = oracle.decode_activations(wl.x_bits, xdt)
        qz, tq = _timed(lambda: oracle.quantize(Ws, f))
        _, tp = _timed(lambda: to_buffers(qz, f))
        w64, td = _timed(lambda: oracle.dequant_f64(qz, f))
        _, tm = _timed(lambda: np.matmul(x64, w64.T))
        sc = N / r
        out.append({"workload": f"{name}: {label}, M={x64.shape[0]} K={K} N={N}",
                    "sample_rows": r,
                    "quantize_s": round(tq * sc, 4), "pack_s": round(tp * sc, 4),
                    "dequant_s": round(td * sc, 4), "matmul_s": round(tm * sc, 5)})
        log("cpu", out[-1])
    wl_cache.clear()
    # whole decode layer, int4 affine, one core
    wl = synth.make("decode_affine", seed=0)
    f = QFormat.affine(4, 64, "bf16")
    qz = oracle.quantize(wl.W, f)
    x64 = oracle.decode_activations(wl.x_bits, "bf16")
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            _, t1 = _timed(lambda: oracle.linear_f64(x64, qz, f))
        single = {"workload": "decode_affine: int4 affine gs64, M=1 K=4096 N=14336, whole "
                              "layer (fp64 dequantize + matvec)", "cores": 1,
                  "forward_s": round(t1, 4)}
    except ImportError:
        single = None
    return out, single


def cpu_baseline(budget_s=12.0):
    """The oracle (NumPy, fp64 dequant + matvec) on the headline workload:
    whole-layer forwards of K=4096, N=14336 int4 affine, repeated until the
    time budget is spent (at least one); then the per-stage times of every
    workload."""
    import oracle
    from oracle import QFormat
    from bit_weight_only_qlinear_amd import synth
    wl = synth.make("decode_affine", seed=0)
    f = QFormat.affine(4, 64, "bf16")
    qz = oracle.quantize(wl.W, f)
    x64 = oracle.decode_activations(wl.x_bits, "bf16")
    N, K = wl.W.shape
    nbytes = N * K // 2 + 2 * N * (K // 64) * 2 + K * 2 + N * 2
    threads = _blas_threads()
    calls = 0
    t0 = time.perf_counter()
    while True:
        oracle.linear_f64(x64, qz, f)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    del wl, qz
    stages, single = cpu_stages()
    return {"value": round(nbytes * calls / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "host_cpu_count": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{calls} whole-layer forwards (fp64 dequantize + matvec) of "
                      f"M=1, K=4096, N=14336 int4 affine gs64 in {el:.1f} s; "
                      f"elementwise NumPy on 1 thread, BLAS on {threads}",
            "stages": stages,
            "stages_note": "per workload: the oracle's quantize, pack, fp64 dequantize and "
                           "fp64 matmul timed once on the first 2048 weight rows (seed 0) "
                           "and scaled to the whole layer",
            "single_core": single}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--quick", action="store_true", help="headline case only")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--qgemm-only", action="store_true",
                    help="only the prefill qGEMM case (for profiling); prints its own line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(its layers would shard along N, one slice of rows per GPU). "
              "Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from bit_weight_only_qlinear_amd import qlinear as q
    from bit_weight_only_qlinear_amd import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written")
        del a, b

    if args.qgemm_only:
        w5 = synth.make("prefill_affine", seed=0)
        r = gemm_case(q, q.QDesc.affine(14336, 4096, 4, 64, "bf16"), w5.W, w5.x_bits,
                      max(10, args.steps // 10), max(3, args.warmup // 4))
        print(json.dumps({"qgemm_only": True, "us_per_call": round(r["us_per_call"], 2),
                          "tflops": round(r["tflops"], 2), "frac": round(r["frac"], 4)}),
              flush=True)
        return

    # ---- headline: decode qGEMV int4 affine
    log("generating decode_affine weights")
    wl = synth.make("decode_affine", seed=0)
    N, K = wl.W.shape
    d4 = q.QDesc.affine(N, K, 4, 64, "bf16")
    head = gemv_case(q, d4, wl.W, 1, wl.x_bits, args.layers, args.steps, args.warmup)
    log("headline", head)

    extras = []
    qgemm = None
    floor = copy_floor_case(head["bytes_per_call"], args.layers, max(20, args.steps // 4),
                            args.warmup)
    calibration = dict(workload="plain device copy moving the headline's bytes per launch "
                                "(half read, half written), 32 distinct buffer pairs in one "
                                "graph, timed like the qGEMV (torch copy_)",
                       us_per_call=round(floor["us_per_call"], 3),
                       gbs=round(floor["gbs"], 1), frac=round(floor["gbs"] / HBM_PEAK_GBS, 4))
    log("calibration", calibration)
    if not args.quick:
        for bits in (2, 8):
            d = q.QDesc.affine(N, K, bits, 64, "bf16")
            r = gemv_case(q, d, wl.W, 1, wl.x_bits, args.layers, max(20, args.steps // 4),
                          args.warmup)
            extras.append(dict(workload=f"decode qGEMV int{bits} affine gs64 M=1 K=4096 N=14336",
                               gbs=round(r["gbs"], 1), frac=round(r["gbs"] / HBM_PEAK_GBS, 4),
                               us_per_call=round(r["us_per_call"], 3)))
            log(extras[-1])
        del wl
        log("generating decode_q4k weights")
        w3 = synth.make("decode_q4k", seed=0)
        d = q.QDesc.q4k(25600, 5120)
        r = gemv_case(q, d, w3.W, 1, w3.x_bits, 14, max(20, args.steps // 4), args.warmup)
        extras.append(dict(workload="decode qGEMV Q4_K-style M=1 K=5120 N=25600",
                           gbs=round(r["gbs"], 1), frac=round(r["gbs"] / HBM_PEAK_GBS, 4),
                           us_per_call=round(r["us_per_call"], 3)))
        log(extras[-1])
        del w3
        log("generating decode_8k weights")
        w4 = synth.make("decode_8k", seed=0, M=8)
        for dname, d, layers in (("Q6_K-style int6", q.QDesc.q6k(8192, 8192), 19),
                                 ("sym int4 per-channel", q.QDesc.sym4(8192, 8192), 31)):
            for M in (1, 4, 8):
                r = gemv_case(q, d, w4.W, M, w4.x_bits, layers, max(20, args.steps // 4),
                              args.warmup)
                extras.append(dict(workload=f"decode qGEMV {dname} M={M} K=8192 N=8192",
                                   gbs=round(r["gbs"], 1),
                                   frac=round(r["gbs"] / HBM_PEAK_GBS, 4),
                                   us_per_call=round(r["us_per_call"], 3)))
                log(extras[-1])
        w4s = synth.make("decode_8k", seed=0, M=16)
        for M in (1, 4, 8, 16):
            r = a8w4_case(q, q.QDesc.sym4(8192, 8192), w4s.W, M, w4s.x_bits, 31,
                          max(20, args.steps // 4), args.warmup)
            extras.append(dict(workload=f"decode a8w4 (int8 per-token activations x sym int4 "
                                        f"per-channel) M={M} K=8192 N=8192, quantize + forward",
                               gbs=round(r["gbs"], 1), frac=round(r["gbs"] / HBM_PEAK_GBS, 4),
                               us_per_call=round(r["us_per_call"], 3)))
            log(extras[-1])
        del w4, w4s
        xq = synth.make("decode_affine", seed=1, N=8).x_bits   # x ~ N(0, 1) bf16, K = 4096
        r = concat_case(q, 4096, (4096, 1024, 1024), xq, 32, max(20, args.steps // 4),
                        args.warmup)
        extras.append(dict(workload="fused-N projections (q 4096 + k 1024 + v 1024 rows, "
                                    "K=4096, int4 affine gs64, M=1): three forward calls vs one "
                                    "over their qpack_concat_n stack",
                           us_separate=round(r["us_separate"], 3),
                           us_fused=round(r["us_fused"], 3)))
        log(extras[-1])
        log("generating prefill_affine weights")
        w5 = synth.make("prefill_affine", seed=0)
        r = gemm_case(q, q.QDesc.affine(14336, 4096, 4, 64, "bf16"), w5.W, w5.x_bits,
                      max(10, args.steps // 10), max(3, args.warmup // 4))
        qgemm = dict(workload="prefill qGEMM int4 affine gs64 M=2048 K=4096 N=14336, "
                              "fp16 MFMA, fp32 accumulate, bf16 out; one-pass activation "
                              "staging (row exponent + fp16 fragments) and the 224-row-tile "
                              "kernel, both timed",
                     value=round(r["tflops"], 2), unit="TFLOP/s",
                     peak=MFMA_F16_PEAK_TFLOPS, frac=round(r["frac"], 4),
                     us_per_call=round(r["us_per_call"], 2),
                     tok_s_per_layer=round(r["tok_s_per_layer"], 1),
                     warmup="untimed graph replays for >= 0.3 s (clocks settle under MFMA load)",
                     plain_c_call_us=round(r["plain_c_us"], 2),
                     plain_c_call="qlinear_forward (the C call without a workspace argument: "
                                  "workspace from the library's pool), eager launches")
        log("qgemm", qgemm)
        del w5

    cpu = None if args.no_cpu else cpu_baseline()

    per_step_s = head["wall_s"] / args.steps
    value = head["bytes_per_call"] * args.layers * args.steps / head["wall_s"] / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded W ~ N(0,0.02) with 4 outlier columns x20, x ~ N(0,1))",
        "config": {
            "workload": "decode qGEMV int4 affine gs64 (bf16 scale/bias), M=1, K=4096, "
                        "N=14336, x bf16, y bf16",
            "layers_per_step": args.layers,
            "bytes_per_call": head["bytes_per_call"],
            "us_per_call": round(head["us_per_call"], 3),
            "tok_s_per_layer": round(head["tok_s_per_layer"], 1),
            "graph": "one HIP graph per step",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_gemv (int4 affine, one activation row)",
            "achieved": round(head["gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["gbs"] / HBM_PEAK_GBS, 4),
            "us_per_launch": round(head["us_per_call"], 3),
            "algorithmic_bytes": head["bytes_per_call"],
            "traffic": measured_traffic(),
            "calibration": calibration,
        },
        "cpu_baseline": cpu,
        "qgemm": qgemm,
        "also": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
