"""Pins of the CPU oracle against what the pages and mathematics fix.

Sources: HF Transformers "Metal" page (uint32-packed weights, per-group
scale/bias, bits 2/4/8, group 64); ExecuTorch PR #20571 "Nested Superscale
Quantization" ("Quant schema update": w = (q - zero)*scale, Q4_K-style int4
gs=32 / super-block 256 / 4.625 bpw, Q6_K-style int6 gs=16 / 6.5625 bpw;
"Analysis": codes identical to the source values; ablation table: per-256
steps beat per-row steps); ExecuTorch PR #16577 (int4 in int8, qmin=-7,
qmax=7).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import QFormat
from oracle.packing import (pack_bits, unpack_bits, pack_codes, unpack_codes,
                            q4k_step_words, to_buffers, from_buffers)
from oracle.quantize import _encode_per_super
from oracle.scalar import quantize_scalar, dequant_scalar_f64, linear_scalar_f64

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "closed_forms.json")))


def _fmt(case):
    if case["fmt"] == "affine":
        return QFormat.affine(case["bits"], case["gs"], case["meta"])
    if case["fmt"] == "q4k":
        return QFormat.q4k()
    if case["fmt"] == "q6k":
        return QFormat.q6k()
    return QFormat.sym4(case["gs"])


def _codes_rule(case):
    K = case["K"]
    k = np.arange(K)
    rule = case["codes_rule"]
    if rule == "code at k = k % 16":
        return (k % 16)[None, :]
    if rule == "code at k = 5":
        return np.full((1, K), 5)
    if rule == "code at k = 15":
        return np.full((1, K), 15)
    if rule == "code at k = (k % 63) - 31":
        return ((k % 63) - 31)[None, :]
    raise KeyError(rule)


def _as_fraction(v):
    return Fraction(float(v)) if isinstance(v, float) else Fraction(v)


# ---------------------------------------------------------------- P-closed
@pytest.mark.parametrize("case", GOLD["dequant"], ids=lambda c: c["name"][:40])
def test_dequant_closed_form(case):
    f = _fmt(case)
    if case["fmt"] == "affine":
        qz = {"codes": np.array(case["codes"], np.uint8),
              "scales": np.array(case["scales"], np.uint16),
              "biases": np.array(case["biases"], np.uint16)}
    elif case["fmt"] == "sym4":
        qz = {"codes": np.array(case["codes"], np.int8),
              "scales": np.array(case["scales"], np.float32)}
    elif case["fmt"] == "q4k":
        qz = {"codes": _codes_rule(case).astype(np.uint8),
              "sc": np.array(case["sc"], np.uint8),
              "zc": np.array(case["zc"], np.uint8),
              "sstep": np.array(case["sstep_bits"], np.uint16).view(np.float16),
              "zstep": np.array(case["zstep_bits"], np.uint16).view(np.float16)}
    else:
        qz = {"codes": _codes_rule(case).astype(np.int8),
              "sc": np.array(case["sc"], np.int8),
              "step": np.array(case["step_bits"], np.uint16).view(np.float16)}
    w = oracle.dequant_f64(qz, f)
    if "expected" in case:
        exp = [[Fraction(v) for v in row] for row in case["expected"]]
        got = [[Fraction(float(v)) for v in row] for row in w]
        assert got == exp
    else:
        for e in case["expected_at"]:
            assert Fraction(float(w[0, e["k"]])) == Fraction(e["value"]), e
    # the fp32 evaluation agrees with the exact value rounded once
    w32 = oracle.dequant_f32(qz, f)
    assert np.array_equal(w32, w.astype(np.float32))


@pytest.mark.parametrize("case", GOLD["pack"], ids=lambda c: c["name"][:30])
def test_pack_golden(case):
    if "bits" in case:
        fields = np.array([case["fields"]])
        words = pack_bits(fields, case["bits"])
        assert words.tolist() == [[int(case["word"], 16)]]
        assert unpack_bits(words, case["bits"], fields.shape[1]).tolist() == \
            fields.tolist()
    elif case["fmt"] == "sym4":
        planes = pack_codes(np.array([case["codes"]]), QFormat.sym4(8))
        assert planes["qweight"].tolist() == [[int(case["word"], 16)]]
    elif case["fmt"] == "q6k":
        planes = pack_codes(np.array([case["codes"]]), QFormat.q6k())
        assert planes["qweight"].tolist() == [[int(w, 16) for w in case["ql_words"]]]
        assert planes["qweight_hi"].tolist() == [[int(case["qh_word"], 16)]]
    else:
        s = np.array([case["sstep_bits"]], np.uint16).view(np.float16)
        z = np.array([case["zstep_bits"]], np.uint16).view(np.float16)
        assert q4k_step_words(s, z).tolist() == [int(case["word"], 16)]


def _golden_W(case):
    if "W" in case:
        return np.array(case["W"], np.float32)
    k = np.arange(case["K"])
    if case["fmt"] == "q4k":
        q = np.where((k // 16) % 2 == 0, k % 16, 15 - k % 16)
        return ((q - 8) / 16).astype(np.float32)[None, :], q
    q = np.where(k % 16 == 15, 31, (k % 16) * 4 - 31)
    return (q / 64).astype(np.float32)[None, :], q


@pytest.mark.parametrize("case", GOLD["quantize"], ids=lambda c: c["name"][:40])
def test_quantize_golden(case):
    f = _fmt(case)
    if case["fmt"] in ("affine", "sym4"):
        W = _golden_W(case)
        qz = oracle.quantize(W, f)
        assert qz["codes"].tolist() == case["codes"]
        if case["fmt"] == "affine":
            assert qz["scales"].tolist() == case["scales"]
            assert qz["biases"].tolist() == case["biases"]
        else:
            assert qz["scales"].tolist() == case["scales"]
        return
    W, q = _golden_W(case)
    qz = oracle.quantize(W, f)
    assert qz["codes"][0].astype(int).tolist() == q.tolist()
    assert np.all(qz["sc"] == case["sc_all"])
    assert all(Fraction(float(v)) == Fraction(case["s_all"]) for v in qz["s"][0])
    if "z_all" in case:
        assert all(Fraction(float(v)) == Fraction(case["z_all"]) for v in qz["z"][0])
    w = oracle.dequant_f64(qz, f)[0]
    if case["fmt"] == "q4k":
        assert np.all(qz["zc"] == case["zc_all"])
        assert qz["sstep"].view(np.uint16).tolist() == [[case["sstep_bits"]]]
        assert qz["zstep"].view(np.uint16).tolist() == [[case["zstep_bits"]]]
        for k in range(256):
            exp = (Fraction(int(q[k])) - Fraction(255 * 257, 8192)) * Fraction(255 * 257, 1 << 20)
            assert Fraction(float(w[k])) == exp
    else:
        assert qz["step"].view(np.uint16).tolist() == [[case["step_bits"]]]
        for k in range(256):
            assert Fraction(float(w[k])) == int(q[k]) * Fraction(127 * 129, 1 << 20)


def _q4k_qz(case):
    return {"codes": _codes_rule(case).astype(np.uint8),
            "sc": np.array(case["sc"], np.uint8),
            "zc": np.array(case["zc"], np.uint8),
            "sstep": np.array(case["sstep_bits"], np.uint16).view(np.float16),
            "zstep": np.array(case["zstep_bits"], np.uint16).view(np.float16)}


@pytest.mark.parametrize("case", GOLD["dequant_f32_order"], ids=lambda c: c["name"][:30])
def test_dequant_f32_operation_order(case):
    """The fp32 dequantization evaluates (q - zero) * scale in the page's
    order, one IEEE fp32 operation each: where q - zero is inexact this can
    differ by one unit in the last place from the exact value rounded once
    (hand-worked case)."""
    f = QFormat.q4k()
    qz = _q4k_qz(case)
    k = case["k"]
    w = oracle.dequant_f64(qz, f)
    assert Fraction(float(w[0, k])) == Fraction(case["exact"])
    w32 = oracle.dequant_f32(qz, f)
    assert Fraction(float(w32[0, k])) == Fraction(case["f32_in_order"])
    # the two readings really differ here
    assert Fraction(float(np.float32(w[0, k]))) == Fraction(case["f32_rounded_once"])
    assert case["f32_in_order"] != case["f32_rounded_once"]
    # dequant_out('f32') is that same fp32 evaluation
    assert np.array_equal(oracle.dequant_out(qz, f, "f32"), w32)


# ------------------------------------------------------------ bf16 rounding
@pytest.mark.parametrize("case", GOLD["bf16_rne"], ids=lambda c: c["f32"])
def test_bf16_rne_golden(case):
    x = np.array([int(case["f32"], 16)], np.uint32).view(np.float32)
    assert oracle.f32_to_bf16_bits(x).tolist() == [int(case["bf16"], 16)]
    # widening back is exact
    b = np.array([int(case["bf16"], 16)], np.uint16)
    assert oracle.bf16_bits_to_f32(b).view(np.uint32).tolist() == [int(case["bf16"], 16) << 16]


def test_bf16_rne_matches_torch():
    """Against an independent implementation: torch's CPU fp32 -> bfloat16
    conversion (round to nearest, ties to even) on 10^6 random finite bit
    patterns plus every upper half combined with the lower halves around a
    tie (0x7FFF, 0x8000, 0x8001) and 0."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    adv = (hi[:, None] | np.array([0x0000, 0x7FFF, 0x8000, 0x8001], np.uint32)[None, :]).ravel()
    u = np.concatenate([u, adv])
    u = u[(u & 0x7F800000) != 0x7F800000]          # finite inputs only
    x = u.view(np.float32)
    got = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------- SNR
@pytest.mark.parametrize("case", GOLD["snr_db"], ids=lambda c: c["name"][:20])
def test_snr_db_golden(case):
    ref = np.array(case["ref"])
    approx = np.array(case["approx"])
    assert oracle.snr_db(ref, approx) == pytest.approx(case["db"], abs=1e-12)
    # scale invariant, and symmetric in the sign of the error
    assert oracle.snr_db(4 * ref, 4 * approx) == pytest.approx(case["db"], abs=1e-12)
    assert oracle.snr_db(ref, 2 * ref - approx) == pytest.approx(case["db"], abs=1e-12)


# ------------------------------------------------------------- P-roundtrip
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_pack_roundtrip_exhaustive(bits):
    per = 32 // bits
    # every code value at every slot of a word
    vals = np.arange(1 << bits)
    rows = [np.roll(np.resize(vals, per * ((1 << bits) // per + 1)), r)
            for r in range(per)]
    u = np.array([r[:per * 4] for r in rows])
    assert unpack_bits(pack_bits(u, bits), bits, u.shape[1]).tolist() == u.tolist()
    # and words -> fields -> words for random words
    w = np.random.default_rng(1).integers(0, 2**32, size=(3, 5), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(pack_bits(unpack_bits(w, bits, 5 * per), bits), w)


@pytest.mark.parametrize("f", [QFormat.sym4(32), QFormat.q6k(), QFormat.q4k(),
                               QFormat.affine(2), QFormat.affine(8)],
                         ids=lambda f: f"{f.fmt}{f.bits}")
def test_pack_codes_roundtrip_all_values(f):
    K = 512
    rng = np.random.default_rng(3)
    vals = np.arange(f.qmin, f.qmax + 1)
    c = np.stack([np.roll(np.resize(vals, K), s) for s in range(5)])
    rng.shuffle(c, axis=1)
    got = unpack_codes(pack_codes(c, f), f, K)
    assert got.astype(int).tolist() == c.tolist()


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        pack_codes(np.full((1, 8), 8), QFormat.sym4(8))
    with pytest.raises(ValueError):
        pack_codes(np.full((1, 256), -33), QFormat.q6k())


# ----------------------------------------------------------------- P-range
ALL_FORMATS = [QFormat.affine(4, 64, "f16"), QFormat.affine(4), QFormat.affine(2),
               QFormat.affine(8), QFormat.affine(4, 32), QFormat.affine(2, 128),
               QFormat.q4k(), QFormat.q6k(), QFormat.sym4(512), QFormat.sym4(64)]
FID = lambda f: f"{f.fmt}-b{f.bits}-g{f.group_size}-{f.meta}"


@pytest.mark.parametrize("f", ALL_FORMATS, ids=FID)
def test_code_ranges(f):
    rng = np.random.default_rng(5)
    W = rng.laplace(0, 0.015, size=(16, 512)).astype(np.float32)
    W[3] = np.abs(W[3])                  # all-positive row
    W[4] = -np.abs(W[4])                 # all-negative row
    W[5, :64] = 0.0                      # zero groups
    qz = oracle.quantize(W, f)
    c = qz["codes"].astype(int)
    assert c.min() >= f.qmin and c.max() <= f.qmax
    if f.fmt == "q6k":
        assert np.abs(c).max() <= 31     # symmetric in practice
        assert qz["sc"].min() >= 0 and qz["sc"].max() <= 127
    if f.fmt == "q4k":
        assert qz["z"].min() >= 0 and qz["z"].max() <= 15 * (1 + 2**-20)
        assert qz["sc"].dtype == np.uint8 and qz["zc"].dtype == np.uint8
    if f.fmt == "sym4":
        assert c.min() >= -7 and c.max() <= 7


def test_superscale_encoder_rejects_negative():
    with pytest.raises(ValueError):
        _encode_per_super(np.array([[0.5, -0.1, 0, 0, 0, 0, 0, 0]], np.float32),
                          8, 255, 255)


# ------------------------------------------------------------------- P-bpw
def test_bits_per_weight():
    N, K = 256, 4096
    assert oracle.bits_per_weight(QFormat.q4k(), N, K) == 4.625
    assert oracle.bits_per_weight(QFormat.q6k(), N, K) == 6.5625
    for b, exp in [(4, 4.5), (2, 2.5), (8, 8.5)]:
        assert oracle.bits_per_weight(QFormat.affine(b, 64), N, K) == exp
    # a per-256 fp16 zero step costs 16/256 = 0.0625 bpw (the "+0.06 bpw")
    assert oracle.bits_per_weight(QFormat.q4k(), N, K) - 4.5625 == 0.0625
    assert oracle.bits_per_weight(QFormat.sym4(K), N, K) == 4 + 32 / K


# --------------------------------------------------------------- P-lattice
def _lattice_affine(rng, f, N, K):
    gs, qmax = f.group_size, f.qmax
    ng = K // gs
    q = rng.integers(0, qmax + 1, size=(N, ng, gs))
    q[:, :, 0] = 0
    q[:, :, 1] = qmax
    e = rng.integers(6, 12, size=(N, ng, 1))
    c = rng.integers(1, 8, size=(N, ng, 1))              # scale = c*2^-e
    s = c * np.exp2(-e)
    b = rng.integers(-64, 64, size=(N, ng, 1)) * np.exp2(-8)
    W = (q * s + b).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), q * s + b)
    return W.reshape(N, K), q.reshape(N, K)


def _lattice_q4k(rng, N, K):
    ng, nsb = K // 32, K // 256
    q = rng.integers(0, 16, size=(N, ng, 32))
    q[:, :, 0] = 0
    q[:, :, 1] = 15
    sc = rng.integers(1, 256, size=(N, ng))
    d = rng.integers(0, 256, size=(N, ng))
    sc.reshape(N, nsb, 8)[:, :, 0] = 255
    d.reshape(N, nsb, 8)[:, :, 1] = 255
    s = sc * 2.0 ** -12
    z = d / 32.0
    W = (q - z[..., None]) * s[..., None]
    W32 = W.astype(np.float32)
    assert np.array_equal(W32.astype(np.float64), W)
    return W32.reshape(N, K), q.reshape(N, K)


def _lattice_q6k(rng, N, K):
    ng, nsb = K // 16, K // 256
    q = rng.integers(-31, 32, size=(N, ng, 16))
    q[:, :, 0] = rng.choice([-31, 31], size=(N, ng))
    sc = rng.integers(1, 128, size=(N, ng))
    sc.reshape(N, nsb, 16)[:, :, 0] = 127
    s = sc * 2.0 ** -12
    W = q * s[..., None]
    return W.astype(np.float32).reshape(N, K), q.reshape(N, K)


def _lattice_sym4(rng, N, K, gs):
    q = rng.integers(-7, 8, size=(N, K // gs, gs))
    q[:, :, 0] = 7
    s = np.exp2(-rng.integers(4, 10, size=(N, K // gs, 1)))
    return (q * s).astype(np.float32).reshape(N, K), q.reshape(N, K)


@pytest.mark.parametrize("f", ALL_FORMATS, ids=FID)
def test_lattice_lossless_and_linear_exact(f):
    """Weights built on the format's lattice (both extreme codes in every
    group, exactly representable metadata) quantize losslessly; the whole
    pipeline (quantize, pack, unpack, dequantize, linear) then reproduces a
    textbook matmul of x and the original W exactly."""
    rng = np.random.default_rng(11)
    N, K = 24, 512
    if f.fmt == "affine":
        W, q = _lattice_affine(rng, f, N, K)
    elif f.fmt == "q4k":
        W, q = _lattice_q4k(rng, N, K)
    elif f.fmt == "q6k":
        W, q = _lattice_q6k(rng, N, K)
    else:
        W, q = _lattice_sym4(rng, N, K, f.group_size)
    qz = oracle.quantize(W, f)
    assert np.array_equal(qz["codes"].astype(int), q)
    qz2 = from_buffers(to_buffers(qz, f), f, K)
    w = oracle.dequant_f64(qz2, f)
    assert np.array_equal(w, W.astype(np.float64))
    assert np.array_equal(oracle.dequant_f32(qz2, f), W)
    # activations on a coarse grid so the fp64 products and sums are exact
    x = rng.integers(-64, 65, size=(3, K)) / 64.0
    bias = rng.integers(-8, 9, size=N) / 8.0
    y = oracle.linear_f64(x, qz2, f, bias)
    y_ref = np.array([[sum(float(x[m, k]) * float(W[n, k]) for k in range(K))
                       + float(bias[n]) for n in range(N)] for m in range(3)])
    assert np.array_equal(y, y_ref)
    assert y.shape == (3, N)


# --------------------------------------------------------------- P-optimal
@pytest.mark.parametrize("f", ALL_FORMATS, ids=FID)
def test_codes_are_nearest_levels(f):
    """Brute force over every code: each chosen code is (one of) the nearest
    reconstruction level(s) for the scale/offset it was rounded against;
    ties go to the even code."""
    rng = np.random.default_rng(7)
    N, K = 6, 512
    W = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    qz = oracle.quantize(W, f)
    gs = f.group_size
    if f.fmt == "affine":
        s = np.repeat(oracle.numerics.meta_to_f32(qz["scales"], f.meta), gs, 1)
        off = np.repeat(oracle.numerics.meta_to_f32(qz["biases"], f.meta), gs, 1)
    elif f.fmt == "q4k":
        s = np.repeat(qz["s"], 32, 1)
        off = np.repeat(np.minimum(W.reshape(N, -1, 32).min(2), 0), 32, 1)
    elif f.fmt == "q6k":
        s, off = np.repeat(qz["s"], 16, 1), np.zeros((N, K))
    else:
        s, off = np.repeat(qz["scales"], gs, 1), np.zeros((N, K))
    s = s.astype(np.float64)
    off = off.astype(np.float64)
    levels = np.arange(f.qmin, f.qmax + 1, dtype=np.float64)
    dist = np.abs(W[..., None] - (off[..., None] + levels * s[..., None]))
    best = dist.min(axis=2)
    chosen = np.take_along_axis(dist, (qz["codes"].astype(int) - f.qmin)[..., None], 2)[..., 0]
    # fp32 rounding of (w - off)/s can only matter within a hair of a tie
    assert np.all(chosen <= best + 2.0 ** -20 * s)
    # error bound |w - w'| <= s/2 for every element inside the clamp range
    # (meta rounding of scale/bias can push a group's extremes just outside)
    t = (W.astype(np.float64) - off) / s
    inside = (t >= f.qmin - 0.5) & (t <= f.qmax + 0.5)
    assert inside.mean() > 0.95
    assert np.all(chosen[inside] <= 0.5 * s[inside] * (1 + 2.0 ** -20))
    # exact ties go to the even code
    tie = np.abs(t - np.floor(t) - 0.5) == 0
    assert np.all(qz["codes"].astype(int)[tie] % 2 == 0)


# ----------------------------------------------------------------- P-brute
@pytest.mark.parametrize("f", ALL_FORMATS, ids=FID)
@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (3, 512, 3), (8, 256, 1)])
def test_scalar_loop_equals_vectorized(f, N, K, M):
    if K % f.group_size:
        pytest.skip("shape not valid for this group size")
    if f.fmt == "sym4" and f.group_size == 512 and K != 512:
        f = QFormat.sym4(K)
    rng = np.random.default_rng(N * 1000 + K + M)
    W = rng.laplace(0, 0.015, size=(N, K)).astype(np.float32)
    W[0, :16] = 0.0
    a = oracle.quantize(W, f)
    b = quantize_scalar(W, f)
    for key in b:
        assert np.array_equal(np.asarray(a[key]).view(np.uint8) if a[key].dtype == np.float16 else a[key],
                              np.asarray(b[key]).view(np.uint8) if b[key].dtype == np.float16 else b[key]), key
    assert np.array_equal(oracle.dequant_f64(a, f), dequant_scalar_f64(b, f))
    x = rng.normal(size=(M, K))
    bias = rng.normal(size=N)
    y = oracle.linear_f64(x, a, f, bias)
    y2 = linear_scalar_f64(x, b, f, bias)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- tolerance
def test_tolerance_definitions():
    y_ref = np.array([[3.0, 4.0]])
    assert oracle.rel_l2(y_ref * (1 + 1e-3), y_ref) == pytest.approx(1e-3)
    x = np.ones((2, 16))
    bnd = oracle.maxabs_bound(x, 2.0, 16)
    assert bnd.shape == (2, 1) and bnd[0, 0] == pytest.approx(1e-2 * 4 * 2 / 4)


# ------------------------------------------------------------------ P-SNR
def test_per256_steps_beat_per_row_steps():
    """Ablation table of the superscale page: moving the steps from per-row
    to per-256 super-blocks raises the metadata SNR (qualitative only: the
    page's exact dB values come from GGUF tensors that are not available)."""
    rng = np.random.default_rng(2)
    N, K = 64, 4096
    W = rng.laplace(0, 0.015, size=(N, K)).astype(np.float32)
    f = QFormat.q4k()
    qz = oracle.quantize(W, f)
    # the same codes with bf16 metadata (no code quantization)
    ref = (qz["codes"] - np.repeat(qz["z"], 32, 1)) * np.repeat(qz["s"], 32, 1)
    w256 = oracle.dequant_f64(qz, f)
    sc_r, ss_r = _encode_per_super(qz["s"], K // 32, 255, 255)
    zc_r, zs_r = _encode_per_super(qz["z"], K // 32, 255, 255)
    rowq = dict(qz, sc=sc_r.astype(np.uint8), zc=zc_r.astype(np.uint8),
                sstep=np.repeat(ss_r, K // 256, 1), zstep=np.repeat(zs_r, K // 256, 1))
    wrow = oracle.dequant_f64(rowq, f)
    assert oracle.snr_db(ref, w256) > oracle.snr_db(ref, wrow) + 0.5
