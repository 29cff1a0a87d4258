"""Pins of the metadata-encoding ablation (ExecuTorch PR #20571, "[cuda]
Nested Superscale Quantization for CUDA Weights (int4 / int6)", sections
"Ablation study" and "Analysis"): the bits-per-weight column of the table,
the encoding rule against the pinned nested conversion, lattice cases, and
the orderings the page draws from its SNR column, on synthetic Laplace
weights.  The SNR values themselves were measured on GGUF tensors that are
not available (parity unpinned for them)."""
import numpy as np
import pytest

import oracle
from oracle import QFormat
from oracle.ablation import encode_value, dequant_f64, bits_per_weight
from oracle.convert import to_q4k, plain_int4_f64

# (scale code, scale step, its dtype, zero code, zero step, its dtype), bpw
# as printed in the table
TABLE = [
    (("u8", "256", "f16", "u8", "256", "f16"), 4.625),
    (("u8", "256", "f16", "u8", "256", "bf16"), 4.625),
    (("u8", "256", "f16", "u8", "row", "f16"), 4.5625),
    (("u8", "256", "f16", "u8", "row", "bf16"), 4.5625),
    (("u8", "256", "bf16", "u8", "row", "bf16"), 4.5625),
    (("u8", "row", "bf16", "u8", "row", "bf16"), 4.500),
    (("u8", "row", "f16", "u8", "row", "bf16"), 4.500),
    (("u6", "256", "f16", "u8", "256", "f16"), 4.5625),
    (("u6", "256", "f16", "u6", "256", "f16"), 4.500),
]


@pytest.mark.parametrize("enc,bpw", TABLE, ids=lambda v: str(v))
def test_bpw_column(enc, bpw):
    nominal, with_rows = bits_per_weight(enc, 8192)
    assert nominal == bpw
    n_row = sum(1 for c, s in ((enc[0], enc[1]), (enc[3], enc[4])) if s == "row")
    assert with_rows == bpw + 16.0 * n_row / 8192


def test_bpw_last_row_reading():
    """The table's last row (6-bit scale, 8-bit zero, per-row steps) prints
    4.441: 4 + 6/32 + 8/32 = 4.4375 plus the two per-row steps, 32/K,
    which gives 4.441 for K between 8900 and 9400."""
    enc = ("u6", "row", "f16", "u8", "row", "f16")
    assert bits_per_weight(enc, 8192)[0] == 4.4375
    assert round(bits_per_weight(enc, 9142)[1], 3) == 4.441


def test_u8_per256_equals_the_nested_conversion():
    """uint8 codes with per-256 fp16 steps are the Q4K encoding itself."""
    rng = np.random.default_rng(1)
    s = rng.uniform(0, 0.01, size=(3, 32)).astype(np.float32)
    z = rng.uniform(0, 15, size=(3, 32)).astype(np.float32)
    u = rng.integers(0, 16, size=(3, 1024)).astype(np.uint8)
    qz = to_q4k(u, s, z)
    S = qz["sc"].astype(np.float64) * np.repeat(qz["sstep"].astype(np.float64), 8, axis=1)
    Z = qz["zc"].astype(np.float64) * np.repeat(qz["zstep"].astype(np.float64), 8, axis=1)
    assert np.array_equal(encode_value(s, "u8", "256", "f16"), S)
    assert np.array_equal(encode_value(z, "u8", "256", "f16"), Z)
    w = dequant_f64(u, s, z, ("u8", "256", "f16", "u8", "256", "f16"))
    assert np.array_equal(w, oracle.dequant_f64(qz, QFormat.q4k()))


def test_encode_value_hand_worked():
    """6-bit codes on a lattice: values k * 2^-10 with max 63 * 2^-10 give
    step 2^-10 (exact in fp16 and bf16) and codes k; a per-row span of 8
    groups (K = 256) equals the per-256 span; bf16 codes are bf16 rounding
    (1 + 2^-8 is a tie and rounds to 1, 1 + 3 * 2^-8 rounds up)."""
    k = np.array([[63, 0, 31, 32, 1, 62, 17, 40]])
    v = (k * 2.0 ** -10).astype(np.float32)
    for dt in ("f16", "bf16"):
        assert np.array_equal(encode_value(v, "u6", "256", dt), k * 2.0 ** -10)
        assert np.array_equal(encode_value(v, "u6", "row", dt), k * 2.0 ** -10)
    b = np.array([[1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 0.5, 3.0]], np.float32)
    assert encode_value(b, "bf16", "256", "f16").tolist() == [[1.0, 1.0 + 2 * 2.0 ** -7, 0.5, 3.0]]
    # the 6-bit step of a super-block whose max is 1: fp16(1/63) = 1040 * 2^-16
    vv = np.array([[1.0, 0.5, 0.25, 0.0, 0.75, 0.1, 0.9, 0.3]], np.float32)
    out = encode_value(vv, "u6", "256", "f16")
    step = 1040 * 2.0 ** -16
    assert np.array_equal(out, np.rint(vv.astype(np.float64) / step).clip(0, 63) * step)
    with pytest.raises(ValueError):
        encode_value(-vv, "u8", "256", "f16")


def test_ablation_orderings():
    """The orderings the page's analysis states, on Laplace weights (SNR of
    each encoding against the plain per-group form it re-encodes):
    per-256 steps beat per-row steps for the zero point, and per-row for
    both is lowest; a 6-bit scale code loses several dB against uint8, and
    a 6-bit zero code as well loses more."""
    rng = np.random.default_rng(6)
    W = rng.laplace(0, 0.015, size=(128, 8192)).astype(np.float32)
    q4 = oracle.quantize(W, QFormat.q4k())
    ref = plain_int4_f64(q4["codes"], q4["s"], q4["z"])

    def snr(enc):
        return oracle.snr_db(ref, dequant_f64(q4["codes"], q4["s"], q4["z"], enc))

    both256 = snr(("u8", "256", "f16", "u8", "256", "f16"))
    zero_row = snr(("u8", "256", "f16", "u8", "row", "f16"))
    both_row = snr(("u8", "row", "f16", "u8", "row", "f16"))
    s6 = snr(("u6", "256", "f16", "u8", "256", "f16"))
    s6z6 = snr(("u6", "256", "f16", "u6", "256", "f16"))
    assert both256 > zero_row > both_row
    assert both256 - s6 > 3.0
    assert s6 - s6z6 > 3.0
