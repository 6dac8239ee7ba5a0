"""Pins for the other 4-bit data types the pages compare NF4 with (FP4, Int4), no GPU.

"NormalFloat: 4 bits for a bell curve" (QLoRA explainer page) compares NF4 with FP4 and
Int4 and ranks NF4 first for normally distributed weights.  The oracle's FP4 table is the
E2M1 value set scaled by 1/6 and its Int4 table is k/7 (the absmax integer quantizer of
"Quantize in blocks, not all at once" with largest code 7); each has one unused entry
below -1 so that all tables are strictly ascending with 16 entries.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import nf4


def test_fp4_value_set_closed_form():
    """Positive values of a 4-bit float with 2 exponent bits (bias 1) and 1 mantissa bit:
    0, the subnormal 1/2, and the numbers with two significant bits a * 2^b, a in {2, 3},
    b in {-1, 0, 1}; scaled by 1/6 so the largest is 1."""
    pos = {Fraction(0), Fraction(1, 2)} | {Fraction(a) * Fraction(2) ** b for a in (2, 3) for b in (-1, 0, 1)}
    want = sorted({v / 6 for v in pos} | {-v / 6 for v in pos})
    lv = nf4.fp4_levels()
    assert len(want) == 15
    assert lv[0] < -1.0                                      # the unused entry
    np.testing.assert_array_equal(lv[1:], np.array([float(v) for v in want], dtype=np.float32))
    assert lv[1] == -1.0 and lv[-1] == 1.0 and nf4.zero_code(lv) == 8


def test_int4_levels_are_sevenths():
    lv = nf4.int4_levels().astype(np.float64)
    k = np.rint(lv * 7)
    np.testing.assert_array_equal(k, np.arange(-8, 8))
    assert np.all(np.abs(lv * 7 - k) < 1e-6)
    assert lv[1] == -1.0 and lv[-1] == 1.0 and nf4.zero_code(lv) == 8


@pytest.mark.parametrize("name", nf4.CODEBOOKS)
def test_tables_strictly_ascending(name):
    lv = nf4.codebook_levels(name)
    assert lv.dtype == np.float32 and lv.shape == (16,)
    assert np.all(np.diff(lv.astype(np.float64)) > 0)


@pytest.mark.parametrize("name", ["fp4", "int4"])
def test_nearest_level_exact_rational(name):
    """Brute-force nearest in float64 equals the exact-rational nearest (ties to the lower
    index) on random points and on every midpoint and its fp32 neighbours."""
    lv = nf4.codebook_levels(name)
    rng = np.random.default_rng(3)
    pts = list(rng.uniform(-1, 1, 3000).astype(np.float32))
    for k in range(15):
        m = np.float32((float(lv[k]) + float(lv[k + 1])) / 2)
        pts += [np.nextafter(m, np.float32(-2)), m, np.nextafter(m, np.float32(2))]
    pts = np.array(pts, dtype=np.float32)
    got = nf4.nearest_level(pts, lv)
    fl = [Fraction(float(v)) for v in lv]
    for x, g in zip(pts, got):
        fx = Fraction(float(x))
        d = [abs(fx - v) for v in fl]
        assert g == d.index(min(d)), (name, x)
    inside = np.abs(pts) <= 1.0
    assert 0 not in set(got[inside].tolist())                # the unused entry is never chosen in [-1, 1]


@pytest.mark.parametrize("name", ["fp4", "int4"])
def test_quantize_block_structure(name):
    """The block maximum reconstructs exactly without double quant (level +-1 times the
    absmax), zeros stay zero, padding holds the zero code, and requantizing the dequantized
    weight gives the same codes."""
    inp = workloads.custom_linear(4, 256, 40, 8, seed=21)
    W = inp.W
    q = nf4.quantize(W, double_quant=False, codebook=name)
    lv = nf4.codebook_levels(name)
    codes = nf4.unpack_nibbles(q["codes"], W.size).reshape(-1, 64)
    blocks = nf4.bf16_to_f32(W).reshape(-1, 64)
    arg = np.abs(blocks).argmax(axis=1)
    top = codes[np.arange(codes.shape[0]), arg]
    assert set(top.tolist()) <= {1, 15}
    Wd = nf4.dequantize(q, W.shape)
    np.testing.assert_array_equal(nf4.bf16_to_f32(Wd).reshape(-1, 64)[np.arange(codes.shape[0]), arg],
                                  blocks[np.arange(codes.shape[0]), arg])
    q2 = nf4.quantize(Wd, double_quant=False, codebook=name)
    np.testing.assert_array_equal(q2["codes"], q["codes"])
    # a ragged tensor: positions past the end hold the zero code
    qr = nf4.quantize(W.reshape(-1)[:100], double_quant=True, codebook=name)
    tail = nf4.unpack_nibbles(qr["codes"], 128)[100:]
    assert np.all(tail == nf4.zero_code(lv))


def test_mse_ordering_on_gaussian_blocks():
    """On normally distributed weights with per-64 absmax scaling NF4 has the smallest
    quantization error, then FP4, then Int4 (the order the pages give for the data types)."""
    W = workloads.normal_bf16(5, (2048, 512), 0.02)
    w = nf4.bf16_to_f32(W).astype(np.float64)
    err = {}
    for name in nf4.CODEBOOKS:
        q = nf4.quantize(W, double_quant=False, codebook=name)
        d = nf4.bf16_to_f32(nf4.dequantize(q, W.shape)).astype(np.float64)
        err[name] = np.mean((d - w) ** 2) / np.mean(w ** 2)
    assert err["nf4"] < err["fp4"] < err["int4"], err
    assert 0.005 < err["nf4"] < 0.012 and err["int4"] < 0.02
