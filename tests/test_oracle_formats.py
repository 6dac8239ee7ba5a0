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


# ---- block sizes ("Double quantization": smaller blocks quantize more precisely and pay
# the per-block constant more often; larger blocks the reverse) ----------------------------
@pytest.mark.parametrize("block", nf4.BLOCKS)
def test_block_overhead_closed_forms(block):
    """Constant overhead per weight: a 32-bit constant per block is 32/B bits; with double
    quantization an 8-bit constant per block plus a 32-bit scale per 256 blocks, 8/B +
    32/(256 B), plus one 32-bit mean per tensor.  At B = 64: 0.5 and 0.126953125."""
    n = 256 * block * 1000
    assert nf4.constant_bits_per_param(n, False, block) == 32 / block
    assert nf4.constant_bits_per_param(n, True, block) == 8 / block + 32 / (256 * block) + 32 / n
    if block == 64:
        assert nf4.constant_bits_per_param(n, False, block) == 0.5
        assert abs(nf4.constant_bits_per_param(n, True, block) - 32 / n - 0.126953125) < 1e-12
    sb = nf4.storage_bytes(n, True, block)
    assert sb["codes"] == n // 2 and sb["absmax"] == n // block


@pytest.mark.parametrize("block", nf4.BLOCKS)
def test_blocks_are_independent(block):
    """Quantizing a tensor equals quantizing each of its blocks as a tensor of its own (the
    codes and the per-block constant depend on that block alone); the absmax element
    reconstructs exactly without double quantization; requantizing the dequantized weight
    gives the same codes; a ragged tail holds the zero code."""
    nblk = 6
    w = workloads.normal_bf16(60 + block, (nblk * block,), 0.02)
    q = nf4.quantize(w, double_quant=False, block=block)
    codes = nf4.unpack_nibbles(q["codes"], w.size).reshape(nblk, block)
    for b in range(nblk):
        qb = nf4.quantize(w[b * block:(b + 1) * block], double_quant=False, block=block)
        np.testing.assert_array_equal(nf4.unpack_nibbles(qb["codes"], block), codes[b])
        assert qb["absmax_true"][0] == q["absmax_true"][b]
    vals = nf4.bf16_to_f32(w).reshape(nblk, block)
    arg = np.abs(vals).argmax(axis=1)
    d = nf4.bf16_to_f32(nf4.dequantize(q)).reshape(nblk, block)
    np.testing.assert_array_equal(d[np.arange(nblk), arg], vals[np.arange(nblk), arg])
    q2 = nf4.quantize(nf4.dequantize(q), double_quant=False, block=block)
    np.testing.assert_array_equal(q2["codes"], q["codes"])
    qr = nf4.quantize(w[: block + 5], double_quant=True, block=block)
    assert qr["codes"].size == nf4.code_elems(block + 5, block) // 2
    tail = nf4.unpack_nibbles(qr["codes"], nf4.code_elems(block + 5, block))[block + 5:]
    assert np.all(tail == nf4.ZERO_CODE)


def test_block_size_error_ordering():
    """Relative quantization error grows with the block size, on Gaussian weights and more
    steeply with 0.1 % of the entries scaled by 20 (the outliers a larger block shares its
    constant with)."""
    for outlier_p in (0.0, 0.001):
        W = workloads.normal_bf16(7, (1024, 1024), 0.02, outlier_p=outlier_p, mask_seed=8)
        w = nf4.bf16_to_f32(W).astype(np.float64)
        err = []
        for block in nf4.BLOCKS:
            q = nf4.quantize(W, double_quant=True, block=block)
            d = nf4.bf16_to_f32(nf4.dequantize(q, W.shape)).astype(np.float64)
            err.append(np.mean((d - w) ** 2) / np.mean(w ** 2))
        assert all(a < b for a, b in zip(err, err[1:])), (outlier_p, err)
