"""Pins for the NF4 / double-quantization oracle against what the pages and the
mathematics fix (no GPU)."""
import math
import statistics
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nf4
from conftest import read_golden


# ------------------------------------------------------------------------------------------
# Codebook
# ------------------------------------------------------------------------------------------
def test_codebook_structure():
    lv = nf4.nf4_levels()
    assert lv.shape == (16,) and lv.dtype == np.float32
    assert np.all(np.diff(lv.astype(np.float64)) > 0), "levels must be strictly increasing"
    assert (lv < 0).sum() == 7 and (lv > 0).sum() == 8
    assert lv[nf4.ZERO_CODE] == 0.0 and not np.signbit(lv[nf4.ZERO_CODE])
    assert lv[0] == -1.0 and lv[15] == 1.0          # ends exactly at -1 and +1


def test_codebook_printed_values():
    lv = nf4.nf4_levels()
    for idx, val, dec in read_golden("nf4_printed_values.txt"):
        assert round(float(lv[int(idx)]), int(dec)) == float(val), (idx, lv[int(idx)], val)


def test_codebook_two_inverse_cdf_libraries_agree():
    nd = statistics.NormalDist()
    lv_stat = nf4.nf4_levels(lambda p: np.array([nd.inv_cdf(float(q)) for q in np.atleast_1d(p)]))
    assert np.array_equal(lv_stat.view(np.uint32), nf4.nf4_levels().view(np.uint32))


def test_codebook_tail_quantiles():
    # before normalization the extreme levels are the quantiles at the offset probability
    lv64 = nf4.nf4_levels_f64()
    nd = statistics.NormalDist()
    top = nd.inv_cdf(nf4.OFFSET)
    pos_p = [nf4.OFFSET + i * (0.5 - nf4.OFFSET) / 8 for i in range(8)]
    for i, p in enumerate(pos_p):
        assert lv64[15 - i] == pytest.approx(nd.inv_cdf(p) / top, abs=1e-12)
    neg_p = [nf4.OFFSET + i * (0.5 - nf4.OFFSET) / 7 for i in range(7)]
    for i, p in enumerate(neg_p):
        assert lv64[i] == pytest.approx(-nd.inv_cdf(p) / top, abs=1e-12)


def test_equal_mass_on_standard_normal():
    """Each level receives roughly 1/16 of N(0,1) samples at the codebook's own scale."""
    rng = np.random.default_rng(1234)
    z = rng.standard_normal(4_000_000)
    top = statistics.NormalDist().inv_cdf(nf4.OFFSET)
    c = nf4.nearest_level((z / top).astype(np.float32))
    frac = np.bincount(c, minlength=16) / c.size
    assert frac.min() > 0.050 and frac.max() < 0.075, frac


def test_block_occupancy_two_to_nine_percent():
    """With per-64-block absmax the bins hold roughly 2%..9% ([Explainer] "NormalFloat")."""
    rng = np.random.default_rng(99)
    z = rng.standard_normal(2 ** 22).astype(np.float32)
    w = torch.from_numpy(z).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c = nf4.nf4_codes(w)
    frac = np.bincount(c, minlength=16) / c.size
    assert 0.014 < frac.min() < 0.025, frac
    assert 0.085 < frac.max() < 0.097, frac


# ------------------------------------------------------------------------------------------
# bf16 / fp8 conversions against library routines
# ------------------------------------------------------------------------------------------
def _interesting_f32(n=200_000, seed=5):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # ties: exactly half-way between two bf16 values, both parities
    ties = (rng.integers(0, 2 ** 16, size=4000).astype(np.uint32) << 16) | 0x8000
    extra = np.array([0.0, -0.0, 1e-45, -1e-45, 1.1754942e-38, 3.4e38, -3.4e38], dtype=np.float32)
    out = np.concatenate([x, ties.view(np.float32), extra])
    return out[np.isfinite(out)]


def test_bf16_rne_matches_torch():
    x = _interesting_f32()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.f32_to_bf16(x), ref)
    assert np.array_equal(nf4.bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(7)
    vals = [rng.uniform(-448, 448, 100_000), rng.standard_normal(100_000) * 2.0 ** rng.integers(-12, 8, 100_000),
            np.linspace(-448, 448, 20001)]
    # every exact midpoint between adjacent E4M3 values (ties to even) and values just off them
    pos = np.array([nf4.e4m3_decode(np.uint8(c)) for c in range(0x7F)], dtype=np.float64)
    mids = (pos[:-1] + pos[1:]) / 2
    vals += [mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)]
    y = np.concatenate(vals).astype(np.float32)
    y = y[np.abs(y) <= 448]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(nf4.e4m3_encode(y), ref)


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(nf4.e4m3_decode(codes).view(np.uint32), ref.view(np.uint32))


def test_e4m3_encode_slightly_above_448_rounds_to_448():
    y = np.array([448.0, np.nextafter(np.float32(448), np.float32(500)), 448 * (1 + 2 ** -22)], dtype=np.float32)
    assert np.all(nf4.e4m3_encode(y) == 0x7E)
    assert np.all(nf4.e4m3_encode(-y) == 0xFE)


# ------------------------------------------------------------------------------------------
# Encoder
# ------------------------------------------------------------------------------------------
def _threshold_count_codes(x):
    """Independent encoder: count exact midpoints strictly below x (ties go to the lower level)."""
    lv = nf4.nf4_levels().astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0            # exact in float64 for fp32 operands
    return (np.asarray(x, np.float64)[:, None] > mids[None, :]).sum(axis=1).astype(np.uint8)


def test_encoder_exhaustive_bf16_sweep():
    """All finite bf16 patterns as weights, for several block absmax values."""
    allbits = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    w = nf4.bf16_to_f32(allbits)
    w = w[np.isfinite(w)]
    for a in [1.0, 0.02, 0.0390625, 3.0, 1e-3, 448.0, 6.1e-5, 2.0 ** -120]:
        a32 = np.float32(nf4.bf16_to_f32(nf4.f32_to_bf16(np.array([a], np.float32)))[0])
        ww = w[np.abs(w) <= a32]
        x = nf4.normalize_blocks(ww[None, :], np.array([a32], np.float32))[0]
        assert np.array_equal(nf4.nearest_level(x), _threshold_count_codes(x)), a


def test_encoder_exact_rational_on_sample():
    """Pure-Python exact nearest level (Fractions) on a random sample of normalized values."""
    lv = [Fraction(float(v)) for v in nf4.nf4_levels()]
    rng = np.random.default_rng(11)
    x = rng.uniform(-1, 1, 3000).astype(np.float32)
    lvf = nf4.nf4_levels().astype(np.float64)
    x = np.concatenate([x, ((lvf[:-1] + lvf[1:]) / 2).astype(np.float32), nf4.nf4_levels()])
    got = nf4.nearest_level(x)
    for xi, gi in zip(x, got):
        fx = Fraction(float(xi))
        d = [abs(fx - l) for l in lv]
        best = min(range(16), key=lambda k: (d[k], k))
        assert best == gi, (xi, best, gi)


def test_encoder_ties_go_to_lower_index():
    lv = nf4.nf4_levels().astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0
    exact = mids[mids.astype(np.float32).astype(np.float64) == mids]   # midpoints that are fp32 values
    assert exact.size >= 4
    k = np.searchsorted(lv, exact) - 1
    assert np.array_equal(nf4.nearest_level(exact.astype(np.float32)), k.astype(np.uint8))


def test_absmax_element_and_zero_codes():
    rng = np.random.default_rng(3)
    z = (rng.standard_normal((512, 64)) * 0.02).astype(np.float32)
    z[:, 5] = 0.0
    w = nf4.f32_to_bf16(z)
    c = nf4.nf4_codes(w).reshape(512, 64)
    wf = nf4.bf16_to_f32(w).reshape(512, 64)
    am = np.argmax(np.abs(wf), axis=1)
    top = c[np.arange(512), am]
    assert np.all((top == 0) | (top == 15))
    assert np.all(top[wf[np.arange(512), am] > 0] == 15)
    assert np.all(c[:, 5] == nf4.ZERO_CODE)


def test_zero_and_subnormal_blocks():
    w = np.zeros(64 * 3 + 10, dtype=np.uint16)
    w[64:128] = 0x0001                 # a bf16 subnormal block -> flushed zero block
    w[128:192] = 0x3C00                # 2^-7 everywhere -> all +1
    q = nf4.quantize(w, double_quant=False)
    c = nf4.unpack_nibbles(q["codes"], w.size)
    assert np.all(c[:128] == 7) and np.all(c[128:192] == 15) and np.all(c[192:] == 7)
    assert q["absmax_true"][0] == 0 and q["absmax_true"][1] == 0
    d = nf4.dequantize(q)
    assert np.array_equal(d[128:192], w[128:192])


def test_pack_layout_and_ragged_tail():
    codes = np.arange(16, dtype=np.uint8) % 16
    p = nf4.pack_nibbles(codes, 16)
    assert p.size == 32                      # one whole block
    # group 0: bytes hold (e0,e4), (e1,e5), (e2,e6), (e3,e7) as low/high nibbles
    assert list(p[:8]) == [0x40, 0x51, 0x62, 0x73, 0xC8, 0xD9, 0xEA, 0xFB]
    assert np.all(p[8:] == 0x77)             # padding is the exact-zero code
    assert np.array_equal(nf4.unpack_nibbles(p, 16), codes)
    rng = np.random.default_rng(2)
    c = rng.integers(0, 16, 201).astype(np.uint8)
    assert np.array_equal(nf4.unpack_nibbles(nf4.pack_nibbles(c, 201), 201), c)


# ------------------------------------------------------------------------------------------
# Double quantization
# ------------------------------------------------------------------------------------------
def test_mean_exact_sum():
    # values whose naive float32 running sum loses bits, exact rational mean known
    a = np.array([2.0 ** 20] + [1.0] * 1000 + [2.0 ** -10] * 7, dtype=np.float32)
    exact = (Fraction(2 ** 20) + 1000 + Fraction(7, 1024)) / a.size
    assert nf4.absmax_mean(a) == np.float32(float(exact))
    b = np.full(777, 0.0390625, dtype=np.float32)
    assert nf4.absmax_mean(b) == np.float32(0.0390625)


def test_constant_absmax_gives_exact_scales():
    a = np.full(1000, 0.03125, dtype=np.float32)
    c2, c1, mu = nf4.double_quantize(a)
    assert mu == np.float32(0.03125) and np.all(c1 == 0) and np.all(c2 == 0)
    assert np.array_equal(nf4.block_scales_dq(c2, c1, mu), a)


def test_double_quant_error_bound_and_group_max():
    rng = np.random.default_rng(8)
    w = nf4.f32_to_bf16((rng.standard_normal(64 * 5000) * 0.02).astype(np.float32))
    a = nf4.blockwise_absmax(w)
    c2, c1, mu = nf4.double_quantize(a)
    s = nf4.block_scales_dq(c2, c1, mu).astype(np.float64)
    x = a.astype(np.float64) - float(mu)
    sup = np.arange(a.size) // nf4.SUPER
    # E4M3 with 3 fraction bits: relative error <= 2^-4 for normals, absolute <= 2^-10 * c1 below 2^-6
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * c1[sup]) + 4e-7 * (np.abs(a) + abs(float(mu)))
    assert np.all(np.abs(s - a) <= bound)
    # each group's largest centered magnitude maps to +-448
    for j in range(c1.size):
        g = c2[j * nf4.SUPER:(j + 1) * nf4.SUPER]
        assert (g & 0x7F).max() == 0x7E
    assert a.size == 5000 and c1.size == math.ceil(5000 / 256)


def test_no_double_quant_reconstructs_block_max_exactly():
    rng = np.random.default_rng(9)
    w = nf4.f32_to_bf16((rng.standard_normal(64 * 300) * 0.02).astype(np.float32))
    q = nf4.quantize(w, double_quant=False)
    d = nf4.bf16_to_f32(nf4.dequantize(q)).reshape(300, 64)
    wf = nf4.bf16_to_f32(w).reshape(300, 64)
    am = np.argmax(np.abs(wf), axis=1)
    assert np.array_equal(d[np.arange(300), am], wf[np.arange(300), am])


def test_requantize_is_idempotent_without_double_quant():
    rng = np.random.default_rng(10)
    w = nf4.f32_to_bf16((rng.standard_normal(64 * 400) * 0.02).astype(np.float32))
    q1 = nf4.quantize(w, double_quant=False)
    q2 = nf4.quantize(nf4.dequantize(q1), double_quant=False)
    assert np.array_equal(q1["codes"], q2["codes"])
    assert np.array_equal(q1["absmax_true"], q2["absmax_true"])


def test_dequant_error_within_half_level_gap():
    rng = np.random.default_rng(12)
    w = nf4.f32_to_bf16((rng.standard_normal(64 * 1000) * 0.02).astype(np.float32))
    q = nf4.quantize(w, double_quant=False)
    d = nf4.bf16_to_f32(nf4.dequantize(q)).astype(np.float64).reshape(1000, 64)
    wf = nf4.bf16_to_f32(w).astype(np.float64).reshape(1000, 64)
    gap = np.diff(nf4.nf4_levels().astype(np.float64)).max()
    a = q["absmax_true"].astype(np.float64)[:, None]
    assert np.all(np.abs(d - wf) <= a * (gap / 2 + 2 ** -8))


# ------------------------------------------------------------------------------------------
# Storage closed forms printed on the pages
# ------------------------------------------------------------------------------------------
def _closed():
    return {k: (float(v), float(t)) for k, v, t, _ in read_golden("closed_forms.txt")}


def test_closed_form_storage_figures():
    g = _closed()
    big = 64 * 256 * 10 ** 6                                     # many whole groups: the asymptote
    bits_dq = nf4.constant_bits_per_param(big, True)
    bits_no = nf4.constant_bits_per_param(big, False)
    assert bits_dq == pytest.approx(8 / 64 + 32 / (64 * 256), rel=1e-6)
    got = {
        "bits_const_no_dq": bits_no,
        "bits_const_dq": bits_dq,
        "bits_saved": bits_no - bits_dq,
        "bits_total_no_dq": 4 + bits_no,
        "bits_total_dq": 4 + bits_dq,
        "gb_saved_65b": (bits_no - bits_dq) * 65e9 / 8 / 1e9,
    }
    n = 4096 * 4096
    sb = nf4.storage_bytes(n, True)
    got["mb_4096sq_bf16"] = 2 * n / 1e6
    got["mb_4096sq_nf4_dq"] = sum(sb.values()) / 1e6
    got["blocks_4096sq"] = nf4.num_blocks(n)
    got["adapter_numbers_4096_r64"] = 4096 * 64 + 64 * 4096
    got["adapter_mb_4096_r64"] = 2 * (4096 * 64 + 64 * 4096) / 2 ** 20
    got["gb_8b_nf4"] = sum(nf4.storage_bytes(8 * 10 ** 9, True).values()) / 1e9
    got["gb_70b_nf4"] = sum(nf4.storage_bytes(70 * 10 ** 9, True).values()) / 1e9
    for k, (v, tol) in g.items():
        assert got[k] == pytest.approx(v, rel=max(tol, 1e-12), abs=0 if tol else 1e-12), (k, got[k], v)
    assert sum(sb.values()) == 8_654_852
