"""Pins for the oracle helpers that the full-size GPU checks use on selected blocks,
rows or columns only: each must equal the corresponding slice of the whole-tensor
oracle function it stands for.  No GPU."""
import numpy as np
import pytest

import workloads
from oracle import linear, nf4


def _weight(rows, cols, seed, zero_block=None, block=64):
    w = workloads.normal_bf16(seed, (rows, cols), 0.02, outlier_p=0.01, mask_seed=seed + 5)
    if zero_block is not None:
        flat = w.reshape(-1)
        flat[zero_block * block:(zero_block + 1) * block] = 0
    return w


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "int4"])
@pytest.mark.parametrize("block", [32, 64, 128, 256])
def test_codes_for_blocks_equals_full_quantizer(block, codebook):
    """Codes of selected blocks (first, last and ragged, an all-zero block, random ones)
    equal the whole-tensor quantizer's codes of the same blocks, pad positions included."""
    rows, cols = 37, 200                         # 7400 weights: a partial last block for every size
    w = _weight(rows, cols, seed=11 + block, zero_block=3, block=block)
    numel = rows * cols
    lv = nf4.codebook_levels(codebook)
    q = nf4.quantize(w, double_quant=True, codebook=codebook, block=block)
    nblk = nf4.num_blocks(numel, block)
    full = nf4.unpack_nibbles(q["codes"], nf4.code_elems(numel, block))[:nblk * block].reshape(nblk, block)
    ids = np.array([nblk - 1, 0, 3, 3, nblk // 2] + list(np.random.default_rng(block).integers(0, nblk, 9)))
    got = nf4.codes_for_blocks(w, q["absmax_true"], ids, levels=lv, block=block)
    assert got.shape == (ids.size, block)
    np.testing.assert_array_equal(got, full[ids])
    assert np.all(got[2] == nf4.zero_code(lv))               # the all-zero block
    tail = numel - (nblk - 1) * block                          # valid weights of the last block
    if tail < block:
        assert np.all(got[0, tail:] == nf4.zero_code(lv))     # padding takes the zero code


@pytest.mark.parametrize("dq", [True, False])
def test_sampled_dequant_equals_full_dequant(dq):
    """Selected blocks dequantized from their codes and the whole tensor's block scales
    equal the whole-tensor dequantized weight on those blocks."""
    rows, cols = 24, 640
    w = _weight(rows, cols, seed=5, zero_block=7)
    q = nf4.quantize(w, double_quant=dq)
    full = nf4.dequantize(q, (rows, cols)).reshape(-1, 64)
    ids = np.array([0, 7, 239, 100, 101, 5])
    if dq:
        scales = nf4.block_scales_dq(*nf4.double_quantize(nf4.blockwise_absmax(w)))
    else:
        scales = nf4.blockwise_absmax(w)
    np.testing.assert_array_equal(scales, q["scales"])
    codes = nf4.codes_for_blocks(w, nf4.blockwise_absmax(w), ids)
    got = nf4.dequantize_codes(codes.reshape(-1), scales[ids]).reshape(ids.size, 64)
    np.testing.assert_array_equal(got, full[ids])


def test_row_and_adapter_helpers_equal_full_results():
    """forward_rows and backward_dx_rows equal the selected rows of forward / backward,
    adapter_grads equals backward's dA and dB (rows unsorted and repeated)."""
    inp = workloads.custom_linear(40, 192, 128, 16, seed=21)
    Wd = nf4.dequantize(nf4.quantize(inp.W), (128, 192))
    s = 0.75
    y, _ = linear.forward(inp.X, Wd, inp.A, inp.B, s)
    dx, da, db = linear.backward(inp.dY, inp.X, Wd, inp.A, inp.B, s)
    rows = np.array([39, 0, 17, 17, 5])
    np.testing.assert_array_equal(linear.forward_rows(inp.X, Wd, inp.A, inp.B, s, rows), y[rows])
    np.testing.assert_allclose(linear.backward_dx_rows(inp.dY, Wd, inp.A, inp.B, s, rows), dx[rows],
                               rtol=1e-13, atol=1e-13)
    da2, db2 = linear.adapter_grads(inp.dY, inp.X, inp.A, inp.B, s)
    np.testing.assert_array_equal(da2, da)
    np.testing.assert_array_equal(db2, db)
