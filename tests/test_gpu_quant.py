"""GPU parity: quantization, double quantization and dequantization must equal the
oracle bit for bit (codes, 8-bit constants, fp32 group scales, mean, bf16 weights)."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_11_amd as Q
import workloads
from helpers import dev_bf16, host, host_u16, log, require_gpu
from oracle import nf4

pytestmark = pytest.mark.gpu


def _gpu_quant(w_u16: np.ndarray, shape, dq: bool, codebook="nf4", block=64):
    require_gpu()
    W = dev_bf16(w_u16.reshape(-1)).reshape(shape)
    q = Q.qlora_quantize_nf4(W, double_quant=dq, codebook=Q.CODEBOOKS[codebook], block=block)
    deq = Q.qlora_dequant(q)
    torch.cuda.synchronize()
    return q, deq


def _check(w_u16: np.ndarray, shape, dq: bool, label: str, codebook="nf4", block=64):
    log("quantize", label, shape, "dq" if dq else "no-dq", codebook, "block", block)
    q, deq = _gpu_quant(w_u16, shape, dq, codebook, block)
    ref = nf4.quantize(w_u16, double_quant=dq, codebook=codebook, block=block)
    codes = host(q.codes)
    bad = np.flatnonzero(codes != ref["codes"])
    assert bad.size == 0, f"{label}: {bad.size} code bytes differ, first at byte {bad[:5]}"
    if dq:
        assert np.array_equal(host(q.mu).view(np.uint32), np.array([ref["mu"]], np.float32).view(np.uint32)), \
            f"{label}: mu {host(q.mu)} vs {ref['mu']}"
        assert np.array_equal(host(q.c1).view(np.uint32), ref["c1"].view(np.uint32)), f"{label}: c1 differs"
        assert np.array_equal(host(q.absmax), ref["c2"]), f"{label}: c2 differs"
    else:
        assert np.array_equal(host(q.absmax).view(np.uint32), ref["absmax_true"].view(np.uint32))
    want = nf4.dequantize(ref)
    got = host_u16(deq).reshape(-1)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{label}: {bad.size} dequantized values differ, first at {bad[:5]}"
    return q


@pytest.mark.parametrize("shape,dq", [((256, 256), True), ((256, 256), False), ((3, 77), True), ((1, 64), True),
                                      ((1000, 1000), True), ((1, 64 * 256 * 3 + 5), True), ((517, 333), False)])
def test_quantize_small_shapes(shape, dq):
    w = workloads.normal_bf16(7 + shape[0], shape, 0.02)
    _check(w, shape, dq, f"gauss{shape}")


@pytest.mark.parametrize("block", [32, 128, 256])
@pytest.mark.parametrize("shape,dq", [((256, 256), True), ((256, 256), False), ((3, 77), True), ((1, 96), False),
                                      ((1, 64 * 256 * 3 + 5), True), ((4096, 4096), True)])
def test_quantize_block_sizes(block, shape, dq):
    """Blocks of 32, 128 and 256 weights through the same kernels: codes (padding to whole
    blocks and 64-element chunks included), constants and dequantized weights bit-exact."""
    w = workloads.normal_bf16(13 + shape[1] + block, shape, 0.02)
    _check(w, shape, dq, f"block{block}{shape}", block=block)


@pytest.mark.parametrize("codebook", ["fp4", "int4"])
@pytest.mark.parametrize("shape,dq", [((256, 256), True), ((256, 256), False), ((3, 77), True),
                                      ((4096, 4096), True)])
def test_quantize_other_codebooks(codebook, shape, dq):
    """FP4 and Int4 tables through the same kernels: codes, constants and dequantized
    weights bit-exact (ragged tails hold the tables' zero code, index 8)."""
    w = workloads.normal_bf16(11 + shape[1], shape, 0.02)
    _check(w, shape, dq, f"{codebook}{shape}", codebook)


def test_quantize_c1_config():
    lin = workloads.CONFIGS[1].linears[0]
    inp = workloads.linear_inputs(1, lin, which=("W",))
    _check(inp.W, inp.W.shape, True, "C1")


def test_quantize_c2_config():
    lin = workloads.CONFIGS[2].linears[0]
    inp = workloads.linear_inputs(2, lin, which=("W",))
    _check(inp.W, inp.W.shape, True, "C2")


@pytest.mark.parametrize("which", [0, 1])
def test_quantize_c3_outliers(which):
    lin = workloads.CONFIGS[3].linears[which]
    inp = workloads.linear_inputs(3, lin, which=("W",))
    _check(inp.W, inp.W.shape, True, f"C3-{lin.name}")


@pytest.mark.parametrize("codebook", ["nf4", "fp4", "int4"])
def test_quantize_exhaustive_bf16_sweep(codebook):
    """Every finite bf16 pattern as a weight, in blocks led by one of several absmax values
    (the encoder's bin table is built per codebook, so every table is swept)."""
    allb = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    vals = (allb.astype(np.uint32) << 16).view(np.float32)
    finite = allb[np.isfinite(vals)]
    fvals = (finite.astype(np.uint32) << 16).view(np.float32)
    blocks = []
    for a in [1.0, 0.02, 0.0390625, 3.0, 1e-3, 448.0, 6.1e-5, 2.0 ** -120]:
        ab = nf4.f32_to_bf16(np.array([a], np.float32))[0]
        af = (np.uint32(ab) << 16).view(np.float32)
        sel = finite[np.abs(fvals) <= af]
        pad = (-sel.size) % 63
        sel = np.concatenate([sel, np.zeros(pad, np.uint16)]).reshape(-1, 63)
        blocks.append(np.concatenate([np.full((sel.shape[0], 1), ab, np.uint16), sel], axis=1))
    w = np.concatenate(blocks).reshape(-1)
    _check(w, (1, w.size), True, "sweep", codebook)
    _check(w, (1, w.size), False, "sweep", codebook)


def test_quantize_degenerate_blocks():
    rng = np.random.default_rng(5)
    parts = [
        np.zeros(64, np.uint16),                                  # all zero
        np.full(64, 0x0001, np.uint16),                           # bf16 subnormals -> flushed zero block
        np.full(64, 0x8080, np.uint16),                           # -2^-126 everywhere
        nf4.f32_to_bf16(np.full(64, 0.03125, np.float32)),        # constant block
        nf4.f32_to_bf16(np.full(64, -0.03125, np.float32)),
        nf4.f32_to_bf16((rng.standard_normal(64 * 300) * 0.02).astype(np.float32)),
    ]
    w = np.concatenate(parts)
    _check(w, (1, w.size), True, "degenerate")
    # every block with the same absmax: mean equals it, all group scales zero
    c = nf4.f32_to_bf16(np.tile(np.array([0.5] + [0.25] * 63, np.float32), 600))
    _check(c, (600, 64), True, "constant-absmax")
    # block constants over a very wide exponent range (exactness of the mean)
    exps = rng.integers(-120, 120, size=5000)
    z = (rng.standard_normal((5000, 64)) * np.exp2(exps)[:, None]).astype(np.float32)
    _check(nf4.f32_to_bf16(z), (5000, 64), True, "wide-range")


def test_quantize_is_deterministic():
    w = workloads.normal_bf16(99, (2048, 2048), 0.02)
    q1, _ = _gpu_quant(w, (2048, 2048), True)
    q2, _ = _gpu_quant(w, (2048, 2048), True)
    for a, b in [(q1.codes, q2.codes), (q1.absmax, q2.absmax), (q1.c1, q2.c1), (q1.mu, q2.mu)]:
        assert torch.equal(a, b)


def _all_code_weight(seed: int, nan_codes: bool):
    """A 256 x 64 weight, one block per row, whose 8-bit block constant is the row index:
    every E4M3 code once (0x7F and 0xFF, the NaN codes, replaced by 0x7E / 0xFE unless
    `nan_codes`), one group scale and the mean chosen by hand, random 4-bit codes."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, size=256 * 64).astype(np.uint8)
    c2 = np.arange(256, dtype=np.uint8)
    if not nan_codes:
        c2[0x7F], c2[0xFF] = 0x7E, 0xFE
    c1 = np.array([1.3125], np.float32)
    mu = np.float32(0.0078125)
    dev = torch.device("cuda", 0)
    w = Q.NF4Weight(256, 64, True, torch.from_numpy(nf4.pack_nibbles(codes, codes.size)).to(dev),
                    torch.from_numpy(c2).to(dev), torch.from_numpy(c1).to(dev),
                    torch.from_numpy(np.array([mu], np.float32)).to(dev))
    return w, codes, c2, c1, mu


def test_dequant_every_fp8_block_code():
    """The block-scale decode over all 256 E4M3 codes: s' = fl32(fl32(dec(c2) c1) + mu) and
    the bf16 weights equal the oracle bit for bit; the two NaN codes give NaN weights."""
    require_gpu()
    w, codes, c2, c1, mu = _all_code_weight(17, nan_codes=True)
    got = host_u16(Q.qlora_dequant(w)).reshape(256, 64)
    torch.cuda.synchronize()
    nan_rows = np.array([0x7F, 0xFF])
    ok = np.setdiff1d(np.arange(256), nan_rows)
    scales = nf4.block_scales_dq(c2[ok], np.repeat(c1, 1), mu)
    want = nf4.dequantize_codes(codes.reshape(256, 64)[ok].reshape(-1), scales).reshape(-1, 64)
    bad = np.flatnonzero(np.any(got[ok] != want, axis=1))
    assert bad.size == 0, f"codes {ok[bad][:8]} decode differently"
    assert np.all((got[nan_rows] & 0x7FFF) > 0x7F80), "NaN codes must dequantize to NaN"


def test_linear_every_fp8_block_code():
    """The same decode inside the linear kernels, exactly: with one-hot token rows and
    B = 0 every output is a single dequantized weight times one, so the large-M forward
    (Y = deq(W)^T), the skinny forward (16 columns of each row) and dX (= deq(W)) must
    reproduce the oracle's bf16 weights for every non-NaN code."""
    require_gpu()
    dev = torch.device("cuda", 0)
    w, codes, c2, c1, mu = _all_code_weight(19, nan_codes=False)
    want = nf4.bf16_to_f32(nf4.dequantize_codes(codes, nf4.block_scales_dq(c2, c1, mu))).reshape(256, 64)
    rng = np.random.default_rng(23)
    A = dev_bf16(nf4.f32_to_bf16((rng.standard_normal(64 * 64) * 0.1).astype(np.float32))).reshape(64, 64)
    B = torch.zeros((64, 256), dtype=torch.bfloat16, device=dev)
    # large-M forward: X = I (64 tokens), Y[m][n] = W[n][m]
    X = torch.eye(64, dtype=torch.bfloat16, device=dev)
    Y, T = Q.qlora_linear_fwd(X, w, A, B, 0.5)
    assert np.array_equal(host(Y.float()), want.T), "large-M forward differs from deq(W)^T"
    # skinny forward: token m picks reduction index 4m
    Xs = torch.zeros((16, 64), dtype=torch.bfloat16, device=dev)
    Xs[torch.arange(16), 4 * torch.arange(16)] = 1
    Ys, _ = Q.qlora_linear_fwd(Xs, w, A, B, 0.5)
    assert np.array_equal(host(Ys.float()), want[:, 4 * np.arange(16)].T), "skinny forward differs"
    # dX: dY = I (256 tokens), dX[m][k] = W[m][k]
    dY = torch.eye(256, dtype=torch.bfloat16, device=dev)
    Xb = torch.zeros((256, 64), dtype=torch.bfloat16, device=dev)
    Tb = torch.zeros((256, 64), dtype=torch.bfloat16, device=dev)
    dX, dA, dB = Q.qlora_linear_bwd(dY, Xb, Tb, w, A, B, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(host(dX.float()), want), "dX differs from deq(W)"
