"""Pins for the QLoRA linear oracle (forward / backward in float64), no GPU."""
import numpy as np
import pytest
import torch

import workloads
from oracle import linear, nf4


def _case(M=16, d_in=256, d_out=256, r=8, seed=1):
    inp = workloads.custom_linear(M, d_in, d_out, r, seed)
    q = nf4.quantize(inp.W, double_quant=True)
    Wd = nf4.dequantize(q, (d_out, d_in))
    return inp, Wd


def _t64(u16):
    return torch.from_numpy(nf4.bf16_to_f32(u16).astype(np.float64))


@pytest.mark.parametrize("s", [2.0, 0.25, 1.0, 0.3])
def test_backward_matches_autograd(s):
    """Gradients of L = <Y, dY> through an fp64 autograd graph of the forward definition."""
    inp, Wd = _case(M=12, d_in=128, d_out=192, r=8, seed=4)
    X = _t64(inp.X).requires_grad_(True)
    A = _t64(inp.A).requires_grad_(True)
    B = _t64(inp.B).requires_grad_(True)
    W = _t64(Wd).requires_grad_(True)
    Y = X @ W.T + s * (X @ A) @ B
    dY = _t64(inp.dY)
    (Y * dY).sum().backward()
    dx, da, db = linear.backward(inp.dY, inp.X, Wd, inp.A, inp.B, s)
    y, _ = linear.forward(inp.X, Wd, inp.A, inp.B, s)
    np.testing.assert_allclose(y, Y.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx, X.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(da, A.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db, B.grad.numpy(), rtol=1e-11, atol=1e-11)
    # the adapter-only gradients used by the sampled full-size checks, and the slicing
    # they rely on: Y's columns come from the weight's rows (and B's columns), dX's
    # columns from the weight's columns (and A's rows)
    da2, db2 = linear.adapter_grads(inp.dY, inp.X, inp.A, inp.B, s)
    np.testing.assert_allclose(da2, A.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db2, B.grad.numpy(), rtol=1e-11, atol=1e-11)
    cols = np.array([0, 5, 77, 191])
    yc, _ = linear.forward(inp.X, Wd[cols], inp.A, inp.B[:, cols], s)
    np.testing.assert_allclose(yc, Y.detach().numpy()[:, cols], rtol=1e-12, atol=1e-12)
    kc = np.array([1, 64, 127])
    rows = np.arange(12)
    dxc = linear.backward_dx_rows(inp.dY, Wd[:, kc], inp.A[kc], inp.B, s, rows)
    np.testing.assert_allclose(dxc, X.grad.numpy()[:, kc], rtol=1e-11, atol=1e-11)


def test_frozen_weight_gets_no_gradient_and_dX_passes_through_W():
    inp, Wd = _case(seed=5)
    dx_full, _, _ = linear.backward(inp.dY, inp.X, Wd, inp.A, inp.B, 2.0)
    zero_B = np.zeros_like(inp.B)
    dx_base, da, db = linear.backward(inp.dY, inp.X, Wd, inp.A, zero_B, 2.0)
    # with L2 = 0 the adapter path carries no gradient into X or L1
    assert np.all(da == 0)
    np.testing.assert_allclose(dx_base, nf4.bf16_to_f32(inp.dY).astype(np.float64) @ nf4.bf16_to_f32(Wd).astype(np.float64).reshape(256, 256), rtol=1e-12)
    assert not np.allclose(dx_full, dx_base)


def test_finite_differences_c1():
    """Central differences of L(X, A, B) = <Y, dY> on the 256->256 r=8 shape."""
    inp, Wd = _case(seed=6)
    s = 2.0
    x = nf4.bf16_to_f32(inp.X).astype(np.float64)
    a = nf4.bf16_to_f32(inp.A).astype(np.float64)
    b = nf4.bf16_to_f32(inp.B).astype(np.float64)
    w = nf4.bf16_to_f32(Wd).astype(np.float64).reshape(256, 256)
    dy = nf4.bf16_to_f32(inp.dY).astype(np.float64)

    def loss(x, a, b):
        return float(np.sum((x @ w.T + s * (x @ a) @ b) * dy))

    dx, da, db = linear.backward(inp.dY, inp.X, Wd, inp.A, inp.B, s)
    rng = np.random.default_rng(0)
    h = 1e-4
    for _ in range(8):
        i, j = rng.integers(0, 16), rng.integers(0, 256)
        e = np.zeros_like(x); e[i, j] = h
        assert (loss(x + e, a, b) - loss(x - e, a, b)) / (2 * h) == pytest.approx(dx[i, j], rel=1e-6, abs=1e-8)
        i, j = rng.integers(0, 256), rng.integers(0, 8)
        e = np.zeros_like(a); e[i, j] = h
        assert (loss(x, a + e, b) - loss(x, a - e, b)) / (2 * h) == pytest.approx(da[i, j], rel=1e-6, abs=1e-8)
        i, j = rng.integers(0, 8), rng.integers(0, 256)
        e = np.zeros_like(b); e[i, j] = h
        assert (loss(x, a, b + e) - loss(x, a, b - e)) / (2 * h) == pytest.approx(db[i, j], rel=1e-6, abs=1e-8)


def test_special_cases():
    inp, Wd = _case(seed=7)
    x = nf4.bf16_to_f32(inp.X).astype(np.float64)
    a = nf4.bf16_to_f32(inp.A).astype(np.float64)
    b = nf4.bf16_to_f32(inp.B).astype(np.float64)
    w = nf4.bf16_to_f32(Wd).astype(np.float64).reshape(256, 256)
    # B = 0: plain product with the dequantized weight
    y0, _ = linear.forward(inp.X, Wd, inp.A, np.zeros_like(inp.B), 2.0)
    np.testing.assert_allclose(y0, torch.from_numpy(x) @ torch.from_numpy(w).T, rtol=1e-12)
    # all-zero weight -> all codes are the exact zero -> the adapter alone
    q0 = nf4.quantize(np.zeros((256, 256), np.uint16))
    assert np.all(nf4.unpack_nibbles(q0["codes"], 65536) == 7)
    Wz = nf4.dequantize(q0, (256, 256))
    yz, _ = linear.forward(inp.X, Wz, inp.A, inp.B, 2.0)
    np.testing.assert_allclose(yz, 2.0 * (x @ a) @ b, rtol=1e-12)
    # A = 0 -> dB = 0
    _, _, db = linear.backward(inp.dY, inp.X, Wd, np.zeros_like(inp.A), inp.B, 2.0)
    assert np.all(db == 0)


def test_review_page_gradients_with_unit_scale():
    """With s = 1 the oracle's dA, dB equal the two products stated on the review page."""
    inp, Wd = _case(seed=8)
    x = nf4.bf16_to_f32(inp.X).astype(np.float64)
    a = nf4.bf16_to_f32(inp.A).astype(np.float64)
    b = nf4.bf16_to_f32(inp.B).astype(np.float64)
    dy = nf4.bf16_to_f32(inp.dY).astype(np.float64)
    _, da, db = linear.backward(inp.dY, inp.X, Wd, inp.A, inp.B, 1.0)
    np.testing.assert_allclose(db, a.T @ x.T @ dy, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(da, x.T @ dy @ b.T, rtol=1e-12, atol=1e-12)


def test_flop_counts():
    assert linear.flops_fwd_bwd(2048, 4096, 4096, 64) == 143_881_404_416
    assert linear.flops_fwd(1, 8192, 22016, 64) == 2 * 8192 * 22016 + 2 * 64 * (8192 + 22016)


def test_merged_weight_reproduces_the_layer():
    """X merged^T equals the layer's forward in exact arithmetic (the adapter term folds
    into the weight by distributivity); B = 0 leaves the dequantized weight unchanged."""
    inp, Wd = _case(M=12, d_in=128, d_out=64, r=8, seed=9)
    s = 2.0
    Wm = linear.merge_adapter(Wd, inp.A, inp.B, s)
    y, _ = linear.forward(inp.X, Wd, inp.A, inp.B, s)
    x = nf4.bf16_to_f32(inp.X).astype(np.float64)
    np.testing.assert_allclose(x @ Wm.T, y, rtol=1e-12, atol=1e-12)
    W0 = linear.merge_adapter(Wd, inp.A, np.zeros_like(inp.B), s)
    np.testing.assert_array_equal(W0, nf4.bf16_to_f32(Wd).astype(np.float64).reshape(64, 128))
