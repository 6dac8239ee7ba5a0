"""Oracle: forward and backward of the QLoRA linear layer, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions ([Explainer] "The QLoRA layer, end to end", the one-layer code
listing; [Explainer] "LoRA: freeze the base, train a patch" for s = alpha/r;
[Review] "The Gradient Flow Trick" states the same gradients with s = 1):

    forward:   Y  = X W + s (X L1) L2
    backward:  dX = dY W^T + s (dY L2^T) L1^T
               dL1 = s X^T (dY L2^T)
               dL2 = s (X L1)^T dY
    and no gradient for the frozen W.

Here W is the page's [in][out] matrix.  The stored weight is the [out][in]
row-major matrix Wq (the layout of a torch Linear weight), so the page's W is
Wq^T and the dequantized weight enters as X Wq^T.  L1 = A [in][r], L2 = B [r][out].

All inputs are bf16 bit patterns; every product runs in float64 on the exact
bf16 values with no intermediate rounding.
"""
from __future__ import annotations

import numpy as np


def _f64(u16) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def forward(X, Wq, A, B, s: float):
    """Returns (Y [M][out], T = X A [M][r]) in float64.

    The layer output is the frozen product plus the scaled rank-r path; T is the
    rank-r activation, returned because the backward needs it."""
    x, w, a, b = _f64(X), _f64(Wq), _f64(A), _f64(B)
    t = x @ a
    base = x @ w.T
    return base + s * (t @ b), t


def backward(dY, X, Wq, A, B, s: float):
    """Returns (dX [M][in], dA [in][r], dB [r][out]) in float64.

    Chain rule on L = <Y, dY> with Y = X Wq^T + s (X A) B:
      - Y depends on X through Wq^T and through A then B, so dL/dX is dY Wq plus
        s (dY B^T) A^T;
      - Y depends on A only through the product X A, whose gradient is s dY B^T,
        so dL/dA = X^T (s dY B^T);
      - Y depends on B through (X A) B, so dL/dB = s (X A)^T dY;
      - the frozen Wq gets no gradient."""
    dy, x, w, a, b = _f64(dY), _f64(X), _f64(Wq), _f64(A), _f64(B)
    up = dy @ b.T                           # gradient reaching the rank-r activation, before s
    grad_x = dy @ w + s * (up @ a.T)
    grad_a = s * (x.T @ up)
    grad_b = s * ((x @ a).T @ dy)
    return grad_x, grad_a, grad_b


def forward_rows(X, Wq, A, B, s: float, rows):
    """Y for selected token rows only (sampled checks at full size)."""
    rows = np.asarray(rows)
    return forward(np.asarray(X)[rows], Wq, A, B, s)[0]


def backward_dx_rows(dY, Wq, A, B, s: float, rows):
    """dX for selected token rows only (sampled checks at full size)."""
    rows = np.asarray(rows)
    dy, w, a, b = _f64(np.asarray(dY)[rows]), _f64(Wq), _f64(A), _f64(B)
    return dy @ w + s * ((dy @ b.T) @ a.T)


def adapter_grads(dY, X, A, B, s: float):
    """(dA [in][r], dB [r][out]) in float64: the backward's adapter gradients alone,
    for full-size checks where the frozen-weight term of dX is sampled separately."""
    dy, x, a, b = _f64(dY), _f64(X), _f64(A), _f64(B)
    g = dy @ b.T
    return s * (x.T @ g), s * ((x @ a).T @ dy)


def flops_fwd(M, d_in, d_out, r) -> int:
    return 2 * M * d_in * d_out + 2 * M * r * (d_in + d_out)


def flops_fwd_bwd(M, d_in, d_out, r) -> int:
    """fwd (2 M in out + 2 M r (in+out)) + bwd without dW (2 M in out + 4 M r (in+out))."""
    return 4 * M * d_in * d_out + 6 * M * r * (d_in + d_out)


def merge_adapter(Wq, A, B, s: float):
    """The merged weight deq(W) + s (A B)^T [out][in] in float64 with no rounding
    ("QLoRA: quantising the part you are not training", section "What it costs": merging
    the adapter into the base).  Wq is the bf16 dequantized weight [out][in]."""
    return _f64(Wq) + s * (_f64(A) @ _f64(B)).T
