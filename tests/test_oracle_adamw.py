"""Pins for the AdamW oracle (float64), no GPU: torch.optim.AdamW (a library routine) over
several steps, the first-step closed form, and the zero-gradient case."""
import numpy as np
import pytest
import torch

from oracle import adamw


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_matches_torch_adamw(wd):
    rng = np.random.default_rng(1)
    p0 = rng.standard_normal(1000) * 0.02
    grads = [rng.standard_normal(1000) * 10.0 ** rng.uniform(-4, 0) for _ in range(6)]
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=wd)
    p, m, v = p0.copy(), np.zeros(1000), np.zeros(1000)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = adamw.adamw_step(p, g, m, v, t, 2e-4, 0.9, 0.999, 1e-8, wd)
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-16)
    # torch forms the first moment as a lerp, m + (1 - b1)(g - m): the same value, rounded
    # in a different order, so elements where m nearly cancels agree to ~1e-12 only
    st = opt.state[tp]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-11, atol=1e-20)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-11, atol=1e-24)


def test_first_step_is_a_signed_lr_step():
    """At t = 1 the bias corrections cancel: the step is lr * g / (|g| + eps)."""
    g = np.array([3.0, -2.0, 1e-3, -5e-2])
    p, _, _ = adamw.adamw_step(np.zeros(4), g, np.zeros(4), np.zeros(4), 1, 1e-3, eps=1e-8)
    np.testing.assert_allclose(p, -1e-3 * g / (np.abs(g) + 1e-8), rtol=1e-12)


def test_zero_gradient_without_decay_keeps_parameters():
    p0 = np.linspace(-1, 1, 9)
    p, m, v = adamw.adamw_step(p0, np.zeros(9), np.zeros(9), np.zeros(9), 3, 1e-2)
    np.testing.assert_array_equal(p, p0)
    assert np.all(m == 0) and np.all(v == 0)
