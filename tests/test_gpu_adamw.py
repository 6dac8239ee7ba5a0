"""GPU parity of the AdamW step on adapter parameters against the float64 oracle: fp32
parameters and state within a few fp32 roundings of the oracle after several steps, and
the bf16 working copy equal to bf16(parameter) bit for bit."""
import numpy as np
import pytest
import torch

import bit_nf4_quantized_11_amd as Q
from helpers import host, host_u16, log, require_gpu
from oracle import adamw, nf4

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,wd", [(64 * 4096 + 3, 0.0), (4096 * 64, 0.01), (5, 0.1), (1, 0.0)])
def test_adamw_steps_match_oracle(n, wd):
    require_gpu()
    log("adamw", n, wd)
    rng = np.random.default_rng(n)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    # the call takes its hyperparameters as fp32; the oracle gets those same values
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (2e-4, 0.9, 0.999, 1e-8, wd))
    dev = torch.device("cuda", 0)
    p = torch.from_numpy(p0.copy()).to(dev)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    rp, rm, rv = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -1)).astype(np.float32)
        Q.qlora_adamw_step(p, torch.from_numpy(g).to(dev), m, v, t, lr, b1, b2, eps, wd, param_bf16=pb)
        rp, rm, rv = adamw.adamw_step(rp, g, rm, rv, t, lr, b1, b2, eps, wd)
    torch.cuda.synchronize()
    gp, gm, gv = host(p).astype(np.float64), host(m).astype(np.float64), host(v).astype(np.float64)
    # each step rounds a handful of fp32 operations; the update is at most ~lr per step
    assert np.max(np.abs(gp - rp)) <= 8 * 2.0 ** -24 * (np.max(np.abs(rp)) + 5 * lr)
    # m is a sum of signed gradients (it can cancel): its error is bounded against its
    # largest magnitude; v is a sum of squares and keeps an element-wise bound
    assert np.max(np.abs(gm - rm)) <= 1e-6 * np.max(np.abs(rm))
    assert np.max(np.abs(gv - rv) / (np.abs(rv) + 1e-30)) <= 1e-5
    np.testing.assert_array_equal(host_u16(pb), nf4.f32_to_bf16(host(p)))
