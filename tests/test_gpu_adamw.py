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


def _hip_runtime():
    """The HIP runtime this process already loaded (the one torch and the library use)."""
    import ctypes
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    assert len(paths) == 1, paths
    return ctypes.CDLL(paths.pop())


def _device_pointer(hip, t):
    """Device address of a pinned host tensor, from hipHostGetDevicePointer (None if the
    runtime does not map it)."""
    import ctypes
    d = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(d), ctypes.c_void_p(t.data_ptr()), ctypes.c_uint(0))
    return d.value if rc == 0 and d.value else None


def test_adamw_state_in_host_memory():
    """Optimizer state paged out to host memory ("Paged optimizers": the state lives in CPU
    RAM and the GPU reaches it when the step runs): fp32 master, m and v in pinned host
    memory, read and written by the kernel through their mapped device addresses, give
    the same bits as the state in device memory."""
    require_gpu()
    import ctypes

    hip = _hip_runtime()
    n = 4096 * 64 + 5
    rng = np.random.default_rng(11)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    dev = torch.device("cuda", 0)
    hp = torch.from_numpy(p0.copy()).pin_memory()
    hm = torch.zeros(n, dtype=torch.float32).pin_memory()
    hv = torch.zeros(n, dtype=torch.float32).pin_memory()
    ptrs = [_device_pointer(hip, t) for t in (hp, hm, hv)]
    if any(x is None for x in ptrs):
        pytest.skip("pinned host memory is not mapped for the device")
    dp = torch.from_numpy(p0.copy()).to(dev)
    dm = torch.zeros(n, dtype=torch.float32, device=dev)
    dv = torch.zeros(n, dtype=torch.float32, device=dev)
    hb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    db = torch.empty(n, dtype=torch.bfloat16, device=dev)
    lib = Q.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for t in range(1, 4):
        g = torch.from_numpy((rng.standard_normal(n) * 1e-3).astype(np.float32)).to(dev)
        rc = lib.qlora_adamw_step(ctypes.c_void_p(ptrs[0]), ctypes.c_void_p(hb.data_ptr()),
                                  ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(ptrs[1]), ctypes.c_void_p(ptrs[2]),
                                  n, t, 2e-4, 0.9, 0.999, 1e-8, 0.01, stream)
        assert rc == 0
        Q.qlora_adamw_step(dp, g, dm, dv, t, 2e-4, 0.9, 0.999, 1e-8, 0.01, param_bf16=db)
        torch.cuda.synchronize()
    for a, b in ((hp, dp), (hm, dm), (hv, dv)):
        assert torch.equal(a, b.cpu())
    assert torch.equal(hb, db)



def test_state_paged_out_and_back_in():
    """The optimizer state stays in device memory; between steps it is paged out to pinned
    host memory, the device copies are overwritten (the memory taken by something else),
    and it is paged back in ("Paged optimizers").  Every later step gives the same bits as
    a run whose state never left the device, and the parameters stay within the oracle's
    bound."""
    require_gpu()
    n = 4096 * 64 + 7
    rng = np.random.default_rng(23)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    dev = torch.device("cuda", 0)
    lr, b1, b2, eps, wd = (float(np.float32(x)) for x in (2e-4, 0.9, 0.999, 1e-8, 0.01))
    state = {k: torch.from_numpy(p0.copy()).to(dev) if k == "p" else torch.zeros(n, device=dev) for k in "pmv"}
    ref = {k: v.clone() for k, v in state.items()}
    pinned = {k: torch.empty(n, dtype=torch.float32).pin_memory() for k in "pmv"}
    rp, rm, rv = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 7):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        gd = torch.from_numpy(g).to(dev)
        if t in (3, 5):
            log("page out / scribble / page in before step", t)
            for k in "pmv":
                Q.qlora_state_page_out(state[k], pinned[k])
            for k in "pmv":
                state[k].fill_(float("nan"))        # the device memory is reused meanwhile
            for k in "pmv":
                Q.qlora_state_page_in(pinned[k], state[k])
        Q.qlora_adamw_step(state["p"], gd, state["m"], state["v"], t, lr, b1, b2, eps, wd)
        Q.qlora_adamw_step(ref["p"], gd, ref["m"], ref["v"], t, lr, b1, b2, eps, wd)
        rp, rm, rv = adamw.adamw_step(rp, g, rm, rv, t, lr, b1, b2, eps, wd)
    torch.cuda.synchronize()
    for k in "pmv":
        assert torch.equal(state[k], ref[k]), k
    gp = host(state["p"]).astype(np.float64)
    assert np.max(np.abs(gp - rp)) <= 8 * 2.0 ** -24 * (np.max(np.abs(rp)) + 7 * lr)


def test_page_calls_refuse_pageable_host_memory():
    require_gpu()
    d = torch.zeros(1024, device="cuda")
    h = torch.zeros(1024)                         # pageable: not pinned
    lib = Q.lib()
    import ctypes
    st = lib.qlora_state_page_out(ctypes.c_void_p(d.data_ptr()), ctypes.c_void_p(h.data_ptr()), 4096, None)
    assert st == 4                                # QLORA_ERR_UNSUPPORTED
    st = lib.qlora_state_page_in(ctypes.c_void_p(h.data_ptr()), ctypes.c_void_p(d.data_ptr()), 4096, None)
    assert st == 4
