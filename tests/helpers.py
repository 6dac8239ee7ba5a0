"""Shared helpers for the GPU parity tests (host <-> device marshalling, tolerances)."""
import sys
import time

import numpy as np
import torch

# Floating-point outputs: per element |out - ref| <= 1e-2 max|ref| and relative
# Frobenius error <= 5e-3, against the float64 oracle on identical bf16 inputs and
# the bit-exact dequantized weight.
TOL_MAX = 1e-2
TOL_FRO = 5e-3


def log(*a):
    print(time.strftime("%H:%M:%S"), *a, file=sys.stderr, flush=True)


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(u16) -> np.ndarray:
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_errors(out: np.ndarray, ref: np.ndarray):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    d = out - ref
    mref = np.abs(ref).max()
    nref = np.linalg.norm(ref)
    return (np.abs(d).max() / mref if mref > 0 else np.abs(d).max(),
            np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d))


def assert_close(out, ref, name):
    e_max, e_fro = rel_errors(out, ref)
    assert np.all(np.isfinite(out)), f"{name}: non-finite output"
    assert e_max <= TOL_MAX and e_fro <= TOL_FRO, f"{name}: max-rel {e_max:.3e} fro-rel {e_fro:.3e}"
    return e_max, e_fro


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a GPU")
