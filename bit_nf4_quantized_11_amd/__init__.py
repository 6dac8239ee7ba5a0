"""Python binding of libqlora (QLoRA linear layer on MI355X / gfx950).

Thin argument marshalling over the C ABI in include/qlora.h: each function has
the name of the C entry point it calls.  torch is used for device memory and
streams only; every computation runs in the library's HIP kernels.  There is no
CPU fallback: without the built library or a GPU the calls raise.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib

__all__ = [
    "NF4Weight", "QLoRAError", "nf4_alloc", "qlora_nf4_codebook", "qlora_codebook_table", "qlora_nf4_sizes",
    "CODEBOOK_NF4", "CODEBOOK_FP4", "CODEBOOK_INT4", "CODEBOOKS", "qlora_quantize_workspace",
    "qlora_fwd_workspace", "qlora_bwd_workspace", "qlora_quantize_nf4", "qlora_dequant", "qlora_linear_fwd",
    "qlora_linear_bwd", "qlora_merge_adapter", "qlora_adamw_step", "qlora_profile_enable", "qlora_profile_read", "lib",
]


class QLoRAError(RuntimeError):
    pass


# qlora_codebook values: the 16-entry table a quantized weight's codes index
CODEBOOK_NF4, CODEBOOK_FP4, CODEBOOK_INT4 = 0, 1, 2
CODEBOOKS = {"nf4": CODEBOOK_NF4, "fp4": CODEBOOK_FP4, "int4": CODEBOOK_INT4}


def lib():
    return _lib.load()


def _check(status: int, what: str):
    if status != 0:
        msg = lib().qlora_status_str(status).decode()
        raise QLoRAError(f"{what}: {_lib.STATUS.get(status, status)} ({msg})")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _bf16(t, name):
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise QLoRAError(f"{name} must be a contiguous bf16 tensor on the GPU")
    return t


@dataclass
class NF4Weight:
    """A quantized [rows][cols] weight: caller-owned device buffers (torch tensors)."""
    rows: int
    cols: int
    double_quant: bool
    codes: torch.Tensor      # uint8 [32 per 64 weights, padded to whole blocks]
    absmax: torch.Tensor     # uint8 [nblk] (double quant) or float32 [nblk]
    c1: torch.Tensor | None  # float32 [nsup]
    mu: torch.Tensor | None  # float32 [1]
    codebook: int = CODEBOOK_NF4
    block: int = 64          # weights per constant: 32, 64, 128 or 256

    def desc(self) -> _lib.qlora_nf4:
        return _lib.qlora_nf4(self.rows, self.cols, int(self.double_quant), int(self.codebook), int(self.block), 0,
                              self.codes.data_ptr(), self.absmax.data_ptr(),
                              self.c1.data_ptr() if self.c1 is not None else None,
                              self.mu.data_ptr() if self.mu is not None else None)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.absmax, self.c1, self.mu) if t is not None)


def qlora_nf4_codebook():
    """(levels[16], thresholds[15]) as Python floats, computed by the library."""
    lv = (C.c_float * 16)()
    th = (C.c_float * 15)()
    _check(lib().qlora_nf4_codebook(lv, th), "qlora_nf4_codebook")
    return list(lv), list(th)


def qlora_codebook_table(codebook: int = CODEBOOK_NF4):
    """(levels[16], thresholds[15]) of any codebook, computed by the library."""
    lv = (C.c_float * 16)()
    th = (C.c_float * 15)()
    _check(lib().qlora_codebook_table(int(codebook), lv, th), "qlora_codebook_table")
    return list(lv), list(th)


def qlora_nf4_sizes(rows: int, cols: int, double_quant: bool = True, block: int = 64):
    out = [C.c_size_t() for _ in range(4)]
    _check(lib().qlora_nf4_sizes(rows, cols, int(double_quant), int(block), *[C.byref(o) for o in out]),
           "qlora_nf4_sizes")
    return tuple(o.value for o in out)


def qlora_quantize_workspace(rows: int, cols: int, double_quant: bool = True, block: int = 64) -> int:
    return lib().qlora_quantize_workspace(rows, cols, int(double_quant), int(block))


def qlora_fwd_workspace(M: int, d_in: int, d_out: int, r: int) -> int:
    return lib().qlora_fwd_workspace(M, d_in, d_out, r)


def qlora_bwd_workspace(M: int, d_in: int, d_out: int, r: int) -> int:
    return lib().qlora_bwd_workspace(M, d_in, d_out, r)


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def nf4_alloc(rows: int, cols: int, double_quant: bool = True, device="cuda", codebook: int = CODEBOOK_NF4,
              block: int = 64) -> NF4Weight:
    cb, ab, c1b, mub = qlora_nf4_sizes(rows, cols, double_quant, block)
    codes = torch.empty(cb, dtype=torch.uint8, device=device)
    if double_quant:
        absmax = torch.empty(ab, dtype=torch.uint8, device=device)
        c1 = torch.empty(c1b // 4, dtype=torch.float32, device=device)
        mu = torch.empty(1, dtype=torch.float32, device=device)
    else:
        absmax = torch.empty(ab // 4, dtype=torch.float32, device=device)
        c1 = mu = None
    return NF4Weight(rows, cols, double_quant, codes, absmax, c1, mu, codebook, block)


def qlora_quantize_nf4(W: torch.Tensor, double_quant: bool = True, out: NF4Weight | None = None,
                       workspace: torch.Tensor | None = None, stream=None, codebook: int = CODEBOOK_NF4,
                       block: int = 64) -> NF4Weight:
    """Quantize a bf16 [rows][cols] weight (any 2-D shape) to 4-bit codes of `codebook`
    (NF4 by default) with one absmax per `block` weights (+ double quantization).  With
    `out` given, its own codebook and block size are used."""
    _bf16(W, "W")
    rows, cols = (W.shape[0], W.shape[1]) if W.dim() == 2 else (1, W.numel())
    if out is None:
        out = nf4_alloc(rows, cols, double_quant, W.device, codebook, block)
    ws = _workspace(qlora_quantize_workspace(rows, cols, out.double_quant, out.block), W.device, workspace)
    d = out.desc()
    _check(lib().qlora_quantize_nf4(_ptr(W), rows, cols, C.byref(d), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(stream)), "qlora_quantize_nf4")
    return out


def qlora_dequant(w: NF4Weight, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=w.codes.device)
    d = w.desc()
    _check(lib().qlora_dequant(C.byref(d), _ptr(out), _stream(stream)), "qlora_dequant")
    return out


def qlora_linear_fwd(X: torch.Tensor, w: NF4Weight, A: torch.Tensor, B: torch.Tensor, scale: float,
                     Y: torch.Tensor | None = None, save_T: bool = True, T_save: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None):
    """Y = X deq(W)^T + scale (X A) B.  Returns (Y, T) with T = bf16(X A) or None."""
    _bf16(X, "X"); _bf16(A, "A"); _bf16(B, "B")
    M = X.shape[0]
    r = A.shape[1]
    if Y is None:
        Y = torch.empty((M, w.rows), dtype=torch.bfloat16, device=X.device)
    if save_T and T_save is None:
        T_save = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    ws = _workspace(qlora_fwd_workspace(M, w.cols, w.rows, r), X.device, workspace)
    d = w.desc()
    _check(lib().qlora_linear_fwd(_ptr(X), M, C.byref(d), _ptr(A), _ptr(B), r, float(scale), _ptr(Y),
                                  _ptr(T_save if save_T else None), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream)), "qlora_linear_fwd")
    return Y, (T_save if save_T else None)


def qlora_linear_fwd_noalloc(X: torch.Tensor, w: NF4Weight, A: torch.Tensor, B: torch.Tensor, scale: float,
                             Y: torch.Tensor, T_save: torch.Tensor | None = None, stream=None):
    """The forward with the library's own scratch array (no workspace, nothing allocated);
    Y (and T_save, if given) must be allocated by the caller.  Returns (Y, T_save)."""
    _bf16(X, "X"); _bf16(A, "A"); _bf16(B, "B")
    d = w.desc()
    _check(lib().qlora_linear_fwd_noalloc(_ptr(X), X.shape[0], C.byref(d), _ptr(A), _ptr(B), A.shape[1],
                                          float(scale), _ptr(Y), _ptr(T_save), _stream(stream)),
           "qlora_linear_fwd_noalloc")
    return Y, T_save


def qlora_linear_bwd(dY: torch.Tensor, X: torch.Tensor, T_saved: torch.Tensor | None, w: NF4Weight,
                     A: torch.Tensor, B: torch.Tensor, scale: float, need_dX: bool = True,
                     dX: torch.Tensor | None = None, dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None):
    """Returns (dX or None, dA fp32 [in][r], dB fp32 [r][out]); no gradient for W."""
    _bf16(dY, "dY"); _bf16(X, "X"); _bf16(A, "A"); _bf16(B, "B")
    M = X.shape[0]
    r = A.shape[1]
    dev = X.device
    if need_dX and dX is None:
        dX = torch.empty((M, w.cols), dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty((w.cols, r), dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty((r, w.rows), dtype=torch.float32, device=dev)
    ws = _workspace(qlora_bwd_workspace(M, w.cols, w.rows, r), dev, workspace)
    d = w.desc()
    _check(lib().qlora_linear_bwd(_ptr(dY), _ptr(X), _ptr(T_saved), M, C.byref(d), _ptr(A), _ptr(B), r,
                                  float(scale), _ptr(dX if need_dX else None), _ptr(dA), _ptr(dB), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)), "qlora_linear_bwd")
    return (dX if need_dX else None), dA, dB


def qlora_merge_adapter(w: NF4Weight, A: torch.Tensor, B: torch.Tensor, scale: float,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """bf16 [rows][cols] weight deq(W) + scale (A B)^T (requantize it with qlora_quantize_nf4)."""
    _bf16(A, "A"); _bf16(B, "B")
    if out is None:
        out = torch.empty((w.rows, w.cols), dtype=torch.bfloat16, device=A.device)
    d = w.desc()
    _check(lib().qlora_merge_adapter(C.byref(d), _ptr(A), _ptr(B), A.shape[1], float(scale), _ptr(out),
                                     _stream(stream)), "qlora_merge_adapter")
    return out


def qlora_adamw_step(param: torch.Tensor, grad: torch.Tensor, m: torch.Tensor, v: torch.Tensor, step: int,
                     lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                     weight_decay: float = 0.0, param_bf16: torch.Tensor | None = None, stream=None):
    """One AdamW step in place on fp32 `param`, `m`, `v` (same number of elements as the
    fp32 `grad`); writes bf16(param) into `param_bf16` when given."""
    n = param.numel()
    for t, name in ((param, "param"), (grad, "grad"), (m, "m"), (v, "v")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise QLoRAError(f"{name} must be a contiguous float32 tensor of {n} elements")
    if param_bf16 is not None and (param_bf16.dtype != torch.bfloat16 or param_bf16.numel() != n
                                   or not param_bf16.is_contiguous()):
        raise QLoRAError("param_bf16 must be a contiguous bf16 tensor of the same size")
    _check(lib().qlora_adamw_step(_ptr(param), _ptr(param_bf16), _ptr(grad), _ptr(m), _ptr(v), n, int(step),
                                  float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                                  _stream(stream)), "qlora_adamw_step")


def _page_args(dev: torch.Tensor, host: torch.Tensor):
    if not dev.is_cuda or host.is_cuda or not host.is_pinned():
        raise QLoRAError("paging copies between a device tensor and a pinned host tensor")
    if not dev.is_contiguous() or not host.is_contiguous() or dev.nbytes != host.nbytes:
        raise QLoRAError("paging needs two contiguous tensors of the same size")


def qlora_state_page_out(dev: torch.Tensor, host: torch.Tensor, stream=None) -> torch.Tensor:
    """Copy optimizer state from device memory into a pinned host tensor (asynchronous on the
    stream).  Returns `host`."""
    _page_args(dev, host)
    _check(lib().qlora_state_page_out(_ptr(dev), _ptr(host), dev.nbytes, _stream(stream)), "qlora_state_page_out")
    return host


def qlora_state_page_in(host: torch.Tensor, dev: torch.Tensor, stream=None) -> torch.Tensor:
    """Copy optimizer state from a pinned host tensor back into device memory (asynchronous
    on the stream).  Returns `dev`."""
    _page_args(dev, host)
    _check(lib().qlora_state_page_in(_ptr(host), _ptr(dev), dev.nbytes, _stream(stream)), "qlora_state_page_in")
    return dev


def qlora_profile_enable(enable: bool = True):
    _check(lib().qlora_profile_enable(int(enable)), "qlora_profile_enable")


def qlora_profile_read(reset: bool = True) -> dict:
    """{kernel name: (launches, total_ms)} since the last reset (synchronizes the recorded events)."""
    buf = (_lib.qlora_kernel_time * 64)()
    n = lib().qlora_profile_read(buf, 64, int(reset))
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n)}
