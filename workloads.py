"""Seeded synthetic inputs for the QLoRA linear layer, shared by the tests, the
benchmark and the oracle checks.

This module draws random numbers and rounds them once to bfloat16; it holds none
of the method's arithmetic (no quantization, no dequantization, no products).

The inputs stand in for the pages' workloads, which finetune LLaMA 7B..65B on a
chat dataset (QLoRA explainer page, "Guanaco and its benchmarks"); trained
weights and datasets are not available, so the weights are Gaussian at LLaMA
layer shapes, following the premise that pretrained weights are roughly
N(0, sigma^2) (QLoRA explainer page, "NormalFloat: 4 bits for a bell curve").

Recipe (one rounding from fp32 to bf16, round-to-nearest-even, via torch):
  * W  ~ N(0, 0.02^2); for the outlier configuration a Bernoulli(0.001) mask
    scales the selected fp32 entries by 20 before the rounding;
  * A, B (LoRA factors) ~ N(0, 0.02^2), B nonzero;
  * X, dY ~ N(0, 1).
Seeds: seed = 1000*config + 10*layer + tensor_id with tensor ids
W=0, A=1, B=2, X=3, dY=4, outlier mask=5.  Host tensors use NumPy's PCG64;
the 65B layer stack is drawn on the device with torch's Philox generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TID_W, TID_A, TID_B, TID_X, TID_DY, TID_MASK = 0, 1, 2, 3, 4, 5


def seed_for(cfg: int, layer: int, tensor_id: int) -> int:
    return 1000 * cfg + 10 * layer + tensor_id


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bfloat16 (RNE, via torch) and return the uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(seed: int, shape, std: float = 1.0, outlier_p: float = 0.0,
                outlier_scale: float = 20.0, mask_seed: int | None = None) -> np.ndarray:
    """N(0, std^2) drawn in fp32 with PCG64(seed), optional outliers, rounded once to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    if outlier_p > 0.0:
        mrng = np.random.Generator(np.random.PCG64(mask_seed if mask_seed is not None else seed + 5))
        mask = mrng.random(size=shape, dtype=np.float32) < np.float32(outlier_p)
        x[mask] *= np.float32(outlier_scale)
    return _to_bf16_bits(x)


@dataclass(frozen=True)
class Linear:
    name: str
    M: int
    d_in: int
    d_out: int
    r: int
    alpha: float
    outlier_p: float = 0.0

    @property
    def scale(self) -> float:
        return self.alpha / self.r


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    linears: tuple
    backward: bool = True
    layers: int = 1
    note: str = ""
    extra: dict = field(default_factory=dict)


# The five configurations (shapes of LLaMA-7B and LLaMA-65B layers).
CONFIGS = {
    1: Config(1, "single linear 256->256, M=16, r=8", (Linear("lin", 16, 256, 256, 8, 16.0),)),
    2: Config(2, "7B attention projection 4096->4096, M=2048, r=64",
              (Linear("proj", 2048, 4096, 4096, 64, 16.0),)),
    3: Config(3, "7B MLP 4096->11008 and 11008->4096 with 0.1% x20 outliers, M=4096, r=64",
              (Linear("gate_up", 4096, 4096, 11008, 64, 16.0, 0.001),
               Linear("down", 4096, 11008, 4096, 64, 16.0, 0.001))),
    4: Config(4, "65B decode-like skinny M in {1,4,16}, 8192->22016 and 22016->8192, forward only",
              tuple(Linear(f"{nm}_M{m}", m, di, do, 64, 16.0)
                    for m in (1, 4, 16)
                    for nm, di, do in (("up", 8192, 22016), ("down", 22016, 8192))),
              backward=False),
    5: Config(5, "65B layer stack: 80 layers x (q,k,v,o 8192->8192; gate,up 8192->22016; down 22016->8192), M=2048, r=64",
              (Linear("q", 2048, 8192, 8192, 64, 16.0), Linear("k", 2048, 8192, 8192, 64, 16.0),
               Linear("v", 2048, 8192, 8192, 64, 16.0), Linear("o", 2048, 8192, 8192, 64, 16.0),
               Linear("gate", 2048, 8192, 22016, 64, 16.0), Linear("up", 2048, 8192, 22016, 64, 16.0),
               Linear("down", 2048, 22016, 8192, 64, 16.0)),
              layers=80),
}


@dataclass
class LinearInputs:
    """Host bf16 bit patterns for one linear: W [out][in], A [in][r], B [r][out], X [M][in], dY [M][out]."""
    W: np.ndarray
    A: np.ndarray
    B: np.ndarray
    X: np.ndarray
    dY: np.ndarray
    spec: Linear


def linear_inputs(cfg: int, lin: Linear, layer: int = 0, which=("W", "A", "B", "X", "dY")) -> LinearInputs:
    """Host inputs for one linear of a configuration (NumPy PCG64, rounded once to bf16)."""
    s = lambda tid: seed_for(cfg, layer, tid)
    out = {}
    if "W" in which:
        out["W"] = normal_bf16(s(TID_W), (lin.d_out, lin.d_in), 0.02, outlier_p=lin.outlier_p,
                               mask_seed=s(TID_MASK))
    if "A" in which:
        out["A"] = normal_bf16(s(TID_A), (lin.d_in, lin.r), 0.02)
    if "B" in which:
        out["B"] = normal_bf16(s(TID_B), (lin.r, lin.d_out), 0.02)
    if "X" in which:
        out["X"] = normal_bf16(s(TID_X), (lin.M, lin.d_in), 1.0)
    if "dY" in which:
        out["dY"] = normal_bf16(s(TID_DY), (lin.M, lin.d_out), 1.0)
    return LinearInputs(out.get("W"), out.get("A"), out.get("B"), out.get("X"), out.get("dY"), lin)


def device_normal_bf16(seed: int, shape, std: float, device="cuda", outlier_p: float = 0.0,
                       outlier_scale: float = 20.0, mask_seed: int | None = None):
    """N(0, std^2) drawn on the device with torch's Philox generator, optional outliers
    (a Bernoulli(outlier_p) mask scales the fp32 entries), rounded once to bf16."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    if outlier_p > 0.0:
        g.manual_seed(mask_seed if mask_seed is not None else seed + 5)
        mask = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < outlier_p
        x[mask] *= outlier_scale
        del mask
    return x.to(torch.bfloat16)


# The 65B layer stack (configuration 5).  Every linear of every layer has its own
# weight, adapter factors and output gradient.  There is no attention or MLP
# nonlinearity on the path, so the token inputs follow the layer's wiring only: q, k,
# v, gate and up read one shared [M][8192] input (drawn with slot 0's seed), o reads
# its own [M][8192] input (slot 3) and down its own [M][22016] input (slot 6).
# Seeds: seed_for(5, 7*layer + slot, tensor_id), i.e. each linear of the stack counts
# as one "layer" of the general seed rule.
STACK_INPUT_SLOT = (0, 0, 0, 3, 0, 0, 6)


def stack_seed(layer: int, slot: int, tensor_id: int) -> int:
    return seed_for(5, 7 * layer + slot, tensor_id)


def stack_tensor(layer: int, slot: int, what: str, device="cuda"):
    """One device tensor of the 65B stack: "W" [out][in], "A" [in][r], "B" [r][out],
    "X" (the input this linear reads) [M][in], "dY" [M][out]; bf16, torch Philox."""
    lin = CONFIGS[5].linears[slot]
    if what == "W":
        return device_normal_bf16(stack_seed(layer, slot, TID_W), (lin.d_out, lin.d_in), 0.02, device)
    if what == "A":
        return device_normal_bf16(stack_seed(layer, slot, TID_A), (lin.d_in, lin.r), 0.02, device)
    if what == "B":
        return device_normal_bf16(stack_seed(layer, slot, TID_B), (lin.r, lin.d_out), 0.02, device)
    if what == "X":
        src = STACK_INPUT_SLOT[slot]
        return device_normal_bf16(stack_seed(layer, src, TID_X), (lin.M, lin.d_in), 1.0, device)
    if what == "dY":
        return device_normal_bf16(stack_seed(layer, slot, TID_DY), (lin.M, lin.d_out), 1.0, device)
    raise ValueError(what)


def custom_linear(M: int, d_in: int, d_out: int, r: int, seed: int, alpha: float = 16.0,
                  w_std: float = 0.02, outlier_p: float = 0.0) -> LinearInputs:
    """Inputs for an arbitrary shape (used for ragged and edge-case tests)."""
    lin = Linear("custom", M, d_in, d_out, r, alpha, outlier_p)
    return LinearInputs(
        normal_bf16(seed * 10 + TID_W, (d_out, d_in), w_std, outlier_p=outlier_p, mask_seed=seed * 10 + TID_MASK),
        normal_bf16(seed * 10 + TID_A, (d_in, r), 0.02),
        normal_bf16(seed * 10 + TID_B, (r, d_out), 0.02),
        normal_bf16(seed * 10 + TID_X, (M, d_in), 1.0),
        normal_bf16(seed * 10 + TID_DY, (M, d_out), 1.0),
        lin,
    )
