"""Oracle: NF4 blockwise quantization with double quantization, and its inverse.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy, written
for reading, not for speed.  bf16 values travel as uint16 bit patterns.

What is fixed by the pages, and where:
  * NF4 levels: 16 values built from standard-normal quantiles, the two tails
    pulled in by an offset of 0.9677083, 8 positive levels, 7 negative levels and
    an exact zero, the whole set divided by its largest magnitude so that the
    ends are exactly -1 and +1 ([Explainer] "NormalFloat: 4 bits for a bell
    curve", the code-point listing and the two paragraphs around it).
  * Absmax scaling: the scale constant is c = (largest code) / absmax, a value
    is normalized by multiplying it with c ([Explainer] "Quantize in blocks, not
    all at once", the Int8 absmax formula and its dequant).  For NF4 the largest
    code is 1, so c = 1/absmax.
  * Blocks of 64 contiguous weights of the flattened tensor, one constant each
    ([Explainer] "Quantize in blocks, not all at once"; [Addaly] "NF4, and why
    not plain int4").
  * Nearest level ([Review] "What QLoRA Actually Does", item 1).
  * Double quantization: the block constants, after subtracting their mean, are
    stored as 8-bit floats in groups of 256 with one 32-bit scale per group
    ([Explainer] "Double quantization"; [Glossary] calls the 8-bit type FP8).
  * doubleDequant: first rebuild the block scales from c2 (8-bit) and c1
    (fp32), then turn the 4-bit codes into bf16 with those scales ([Explainer]
    "The QLoRA layer, end to end").

Readings where the pages leave a step open (each is listed in the design notes):
  R1  levels computed in float64 by the printed procedure, rounded once to fp32;
  R2  x = fl32(w * fl32(1/absmax)) with a correctly rounded reciprocal;
  R3  nearest fp32 level in exact arithmetic, ties to the lower index;
  R4  a block whose absmax is below the smallest normal fp32 (2^-126) is a zero
      block: stored absmax 0, every code 7 (the exact zero);
  R5  W is the [out][in] row-major weight; blocks run along the flattened array;
  R6  codes are stored as whole 64-blocks of 32 bytes; inside a block, the
      8-element group g (elements 8g..8g+7) sits in bytes 4g..4g+3, byte i of a
      group holding element i in bits 3..0 and element i+4 in bits 7..4;
      positions past the end of the tensor hold code 7 (the exact zero);
  R7  the 8-bit float is OCP FP8 E4M3 (max 448), round to nearest even, the
      group's largest centered magnitude mapped to 448;
  R8  one mean per tensor, mu = fl32(S / nblk) with S the correctly rounded
      float64 value of the exact sum of the stored absmax values;
  R9  c1 = fl32(m / 448); a group whose c1 is below 2^-126 stores c1 = 0 and
      all c2 = 0; otherwise c2 = E4M3(fl32(fl32(a - mu) * fl32(1/c1)));
  R10 s' = fl32(fl32(dec(c2) * c1) + mu), two roundings, no fused multiply-add;
  R11 the codes use the true absmax; dequant uses s';
  R12 dequantized weight = bf16_RNE(fl32(level[code] * s')).
  R20 other block sizes (32, 128, 256; [Explainer] "Double quantization": smaller blocks
      are more precise and cost more constants, larger blocks the reverse): one constant
      per `block` contiguous weights, double quantization still in groups of 256
      constants; the code layout of R6 is unchanged (it is defined per 8-element group)
      and the code buffer is padded with the zero code to whole blocks and to a whole
      number of 64-element chunks.
"""
from __future__ import annotations

import math

import numpy as np

OFFSET = 0.9677083      # [Explainer] "NormalFloat", code-point listing
BLOCK = 64              # [Explainer] "Quantize in blocks"; [Addaly] "NF4, and why not plain int4"
BLOCKS = (32, 64, 128, 256)   # block sizes of the format variants (reading R20)
SUPER = 256             # [Explainer] "Double quantization"; [Addaly] same section
FP8_MAX = 448.0         # largest finite OCP E4M3 value (reading R7)
FP32_MIN_NORMAL = 2.0 ** -126
ZERO_CODE = 7           # index of the exact zero among the sorted levels

_CHUNK = 1 << 20


# ----------------------------------------------------------------------------------------------
# bf16 <-> fp32 (bit level)
# ----------------------------------------------------------------------------------------------
def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest, ties to even.  Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if np.isnan(x).any():
        raise ValueError("NaN has no defined rounding here")
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------------------------
# NF4 codebook
# ----------------------------------------------------------------------------------------------
def _default_ppf(p):
    from scipy.special import ndtri

    return ndtri(p)


def nf4_levels_f64(ppf=None) -> np.ndarray:
    """The 16 NF4 levels in float64, by the procedure of [Explainer] "NormalFloat".

    8 positive quantiles at probabilities evenly spaced from OFFSET down to 1/2
    (1/2 itself excluded), 7 negative ones mirrored the same way with 8 points,
    plus an exact zero; sorted and divided by the largest magnitude.
    """
    ppf = ppf or _default_ppf
    pos = np.asarray(ppf(np.linspace(OFFSET, 0.5, 9)[:-1]), dtype=np.float64)
    neg = -np.asarray(ppf(np.linspace(OFFSET, 0.5, 8)[:-1]), dtype=np.float64)
    v = np.sort(np.concatenate([neg, [0.0], pos]))
    return v / np.max(np.abs(v))


def nf4_levels(ppf=None) -> np.ndarray:
    """The NF4 levels rounded once to fp32 (reading R1)."""
    return nf4_levels_f64(ppf).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# First-level quantization: blockwise absmax + nearest NF4 level
# ----------------------------------------------------------------------------------------------
# ----------------------------------------------------------------------------------------------
# The other 4-bit data types the pages compare NF4 with ([Explainer] "NormalFloat: 4 bits for
# a bell curve": NF4 against FP4 and Int4).  Each is a strictly ascending table of 16 fp32
# values spanning [-1, 1] with an exact zero, used exactly like the NF4 levels.
#   FP4: a 4-bit float with 2 exponent bits (bias 1) and 1 mantissa bit (the OCP E2M1
#        layout; the pages print no FP4 table, so this one is a stated choice): magnitudes
#        m/2 for exponent 0 and 2^(e-1) * (1 + m/2) otherwise, i.e. 0, 0.5, 1, 1.5, 2, 3,
#        4, 6, with both signs, divided by 6 so the block maximum maps to 1.  Its +0 and -0
#        coincide, which leaves 15 values; index 0 gets -4/3, outside [-1, 1], so it is
#        never the nearest level and the table stays strictly ascending.
#   Int4: k/7 for k = -8..7, the 4-bit version of the absmax integer quantizer
#        round(127 x / absmax) of [Explainer] "Quantize in blocks, not all at once" with
#        the largest code 7; k = -8 (index 0) is never the nearest level in [-1, 1].
# ----------------------------------------------------------------------------------------------
def e2m1_magnitude(code3: int) -> float:
    """Magnitude of a 3-bit E2M1 pattern (2 exponent bits, bias 1, 1 mantissa bit)."""
    e, m = code3 >> 1, code3 & 1
    return 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)


def fp4_levels() -> np.ndarray:
    mags = [e2m1_magnitude(c) for c in range(8)]               # 0, 0.5, ..., 6
    vals = [-8.0 / 6.0] + [-v / 6.0 for v in reversed(mags[1:])] + [v / 6.0 for v in mags]
    return np.array(vals, dtype=np.float64).astype(np.float32)


def int4_levels() -> np.ndarray:
    return (np.arange(-8, 8, dtype=np.float64) / 7.0).astype(np.float32)


CODEBOOKS = ("nf4", "fp4", "int4")


def codebook_levels(name: str = "nf4") -> np.ndarray:
    """The 16 fp32 levels of a codebook: "nf4", "fp4" or "int4"."""
    if name == "nf4":
        return nf4_levels()
    if name == "fp4":
        return fp4_levels()
    if name == "int4":
        return int4_levels()
    raise ValueError(name)


def zero_code(levels: np.ndarray) -> int:
    """Index of the exact zero of a table (the code of zero blocks and padding)."""
    idx = np.flatnonzero(np.asarray(levels, dtype=np.float32) == 0.0)
    assert idx.size == 1
    return int(idx[0])


def num_blocks(numel: int, block: int = BLOCK) -> int:
    return -(-numel // block)


def code_elems(numel: int, block: int = BLOCK) -> int:
    """Elements the code buffer holds: whole blocks, and a whole number of 64-element
    chunks of 32 bytes (reading R20)."""
    unit = max(block, 64)
    return -(-numel // unit) * unit


def num_super(nblk: int) -> int:
    return -(-nblk // SUPER)


def _blocks_f32(w_bits: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Flattened weight as fp32 values, zero padded to whole blocks, shape [nblk, block]."""
    flat = bf16_to_f32(np.ravel(w_bits))
    nblk = num_blocks(flat.size, block)
    out = np.zeros(nblk * block, dtype=np.float32)
    out[: flat.size] = flat
    return out.reshape(nblk, block)


def blockwise_absmax(w_bits: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Largest magnitude of each block (padding is zero so it never wins); reading R4 applied."""
    a = np.abs(_blocks_f32(w_bits, block)).max(axis=1)
    a[a < np.float32(FP32_MIN_NORMAL)] = 0.0
    return a.astype(np.float32)


def nearest_level(x: np.ndarray, levels: np.ndarray | None = None) -> np.ndarray:
    """Index of the nearest level to each fp32 x, ties to the lower index (reading R3).

    Brute force over the 16 levels in float64.  x and the levels are fp32, so
    x - level is exact in float64 whenever the two are within 29 binades of one
    another, which covers every case where two distances could be equal or
    close; argmin returns the first (lower) index on ties.
    """
    lv = (nf4_levels() if levels is None else levels).astype(np.float64)
    x = np.ravel(np.asarray(x, dtype=np.float32))
    out = np.empty(x.size, dtype=np.uint8)
    for s in range(0, x.size, _CHUNK):
        xs = x[s:s + _CHUNK].astype(np.float64)
        out[s:s + _CHUNK] = np.argmin(np.abs(xs[:, None] - lv[None, :]), axis=1)
    return out


def normalize_blocks(blocks: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """x = fl32(w * fl32(1/absmax)) per block (reading R2); zero blocks give x = 0."""
    inv = np.zeros_like(absmax, dtype=np.float32)
    nz = absmax > 0
    inv[nz] = np.float32(1.0) / absmax[nz]
    x = (blocks * inv[:, None]).astype(np.float32)
    x[~nz] = 0.0
    return x


def nf4_codes(w_bits: np.ndarray, absmax: np.ndarray | None = None, levels: np.ndarray | None = None,
              block: int = BLOCK) -> np.ndarray:
    """Unpacked 4-bit codes (one uint8 per element, padded to whole blocks); NF4 unless
    another table is given."""
    lv = nf4_levels() if levels is None else levels
    blocks = _blocks_f32(w_bits, block)
    if absmax is None:
        absmax = blockwise_absmax(w_bits, block)
    codes = np.empty(blocks.shape, dtype=np.uint8)
    rows_per_chunk = max(1, _CHUNK // block)
    for s in range(0, blocks.shape[0], rows_per_chunk):
        x = normalize_blocks(blocks[s:s + rows_per_chunk], absmax[s:s + rows_per_chunk])
        codes[s:s + rows_per_chunk] = nearest_level(x, lv).reshape(x.shape)
    codes[absmax == 0] = zero_code(lv)
    return codes.reshape(-1)


def codes_for_blocks(w_bits: np.ndarray, absmax: np.ndarray, block_ids: np.ndarray,
                     levels: np.ndarray | None = None, block: int = BLOCK) -> np.ndarray:
    """Unpacked codes [len(block_ids), block] of selected blocks only (for sampled checks at full size)."""
    lv = nf4_levels() if levels is None else levels
    flat = np.ravel(w_bits)
    block_ids = np.asarray(block_ids, dtype=np.int64)
    blocks = np.zeros((block_ids.size, block), dtype=np.float32)
    for i, b in enumerate(block_ids):
        seg = bf16_to_f32(flat[b * block:(b + 1) * block])
        blocks[i, : seg.size] = seg
    a = absmax[block_ids]
    codes = nearest_level(normalize_blocks(blocks, a), lv).reshape(blocks.shape)
    codes[a == 0] = zero_code(lv)
    return codes


def pack_nibbles(codes: np.ndarray, numel: int, pad_code: int = ZERO_CODE, block: int = BLOCK) -> np.ndarray:
    """Codes -> 32 bytes per 64 elements in the layout of reading R6, for code_elems(numel,
    block) elements.  Positions past numel hold pad_code (the table's zero; 7 for NF4)."""
    c = np.full(code_elems(numel, block), pad_code, dtype=np.uint8)
    c[:numel] = np.ravel(codes)[:numel]
    g = c.reshape(-1, 8)                                   # one row per 8-element group
    return (g[:, 0:4] | (g[:, 4:8] << 4)).astype(np.uint8).reshape(-1)


def unpack_nibbles(packed: np.ndarray, numel: int) -> np.ndarray:
    """Inverse of pack_nibbles; returns the first numel codes."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1, 4)
    out = np.empty((p.shape[0], 8), dtype=np.uint8)
    out[:, 0:4] = p & 0x0F
    out[:, 4:8] = p >> 4
    return out.reshape(-1)[:numel]


# ----------------------------------------------------------------------------------------------
# FP8 E4M3 (the 8-bit float of the second quantization; reading R7)
# ----------------------------------------------------------------------------------------------
def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3 code, round to nearest even; magnitudes above 448 clamp to 448.

    Normal codes: exponent field e in 1..15 (bias 7), 3 fraction bits; field 0
    holds the subnormals m * 2^-9.  Code 0x7F (and 0xFF) is NaN and is never
    produced.  The sign of a value that rounds to zero is kept.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y.astype(np.float64)).ravel()
    code = np.zeros(a.size, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)          # 0..8; 8 is the smallest normal
    nor = ~sub
    mant, ex = np.frexp(a[nor])                                        # a = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1                                        # a = (2 mant) * 2^e
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)            # 3-bit fraction, 0..8
    e = np.where(q == 8, e + 1, e)
    q = np.where(q == 8, 0, q)
    code[nor] = (e + 7) * 8 + q
    code = np.minimum(code, 0x7E)
    code |= np.signbit(y).ravel().astype(np.int64) << 7
    return code.astype(np.uint8).reshape(y.shape)


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    """OCP E4M3 code -> fp32 value (exact)."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return (sign * mag).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# Double quantization of the block constants
# ----------------------------------------------------------------------------------------------
def absmax_mean(absmax: np.ndarray) -> np.float32:
    """mu = fl32(S / nblk), S = the correctly rounded float64 sum of all block constants (R8)."""
    a = np.asarray(absmax, dtype=np.float32)
    s = math.fsum(a.astype(np.float64).tolist())
    return np.float32(s / a.size)


def double_quantize(absmax: np.ndarray):
    """Block constants -> (c2 uint8 [nblk], c1 fp32 [nsup], mu fp32); readings R7..R9."""
    a = np.asarray(absmax, dtype=np.float32)
    nblk = a.size
    nsup = num_super(nblk)
    mu = absmax_mean(a)
    x = (a - mu).astype(np.float32)                                    # fl32(a - mu)
    xp = np.zeros(nsup * SUPER, dtype=np.float32)
    xp[:nblk] = x
    m = np.abs(xp.reshape(nsup, SUPER)).max(axis=1)
    c1 = (m / np.float32(FP8_MAX)).astype(np.float32)                 # fl32(m / 448)
    c1[c1 < np.float32(FP32_MIN_NORMAL)] = 0.0
    inv = np.zeros_like(c1)
    nz = c1 > 0
    inv[nz] = np.float32(1.0) / c1[nz]
    sup = np.arange(nblk) // SUPER
    y = (x * inv[sup]).astype(np.float32)                              # fl32(x * fl32(1/c1))
    c2 = e4m3_encode(y)
    c2[~nz[sup]] = 0
    return c2, c1, mu


def block_scales_dq(c2: np.ndarray, c1: np.ndarray, mu: np.float32) -> np.ndarray:
    """Inner dequant of doubleDequant: s' = fl32(fl32(dec(c2) * c1) + mu) (reading R10)."""
    sup = np.arange(np.asarray(c2).size) // SUPER
    prod = (e4m3_decode(c2) * np.asarray(c1, dtype=np.float32)[sup]).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# Whole-tensor quantize / dequantize
# ----------------------------------------------------------------------------------------------
def quantize(w_bits: np.ndarray, double_quant: bool = True, codebook: str = "nf4", block: int = BLOCK) -> dict:
    """Quantize a bf16 weight (any shape; flattened row-major) to 4-bit codes of a codebook
    (NF4 by default) in blocks of `block` weights (64 by default), with optional double quant."""
    assert block in BLOCKS
    numel = int(np.asarray(w_bits).size)
    lv = codebook_levels(codebook)
    absmax = blockwise_absmax(w_bits, block)
    codes = nf4_codes(w_bits, absmax, lv, block)
    q = {"numel": numel, "codes": pack_nibbles(codes, numel, zero_code(lv), block), "absmax_true": absmax,
         "double_quant": bool(double_quant), "codebook": codebook, "block": block}
    if double_quant:
        c2, c1, mu = double_quantize(absmax)
        q.update(c2=c2, c1=c1, mu=mu, scales=block_scales_dq(c2, c1, mu))
    else:
        q.update(scales=absmax.copy())
    return q


def dequantize_codes(codes_unpacked: np.ndarray, scales: np.ndarray, levels: np.ndarray | None = None,
                     block: int = BLOCK) -> np.ndarray:
    """Outer dequant: bf16_RNE(fl32(level[code] * s')) per element (reading R12); NF4
    levels unless another table is given."""
    lv = nf4_levels() if levels is None else levels
    c = np.asarray(codes_unpacked, dtype=np.uint8).ravel()
    blk = np.arange(c.size) // block
    out = np.empty(c.size, dtype=np.uint16)
    for s in range(0, c.size, _CHUNK):
        prod = (lv[c[s:s + _CHUNK]] * scales[blk[s:s + _CHUNK]]).astype(np.float32)
        out[s:s + _CHUNK] = f32_to_bf16(prod)
    return out


def dequantize(q: dict, shape=None) -> np.ndarray:
    """doubleDequant of a quantized tensor -> bf16 bit patterns (flattened, or reshaped)."""
    numel = q["numel"]
    out = dequantize_codes(unpack_nibbles(q["codes"], numel), q["scales"], codebook_levels(q.get("codebook", "nf4")),
                           q.get("block", BLOCK))
    return out.reshape(shape) if shape is not None else out


# ----------------------------------------------------------------------------------------------
# Storage accounting ([Explainer] "Double quantization" and "The QLoRA layer, end to end")
# ----------------------------------------------------------------------------------------------
def storage_bytes(numel: int, double_quant: bool = True, block: int = BLOCK) -> dict:
    """Bytes of each stored buffer: codes, block constants, second-level scales, mean."""
    nblk = num_blocks(numel, block)
    codes = code_elems(numel, block) // 2
    if double_quant:
        return {"codes": codes, "absmax": nblk, "c1": 4 * num_super(nblk), "mu": 4}
    return {"codes": codes, "absmax": 4 * nblk, "c1": 0, "mu": 0}


def constant_bits_per_param(numel: int, double_quant: bool = True, block: int = BLOCK) -> float:
    """Bits of quantization constants per weight (everything except the 4-bit codes)."""
    b = storage_bytes(numel, double_quant, block)
    return 8.0 * (b["absmax"] + b["c1"] + b["mu"]) / numel
