// Device helpers shared by the libqlora kernels (gfx950).
//
// Number formats ("QLoRA: Efficient Finetuning of Quantized LLMs", sections
// "NormalFloat: 4 bits for a bell curve" and "Double quantization"):
//   * NF4: a 4-bit index into 16 fp32 levels;
//   * block constants stored as OCP FP8 E4M3 codes (the pages' "8-bit float");
//   * bf16 compute type.
// Every value that must match the definition bit for bit is computed with
// explicit single roundings (__fmul_rn / __fadd_rn; the library is also built
// with -ffp-contract=off).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;    // weights per NF4 block
constexpr int kSuper = 256;   // block constants per second-level group
constexpr int kBlockBytes = 32;   // code bytes per 64 weights (the code layout's chunk)
constexpr int kQuantSlots = 512;  // quantize workgroups at most: one partial sum slot each (workspace)
constexpr int kSumLimbs = 10;     // 32-bit limbs of an exact sum of block constants (320 bits)

// Passed by value to every kernel that encodes or decodes NF4 (lives in SGPRs /
// the kernel-argument segment).
struct NF4Table {
  float level[16];
  float thr[15];
  float pad_;
};

// Encoder table: the normalized weights' range split into kLutBins bins (bin_of below); for
// each bin, the number of thresholds that lie below every value the bin can hold, and the one
// threshold (or +inf) that lies inside it.  The code of x is base[b] + (x > t[b]), which equals
// the number of thresholds below x exactly, for every fp32 x (thresholds are at least two bins
// apart in every table).
constexpr int kLutBins = 64;
struct ThrLut {
  float t[kLutBins];
  uint32_t base[kLutBins];
};

// The bin of a normalized weight: floor(32 x + 32) computed with one fused multiply-add,
// clamped to [0, 63] (NaN -> 0).  Host and device evaluate the same IEEE operations.
__host__ __device__ __forceinline__ int lut_bin(float x) {
  float y = __builtin_fmaf(x, 32.0f, 32.0f);
  y = __builtin_fmaxf(y, 0.0f);
  y = __builtin_fminf(y, (float)(kLutBins - 1));
  return (int)__builtin_floorf(y);
}

// Describes a quantized weight inside kernels.
struct NF4View {
  const uint8_t* codes;   // 32 bytes per 64 weights (code layout of qlora.h)
  const void* absmax;     // u8 E4M3 codes (dq) or fp32
  const float* c1;
  const float* mu;
  int32_t dq;
  int32_t cb;             // codebook: index of the 16-entry table the codes refer to
  int32_t bshift;         // log2 of the block size (5..8): one constant per 2^bshift weights
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// bf16
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest even, integer form (exact for every finite input, denormals included).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Two fp32 -> {bf16(lo), bf16(hi)} with round to nearest even.  On gfx950 this is
// one v_cvt_pk_bf16_f32, which was checked against the integer rounding above on
// every non-NaN fp32 bit pattern (denormals and ties included) with no mismatch.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ------------------------------------------------------------------------------------------
// FP8 E4M3 (OCP e4m3fn): bias 7, 3 fraction bits, max 448, subnormals m * 2^-9,
// codes 0x7F and 0xFF are NaN.
// ------------------------------------------------------------------------------------------
// Decode with the gfx950 conversion instruction (v_cvt_f32_fp8 reads OCP e4m3fn on this
// architecture; every E4M3 value is exact in fp32).  A test dequantizes a weight whose
// block constants run through all 256 codes and compares with the definition.
__device__ __forceinline__ float e4m3_decode(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }
// the code in byte 1 of c
__device__ __forceinline__ float e4m3_decode_byte1(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 1); }

// Round-to-nearest-even encode; magnitudes above 448 clamp to 448 (never reached
// by the quantizer, whose values stay within 448 * (1 + 2^-22)).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  uint32_t bits = __float_as_uint(y);
  uint32_t sign = (bits >> 31) << 7;
  uint32_t a = bits & 0x7FFFFFFFu;
  float af = __uint_as_float(a);
  uint32_t code;
  if (af < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(__fmul_rn(af, 512.0f));   // 0..8, 8 == smallest normal
  } else {
    uint32_t mant = a & 0x7FFFFFu;
    int e = (int)(a >> 23) - 127;
    uint32_t q = mant >> 20, rem = mant & 0xFFFFFu;
    uint32_t up = (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    code = (uint32_t)((e + 7) << 3) + q + up;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

// ------------------------------------------------------------------------------------------
// Block scales ("doubleDequant", inner step): s' = fl32(fl32(dec(c2) * c1) + mu)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float block_scale(const NF4View& w, int64_t blk) {
  if (w.dq) {
    uint32_t c2 = ((const uint8_t*)w.absmax)[blk];
    float c1 = w.c1[blk >> 8];
    return __fadd_rn(__fmul_rn(e4m3_decode(c2), c1), *w.mu);
  }
  return ((const float*)w.absmax)[blk];
}

// ------------------------------------------------------------------------------------------
// Scaled 16-entry bf16 table in byte planes, and nibble lookup with v_perm_b32.
//
// val[c] = bf16_RNE(fl32(level[c] * s)) for c = 0..15.  lo[i] holds the low
// bytes of val[4i..4i+3], hi[i] the high bytes.  A lookup of four 4-bit codes
// (one per byte of `idx`) returns the low and high bytes of the four values;
// v_perm_b32 selects a byte out of an 8-byte pair, so entries 0..7 and 8..15
// are looked up separately and merged on bit 3 of each code.
// ------------------------------------------------------------------------------------------
struct Planes {
  uint32_t lo[4];
  uint32_t hi[4];
};

__device__ __forceinline__ Planes make_planes(const NF4Table& t, float s) {
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = pack_bf16x2(__fmul_rn(t.level[2 * i], s), __fmul_rn(t.level[2 * i + 1], s));
  Planes p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // v[2i] = {val[4i], val[4i+1]}, v[2i+1] = {val[4i+2], val[4i+3]}
    p.lo[i] = __builtin_amdgcn_perm(v[2 * i + 1], v[2 * i], 0x06040200u);
    p.hi[i] = __builtin_amdgcn_perm(v[2 * i + 1], v[2 * i], 0x07050301u);
  }
  return p;
}

// Four codes -> two dwords of bf16 pairs, in order {val[c0], val[c1]} and {val[c2], val[c3]}.
// sel holds the low three bits of each code (one per byte), mask is 0xFF in each byte
// whose code is 8 or more: entries 0..7 and 8..15 are looked up separately (v_perm_b32
// selects a byte out of an 8-byte pair) and merged on the mask.
__device__ __forceinline__ void lookup4(const Planes& p, uint32_t sel, uint32_t mask, uint32_t& d0, uint32_t& d1) {
  const uint32_t lo_a = __builtin_amdgcn_perm(p.lo[1], p.lo[0], sel);
  const uint32_t lo_b = __builtin_amdgcn_perm(p.lo[3], p.lo[2], sel);
  const uint32_t hi_a = __builtin_amdgcn_perm(p.hi[1], p.hi[0], sel);
  const uint32_t hi_b = __builtin_amdgcn_perm(p.hi[3], p.hi[2], sel);
  const uint32_t lo = (lo_b & mask) | (lo_a & ~mask);
  const uint32_t hi = (hi_b & mask) | (hi_a & ~mask);
  d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// 0xFF in byte j of the result where bit 7 of byte j of x is set.  v_perm_b32 selectors
// 8..11 replicate bit 7 of bytes 1, 3, 5 and 7 of its 8-byte input {S0, S1}; with S1 = x
// and S0 = x << 8 those are bytes 1, 3, 0 and 2 of x.
__device__ __forceinline__ uint32_t top_bit_mask(uint32_t x) {
  return __builtin_amdgcn_perm(x << 8, x, 0x090B080Au);
}

// One code dword = 8 weights of a group; byte i holds element i in bits 3..0 and
// element i+4 in bits 7..4.  Output: 4 dwords = 8 bf16 in element order.
__device__ __forceinline__ u32x4 dequant8(const Planes& p, uint32_t codes) {
  u32x4 o;
  uint32_t a, b, c, d;
  // low nibbles: bit 3 of each byte moves to bit 7 with a shift by 4
  lookup4(p, codes & 0x07070707u, top_bit_mask(codes << 4), a, b);
  lookup4(p, (codes >> 4) & 0x07070707u, top_bit_mask(codes), c, d);
  o.x = a; o.y = b; o.z = c; o.w = d;
  return o;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

}  // namespace qlora
