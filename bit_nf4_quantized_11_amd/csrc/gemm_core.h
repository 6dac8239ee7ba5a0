// Shared pieces of the two large-M dequantizing GEMMs (forward Y and backward dX).
//
// Both compute a [256 tokens] x [128 features] output tile per workgroup of 512
// threads with v_mfma_f32_32x32x16_bf16, reducing over 64 at a time through a
// double-buffered LDS stage.  The eight waves run two per SIMD: wave w owns the
// 128-token x 64-feature quarter (w & 3) of the tile (token half (w & 1), feature
// half (w >> 1 & 1)) for the reduction slices 32 (w >> 2) .. +31 of every stage, and
// the two waves of a quarter add their accumulators through LDS at the end.  Two
// waves per SIMD keep the LDS busy while the other wave of the pair issues MFMAs.
//
// LDS tiles (bf16):
//   token tile    [256 rows][64 reduction]   (X or dY, or the adapter activations)
//   feature tile  [128 rows][64 reduction]   (forward: the dequantized weight rows;
//                                             backward adapter: rows of A)
//   natural tile  [64 reduction][128 features] (backward: the dequantized weight as
//                                             stored, row n = one weight row;
//                                             forward adapter: rows of B)
// The gfx950 LDS serves 256 bytes per clock from 64 four-byte banks: a 16-byte
// access is conflict-free when each group of 16 lanes covers 256 distinct bytes
// modulo 256, an 8-byte access when each group of 32 lanes does.
// Row-major tiles of 64 reduction values are kept as two halves (reduction 0..31
// and 32..63) of 64-byte rows of four 16-byte chunks; chunk c of row r in half h
// sits at position c ^ ((r >> 2) & 3) ^ h.  Then 16 consecutive rows of one half
// fill all banks for any chunk (an MFMA fragment read), and so do the store patterns
// used below: four rows x the four chunks of one half (tokens) and four rows x chunks
// {d, 2+d, 4+d, 6+d} (weight rows, four threads per row).  The natural tile has
// 256-byte rows of sixteen 16-byte chunks; chunk g of row r sits at
// g ^ 4 (r & 3) ^ (r & 1): its stores (two rows x the eight chunks of one parity)
// and its transposing fragment reads (four rows x 64 bytes per 32 lanes) are
// conflict-free.
//
// Global loads go through raw buffer resources: an access whose vector offset is
// past the end of a buffer returns zero, so tile edges need no branches.  Only
// offsets that can never cross the end (a column inside a row, a stage inside a
// weight row) go into the scalar offset; row offsets stay in the vector offset.
//
// The MFMA computes C[feature][token]: operand A = feature rows, operand B = token
// rows.  Lane l of a 32x32 result holds C[8*(v/4) + 4*(l/32) + v%4][l % 32],
// v = 0..15: groups of four consecutive features of one token, each stored as one
// 8-byte write of the row-major [token][feature] output.
#pragma once

#include "common.h"

namespace qlora {
namespace gemm {

constexpr int BT = 256;   // tokens per tile
constexpr int BF = 128;   // features per tile
constexpr int BR = 64;    // reduction per stage
constexpr int NT = 512;   // threads (8 waves)

constexpr int HALF_T = BT * 32;   // elements per half of the token tile
constexpr int HALF_F = BF * 32;
constexpr int TILE_T = BT * BR;   // elements per token-tile buffer
constexpr int TILE_F = BF * BR;   // elements per feature (or natural) tile buffer
// LDS of one workgroup: two token buffers and two feature buffers (96 KiB); the final
// exchange of accumulators reuses it.
constexpr int SMEM_ELEMS = 2 * TILE_T + 2 * TILE_F;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  // raw buffer (stride 0), 32-bit data format word of gfx9-family buffer descriptors
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v.x, v.y);
}

// wave roles
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int wave_t() { return wave_id() & 1; }          // token half of the tile
__device__ __forceinline__ int wave_f() { return (wave_id() >> 1) & 1; }   // feature half of the tile
__device__ __forceinline__ int wave_k() { return wave_id() >> 2; }         // reduction half of a stage

// element offset of 16-byte chunk `chunk` (0..7) of row `row` in a tile of halves of `half_elems`
__device__ __forceinline__ int swz(int half_elems, int row, int chunk) {
  const int h = chunk >> 2;
  return h * half_elems + row * 32 + ((((chunk & 3) ^ ((row >> 2) & 3)) ^ h) << 3);
}
__device__ __forceinline__ int swzT(int row, int chunk) { return swz(HALF_T, row, chunk); }
__device__ __forceinline__ int swzF(int row, int chunk) { return swz(HALF_F, row, chunk); }

// element offset of 16-byte chunk g (0..15) of row r of the natural [64][128] tile
__device__ __forceinline__ int swzN(int row, int g) {
  return row * 128 + ((g ^ ((row & 3) << 2) ^ (row & 1)) << 3);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---- token operand --------------------------------------------------------------------------
// Rows m0..m0+255 of a row-major [rows][ld] bf16 matrix, reduction columns c0..c0+63.
// Part i (0..3) of thread t: row 128 (i % 2) + t / 4, half i / 2, chunk 4 (i / 2) + t % 4.
struct TokenSrc {
  rsrc_t r;
  uint32_t row_off[2];   // byte offset of this thread's row of part i % 2, plus its chunk
  uint32_t end;          // buffer size in bytes: an offset that reads as zero
};

__device__ __forceinline__ TokenSrc token_src(const void* p, uint64_t bytes, uint32_t ld, uint32_t m0) {
  const int t = threadIdx.x;
  TokenSrc s;
  s.r = make_rsrc(p, bytes);
  s.end = (uint32_t)bytes;
#pragma unroll
  for (int q = 0; q < 2; ++q) s.row_off[q] = (m0 + (uint32_t)(128 * q + (t >> 2))) * ld * 2 + (uint32_t)(t & 3) * 16;
  return s;
}

struct TokenRegs {
  uint4 v[4];
};

// columns c0.. of a matrix whose every row has at least c0 + 64 columns
__device__ __forceinline__ void load_tokens(TokenRegs& R, const TokenSrc& s, uint32_t c0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) R.v[i] = ld16(s.r, s.row_off[i & 1], c0 * 2 + (uint32_t)(i >> 1) * 64);
}

// columns c0..c0+63 where the rows end at ncols (a multiple of 8): chunks past the end read zero
__device__ __forceinline__ void load_tokens_edge(TokenRegs& R, const TokenSrc& s, uint32_t c0, uint32_t ncols) {
  const uint32_t col = c0 + (uint32_t)(threadIdx.x & 3) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool in = col + (uint32_t)(i >> 1) * 32 < ncols;
    R.v[i] = ld16(s.r, in ? s.row_off[i & 1] + c0 * 2 + (uint32_t)(i >> 1) * 64 : s.end);
  }
}

__device__ __forceinline__ void store_tokens_part(const TokenRegs& R, uint16_t* __restrict__ sT, int i) {
  const int t = threadIdx.x;
  *reinterpret_cast<uint4*>(sT + swzT(128 * (i & 1) + (t >> 2), 4 * (i >> 1) + (t & 3))) = R.v[i];
}

// ---- accumulators and fragments ---------------------------------------------------------------
struct Acc {
  f32x16 c[2][4];   // [32-feature tile][32-token tile]
};

__device__ __forceinline__ void acc_zero(Acc& a) {
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int v = 0; v < 16; ++v) a.c[f][m][v] = 0.0f;
}

struct Frags {
  u32x4 fa[2], tb[4];
};

// ks (0..3) selects 16 of the 64 reduction values of the stage
__device__ __forceinline__ void read_tokens(Frags& F, const uint16_t* __restrict__ sT, int ks) {
  const int lane = threadIdx.x & 63, wt = wave_t();
  const int chunk = ks * 2 + (lane >> 5);
#pragma unroll
  for (int m = 0; m < 4; ++m)
    F.tb[m] = *reinterpret_cast<const u32x4*>(sT + swzT(wt * 128 + m * 32 + (lane & 31), chunk));
}

// feature operand from a feature tile [128][64]
__device__ __forceinline__ void read_frags(Frags& F, const uint16_t* __restrict__ sT,
                                           const uint16_t* __restrict__ sF, int ks) {
  const int lane = threadIdx.x & 63, wf = wave_f();
  const int chunk = ks * 2 + (lane >> 5);
#pragma unroll
  for (int f = 0; f < 2; ++f)
    F.fa[f] = *reinterpret_cast<const u32x4*>(sF + swzF(wf * 64 + f * 32 + (lane & 31), chunk));
  read_tokens(F, sT, ks);
}

// feature operand from a natural tile [64][128] with transposing reads: 16-lane group
// G = lane / 16 takes features 16 (G % 2) + 0..15 of the 32, reduction rows
// 16 ks + 8 (G / 2) + 4 half + 0..3; lane j of the group points at row + j / 4, column 4 (j % 4),
// and receives the four rows of column j.
__device__ __forceinline__ u32x4 read_natural_a(const uint16_t* __restrict__ sN, int fcol, int ks) {
  const int lane = threadIdx.x & 63, j = lane & 15, G = lane >> 4;
  const int row = ks * 16 + (G >> 1) * 8 + (j >> 2);
  const int col = fcol + (G & 1) * 16 + (j & 3) * 4;
  const int g = col >> 3, sub = col & 7;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(sN + swzN(row, g) + sub));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(sN + swzN(row + 4, g) + sub));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  u32x4 o;
  o.x = a.x; o.y = a.y; o.z = b.x; o.w = b.y;
  return o;
}

__device__ __forceinline__ void read_frags_natural(Frags& F, const uint16_t* __restrict__ sT,
                                                   const uint16_t* __restrict__ sN, int ks) {
  const int wf = wave_f();
#pragma unroll
  for (int f = 0; f < 2; ++f) F.fa[f] = read_natural_a(sN, wf * 64 + f * 32, ks);
  read_tokens(F, sT, ks);
}

__device__ __forceinline__ void mma_group(Acc& a, const Frags& F, int f) {
#pragma unroll
  for (int m = 0; m < 4; ++m) a.c[f][m] = mfma32(F.fa[f], F.tb[m], a.c[f][m]);
}

// Scheduling hint for one main-loop stage of a wave (16 MFMAs next to about 70 VALU
// instructions of dequantization): MFMAs in pairs, each pair followed by up to eight VALU
// instructions.  Left to itself the scheduler clusters the MFMAs of one of the two stages
// of a loop trip ahead of all of that stage's dequantization, which leaves the matrix core
// idle while the wave works through it; measured, the pairing is 5-7 % faster.
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
  }
}

// This wave's half of one 64-deep stage, without interleaved work (tail and adapter stages).
template <bool NATURAL>
__device__ __forceinline__ void mma_stage(Acc& a, const uint16_t* __restrict__ sT, const uint16_t* __restrict__ sF) {
  Frags F;
  const int kh = wave_k();
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    if constexpr (NATURAL)
      read_frags_natural(F, sT, sF, 2 * kh + k2);
    else
      read_frags(F, sT, sF, 2 * kh + k2);
    mma_group(a, F, 0);
    mma_group(a, F, 1);
  }
}

// Add the accumulators of the two waves of each quarter: waves 4..7 hand theirs to waves
// 0..3 through LDS (`smem`, free at this point), one feature tile at a time.  Returns true
// in the waves that hold the sum.
__device__ __forceinline__ bool combine_halves(Acc& a, uint16_t* __restrict__ smem) {
  const int lane = threadIdx.x & 63, q = wave_id() & 3;
  const bool upper = wave_k() != 0;
  float4* x = reinterpret_cast<float4*>(smem);
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    if (upper) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x16 c = a.c[f][m];
          x[((q * 4 + m) * 4 + v4) * 64 + lane] = make_float4(c[4 * v4], c[4 * v4 + 1], c[4 * v4 + 2], c[4 * v4 + 3]);
        }
    }
    __syncthreads();
    if (!upper) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const float4 o = x[((q * 4 + m) * 4 + v4) * 64 + lane];
          a.c[f][m][4 * v4 + 0] += o.x;
          a.c[f][m][4 * v4 + 1] += o.y;
          a.c[f][m][4 * v4 + 2] += o.z;
          a.c[f][m][4 * v4 + 3] += o.w;
        }
    }
    __syncthreads();
  }
  return !upper;
}

// Store bf16(acc) of this wave's quarter into out [ntok][nfeat] row-major (nfeat % 8 == 0).
__device__ __forceinline__ void store_out(const Acc& a, uint16_t* __restrict__ out, int64_t ld, int64_t m0,
                                          int64_t ntok, int64_t f0, int64_t nfeat) {
  const int lane = threadIdx.x & 63;
  const int wt = wave_t(), wf = wave_f();
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t tok = m0 + wt * 128 + m * 32 + (lane & 31);
    if (tok >= ntok) continue;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t feat = f0 + wf * 64 + f * 32 + 8 * g + 4 * (lane >> 5);
        if (feat >= nfeat) continue;
        const f32x16 v = a.c[f][m];
        uint2 o;
        o.x = pack_bf16x2(v[4 * g + 0], v[4 * g + 1]);
        o.y = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
        *reinterpret_cast<uint2*>(out + tok * ld + feat) = o;
      }
  }
}

// Store the fp32 accumulators of this wave's quarter into out [ntok][ld] (ld % 4 == 0, 16-byte
// aligned rows), features below nfeat only.
__device__ __forceinline__ void store_out_f32(const Acc& a, float* __restrict__ out, int64_t ld, int64_t m0,
                                              int64_t ntok, int64_t f0, int64_t nfeat) {
  const int lane = threadIdx.x & 63;
  const int wt = wave_t(), wf = wave_f();
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t tok = m0 + wt * 128 + m * 32 + (lane & 31);
    if (tok >= ntok) continue;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t feat = f0 + wf * 64 + f * 32 + 8 * g + 4 * (lane >> 5);
        if (feat >= nfeat) continue;
        const f32x16 v = a.c[f][m];
        *reinterpret_cast<float4*>(out + tok * ld + feat) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
      }
  }
}

// ---- NF4 weight producer --------------------------------------------------------------------
// Per stage every thread dequantizes 16 weights (8 code bytes, a quarter of a block); the
// four threads of a block sit in one DPP quad (lanes 4j..4j+3, quarter = lane % 4) and
// build the block's scaled 16-entry table together: lane q forms the bf16 values of levels
// 4q..4q+3 and the quad exchanges them.
struct QuadLevels {
  float l[4];   // level[4q + i] of this lane's quarter q
};

__device__ __forceinline__ QuadLevels quad_levels(const NF4Table& t) {
  const int q = threadIdx.x & 3;
  QuadLevels L;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    L.l[i] = q == 0 ? t.level[i] : q == 1 ? t.level[4 + i] : q == 2 ? t.level[8 + i] : t.level[12 + i];
  return L;
}

template <int SRC>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  // DPP quad_perm [SRC, SRC, SRC, SRC]
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, SRC | (SRC << 2) | (SRC << 4) | (SRC << 6), 0xF, 0xF, false);
}

// Planes of val[c] = bf16_RNE(fl32(level[c] * s)) (see make_planes), built across the quad.
__device__ __forceinline__ Planes quad_planes(const QuadLevels& L, float s) {
  const uint32_t v0 = pack_bf16x2(__fmul_rn(L.l[0], s), __fmul_rn(L.l[1], s));
  const uint32_t v1 = pack_bf16x2(__fmul_rn(L.l[2], s), __fmul_rn(L.l[3], s));
  const uint32_t lo = __builtin_amdgcn_perm(v1, v0, 0x06040200u);
  const uint32_t hi = __builtin_amdgcn_perm(v1, v0, 0x07050301u);
  Planes p;
  p.lo[0] = quad_bcast<0>(lo);
  p.lo[1] = quad_bcast<1>(lo);
  p.lo[2] = quad_bcast<2>(lo);
  p.lo[3] = quad_bcast<3>(lo);
  p.hi[0] = quad_bcast<0>(hi);
  p.hi[1] = quad_bcast<1>(hi);
  p.hi[2] = quad_bcast<2>(hi);
  p.hi[3] = quad_bcast<3>(hi);
  return p;
}

// Map a linear workgroup id to a (token tile, feature tile) pair.  Workgroups are
// dispatched round-robin over the 8 XCDs; give each XCD a contiguous run of tiles
// (token-tile major) so the tiles sharing a token panel share an L2.
__device__ __forceinline__ void tile_of(int64_t tiles_t, int64_t tiles_f, int64_t& tt, int64_t& tf,
                                        int64_t id = -1) {
  const int64_t n = tiles_t * tiles_f;
  int64_t L = id < 0 ? (int64_t)blockIdx.x : id;
  if ((n & 7) == 0) L = (L & 7) * (n >> 3) + (L >> 3);
  tt = L / tiles_f;
  tf = L - tt * tiles_f;
}

}  // namespace gemm
}  // namespace qlora
