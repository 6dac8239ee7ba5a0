// Shared pieces of the two large-M dequantizing GEMMs (forward Y and backward dX).
//
// Both compute a [256 tokens] x [128 features] output tile per workgroup of 256
// threads (4 waves, each 128 tokens x 64 features) with v_mfma_f32_16x16x32_bf16,
// reducing over 64 at a time through a double-buffered LDS stage:
//   sT  [256][64]  token operand (X or dY, or the adapter activations), bf16
//   sF  [128][64]  feature operand (dequantized weight, or the adapter factor), bf16
// Each tile is stored as two halves (reduction 0..31 and 32..63), each half as rows
// of four 16-byte chunks (64 bytes).  Chunk c of row r sits at position
// c ^ ((r >> 1) & 3): eight consecutive rows then cover all 32 banks for any chunk,
// which is what one MFMA fragment read touches per cycle, and the second half and
// the second buffer are constant offsets (immediate fields of the LDS instructions).
//
// Global loads go through raw buffer resources: an access past the end of a
// buffer returns zero, so tile edges need no branches.  Stage s is loaded into
// registers two stages ahead, and its LDS store is cut into eight pieces that
// sit between the eight groups of MFMAs of the stage being computed.
//
// The MFMA computes C[feature][token]: operand A = feature rows, operand B =
// token rows.  Lane l of a 16x16 result holds C[4*(l/16) + v][l % 16], v = 0..3,
// i.e. four consecutive features of one token, which are stored as one 8-byte
// write of the row-major [token][feature] output.
#pragma once

#include "common.h"

namespace qlora {
namespace gemm {

constexpr int BT = 256;   // tokens per tile
constexpr int BF = 128;   // features per tile
constexpr int BR = 64;    // reduction per stage
constexpr int NT = 256;   // threads

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  // raw buffer, 32-bit data format word for gfx9-family buffer instructions
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t byte_off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// element offset of 16-byte chunk `chunk` (0..7) of row `row` in a tile of `rows` rows
__device__ __forceinline__ int swz_t(int rows, int row, int chunk) {
  return (chunk >> 2) * rows * 32 + row * 32 + (((chunk & 3) ^ ((row >> 1) & 3)) << 3);
}
__device__ __forceinline__ int swzT(int row, int chunk) { return swz_t(BT, row, chunk); }
__device__ __forceinline__ int swzF(int row, int chunk) { return swz_t(BF, row, chunk); }

// Token operand: rows m0..m0+255, columns c0..c0+63 of a row-major [rows][ld] bf16
// matrix.  Thread t holds chunk t%8 of rows t/8 + 32 i.
struct TokenRegs {
  uint4 v[8];
};

__device__ __forceinline__ void load_tokens(TokenRegs& R, rsrc_t src, uint32_t ld, uint32_t m0, uint32_t c0) {
  const int t = threadIdx.x;
  const uint32_t base = ((m0 + (t >> 3)) * ld + c0 + (t & 7) * 8) * 2;
#pragma unroll
  for (int i = 0; i < 8; ++i) R.v[i] = ld16(src, base + (uint32_t)(32 * i) * ld * 2);
}

__device__ __forceinline__ void store_tokens_part(const TokenRegs& R, uint16_t* __restrict__ sT, int i) {
  const int t = threadIdx.x;
  *reinterpret_cast<uint4*>(sT + swzT((t >> 3) + 32 * i, t & 7)) = R.v[i];
}

struct Acc {
  f32x4 c[4][8];   // [feature tile][token tile]
};

__device__ __forceinline__ void acc_zero(Acc& a) {
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int m = 0; m < 8; ++m) a.c[f][m] = f32x4{0.f, 0.f, 0.f, 0.f};
}

struct Frags {
  u32x4 fa[4], tb[8];
};

// wave (wt, wf) covers tokens wt*128.., features wf*64..; ks selects 32 of the 64
__device__ __forceinline__ void read_frags(Frags& F, const uint16_t* __restrict__ sT,
                                           const uint16_t* __restrict__ sF, int ks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wt = wave & 1, wf = wave >> 1;
  const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
  for (int f = 0; f < 4; ++f)
    F.fa[f] = *reinterpret_cast<const u32x4*>(sF + swzF(wf * 64 + f * 16 + (lane & 15), chunk));
#pragma unroll
  for (int m = 0; m < 8; ++m)
    F.tb[m] = *reinterpret_cast<const u32x4*>(sT + swzT(wt * 128 + m * 16 + (lane & 15), chunk));
}

__device__ __forceinline__ void mma_group(Acc& a, const Frags& F, int f) {
#pragma unroll
  for (int m = 0; m < 8; ++m) a.c[f][m] = mfma16(F.fa[f], F.tb[m], a.c[f][m]);
}

// One 64-deep stage without interleaved work (tail stages).
__device__ __forceinline__ void mma_stage(Acc& a, const uint16_t* __restrict__ sT, const uint16_t* __restrict__ sF) {
  Frags F;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    read_frags(F, sT, sF, ks);
#pragma unroll
    for (int f = 0; f < 4; ++f) mma_group(a, F, f);
  }
}

// Store bf16(acc) into out [ntok][nfeat] row-major (nfeat % 8 == 0).
__device__ __forceinline__ void store_out(const Acc& a, uint16_t* __restrict__ out, int64_t ld, int64_t m0,
                                          int64_t ntok, int64_t f0, int64_t nfeat) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wt = wave & 1, wf = wave >> 1;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t feat = f0 + wf * 64 + f * 16 + 4 * (lane >> 4);
    if (feat >= nfeat) continue;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int64_t tok = m0 + wt * 128 + m * 16 + (lane & 15);
      if (tok >= ntok) continue;
      const f32x4 v = a.c[f][m];
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(out + tok * ld + feat) = o;
    }
  }
}

// Map a linear workgroup id to a (token tile, feature tile) pair.  Workgroups are
// dispatched round-robin over the 8 XCDs; give each XCD a contiguous run of tiles
// (token-tile major) so the tiles sharing a token panel share an L2.
__device__ __forceinline__ void tile_of(int64_t tiles_t, int64_t tiles_f, int64_t& tt, int64_t& tf) {
  const int64_t n = tiles_t * tiles_f;
  int64_t L = blockIdx.x;
  if ((n & 7) == 0) L = (L & 7) * (n >> 3) + (L >> 3);
  tt = L / tiles_f;
  tf = L - tt * tiles_f;
}

}  // namespace gemm
}  // namespace qlora
