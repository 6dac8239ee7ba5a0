// Shared pieces of the two large-M dequantizing GEMMs (forward Y and backward dX).
//
// Both compute a [256 tokens] x [128 features] output tile per workgroup of 256
// threads (4 waves, each 128 tokens x 64 features) with v_mfma_f32_16x16x32_bf16,
// reducing over 64 at a time through a double-buffered LDS stage:
//   sT  [256][64]  token operand (X or dY, or the adapter activations), bf16
//   sF  [128][64]  feature operand (dequantized weight, or the adapter factor), bf16
// Rows of both are 64 bf16 = eight 16-byte chunks; chunk c of row r is stored at
// chunk position c ^ (r & 7), so the 16 rows read by one MFMA fragment fall in
// distinct banks.
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

__device__ __forceinline__ int swz(int row, int chunk) { return row * BR + ((chunk ^ (row & 7)) << 3); }

// Token operand stage: rows m0..m0+255, reduction columns c0..c0+63 of a row-major
// [rows][ld] bf16 matrix; rows >= nrows and columns >= ncols read as zero
// (ncols % 8 == 0).  Thread t loads chunk t%8 of rows t/8 + 32 i.
struct TokenRegs {
  uint4 v[8];
};

__device__ __forceinline__ void load_tokens(TokenRegs& R, const uint16_t* __restrict__ P, int64_t ld, int64_t m0,
                                            int64_t nrows, int64_t c0, int64_t ncols) {
  const int t = threadIdx.x;
  const int c = t & 7;
  const int64_t col = c0 + c * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + (t >> 3) + 32 * i;
    R.v[i] = make_uint4(0, 0, 0, 0);
    if (row < nrows && col < ncols) R.v[i] = *reinterpret_cast<const uint4*>(P + row * ld + col);
  }
}

__device__ __forceinline__ void store_tokens(const TokenRegs& R, uint16_t* __restrict__ sT) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(sT + swz((t >> 3) + 32 * i, t & 7)) = R.v[i];
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

// One 64-deep stage: wave (wt, wf) covers tokens wt*128.., features wf*64..
__device__ __forceinline__ void mma_stage(Acc& a, const uint16_t* __restrict__ sT, const uint16_t* __restrict__ sF) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wt = wave & 1, wf = wave >> 1;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int chunk = ks * 4 + (lane >> 4);
    u32x4 fa[4], tb[8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
      fa[f] = *reinterpret_cast<const u32x4*>(sF + swz(wf * 64 + f * 16 + (lane & 15), chunk));
#pragma unroll
    for (int m = 0; m < 8; ++m)
      tb[m] = *reinterpret_cast<const u32x4*>(sT + swz(wt * 128 + m * 16 + (lane & 15), chunk));
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int m = 0; m < 8; ++m) a.c[f][m] = mfma16(fa[f], tb[m], a.c[f][m]);
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
