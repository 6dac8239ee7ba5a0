// One split-K tile of a rank-r product, C[64][64] over a slice of the reduction, computed by a
// 512-thread workgroup of another kernel (both operands stored contiguously along the
// reduction: A(i, k) = A[i * a_si + k], B(k, j) = B[j * b_sj + k]).  Used to run the split-K
// workgroups of G = dY B^T inside the launch of the split dX GEMM, whose epilogue adds the
// partials: the same tiles, splits and partial layout as k_lora_gemm, so the sums are the
// same.  Eight waves: wave w takes the 32 x 32 quarter (w & 1, (w >> 1) & 1) of the tile for
// the reduction half w >> 2 of every 64-deep step (one v_mfma_f32_16x16x32_bf16 step), and
// the two halves are added through LDS at the end.
#pragma once

#include "gemm_core.h"
#include "kernels.h"

namespace qlora {
namespace lora_tile {

// [row][k] tile of 64 x 64 bf16 (128-byte rows of eight 16-byte chunks): chunk c of row r at
// c ^ ((r >> 1) & 7); 16 consecutive rows of one chunk (a fragment read) and 2 rows x 8 chunks
// (a store) are conflict-free.
__device__ __forceinline__ int kcpos(int row, int c) { return row * 64 + ((c ^ ((row >> 1) & 7)) << 3); }

constexpr int CH = 8;   // steps per batch of loads

// lds: at least 2 x 2 x 64 x 64 bf16 (32 KiB), 16-byte aligned.  Called by all 512 threads.
__device__ __forceinline__ void tile_kc512(const LoraProblem& P, int64_t wg, uint16_t* __restrict__ lds) {
  const SmallGemm& g = P.g;
  const int split = (int)(wg % P.splits);
  const int64_t tile = wg / P.splits;
  const int64_t ti = tile / P.tiles_j, tj = tile - ti * P.tiles_j;
  const int64_t i0 = ti * 64, j0 = tj * 64;
  const int64_t kbeg = (int64_t)split * P.k_per_split;
  const int64_t kend = min(g.K, kbeg + P.k_per_split);
  const int nsteps = (int)((kend - kbeg + 63) / 64);
  const uint64_t a_ext = (uint64_t)((g.I - 1) * g.a_si + (g.K - 1) + 1);
  const uint64_t b_ext = (uint64_t)((g.K - 1) + (g.J - 1) * g.b_sj + 1);
  const gemm::rsrc_t rA = gemm::make_rsrc(g.A, a_ext * 2), rB = gemm::make_rsrc(g.B, b_ext * 2);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wi = w & 1, wj = (w >> 1) & 1, wk = w >> 2;
  const int lr = t >> 3, lc = t & 7;   // this thread's row and 16-byte chunk of a panel
  uint16_t* const sA = lds;                 // [2][64 * 64]
  uint16_t* const sB = lds + 2 * 64 * 64;   // [2][64 * 64]
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // elements past the rows or the slice read zero (kend % 8 == 0)
  auto ld = [&](int64_t k0, uint4& va, uint4& vb) {
    const int64_t k = k0 + lc * 8;
    const bool kin = k < kend;
    va = gemm::ld16(rA, kin && i0 + lr < g.I ? (uint32_t)(((i0 + lr) * g.a_si + k) * 2) : (uint32_t)(a_ext * 2));
    vb = gemm::ld16(rB, kin && j0 + lr < g.J ? (uint32_t)(((j0 + lr) * g.b_sj + k) * 2) : (uint32_t)(b_ext * 2));
  };
  for (int c0 = 0; c0 < nsteps; c0 += CH) {
    uint4 va[CH], vb[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) ld(kbeg + (int64_t)(c0 + q) * 64, va[q], vb[q]);
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (c0 + q >= nsteps) break;   // workgroup-uniform
      const int cb = q & 1;
      *reinterpret_cast<uint4*>(sA + cb * 4096 + kcpos(lr, lc)) = va[q];
      *reinterpret_cast<uint4*>(sB + cb * 4096 + kcpos(lr, lc)) = vb[q];
      __syncthreads();
      u32x4 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *reinterpret_cast<const u32x4*>(sA + cb * 4096 + kcpos(wi * 32 + a * 16 + (lane & 15), wk * 4 + (lane >> 4)));
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bfr[b] = *reinterpret_cast<const u32x4*>(sB + cb * 4096 + kcpos(wj * 32 + b * 16 + (lane & 15), wk * 4 + (lane >> 4)));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
    }
  }
  // waves 4..7 hand their reduction half to waves 0..3 (the LDS tiles are free after a barrier),
  // which add it (lower half first) and store the partial tile:
  // acc[a][b][v] = C[wi*32 + a*16 + 4*(lane/16) + v][wj*32 + b*16 + lane%16]
  __syncthreads();
  f32x4* const x = reinterpret_cast<f32x4*>(lds);
  if (wk) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) x[((w & 3) * 4 + a * 2 + b) * 64 + lane] = acc[a][b];
  }
  __syncthreads();
  if (!wk) {
    float* const part = P.partial + (tile * P.splits + split) * 4096;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const f32x4 o = x[(w * 4 + a * 2 + b) * 64 + lane];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          part[(wi * 32 + a * 16 + 4 * (lane >> 4) + v) * 64 + wj * 32 + b * 16 + (lane & 15)] =
              __fadd_rn(acc[a][b][v], o[v]);
      }
  }
}

}  // namespace lora_tile
}  // namespace qlora
