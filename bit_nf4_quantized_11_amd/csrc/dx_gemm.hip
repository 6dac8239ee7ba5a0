// Backward input gradient ("QLoRA: Efficient Finetuning of Quantized LLMs",
// section "The QLoRA layer, end to end": the gradient passes through the frozen
// weight, which forces a second dequantization on the backward pass):
//
//   dX[M][K] = bf16( dY[M][N] deq(W) + Gs[M][rp] A~^T ),  A~(k, j) = A[k][j] (j < r), 0 otherwise
//
// with Gs = bf16(s * dY B^T) from the rank-r kernel.  The reduction runs over the
// weight's rows n, while each stored row is contiguous along k, so the
// dequantized tile is written transposed into the feature-major LDS tile
// sF[k][n] (2-byte stores).  The adapter stages need no transpose: A is [K][r].
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace qlora {

namespace {

using namespace gemm;

struct DxParams {
  const uint16_t* dY;
  int64_t M, K, N;
  NF4View w;
  const uint16_t* Gs;
  int64_t rp;
  const uint16_t* A;
  int64_t r;
  uint16_t* dX;
  NF4Table tab;
};

struct FeatRegs {
  uint4 code;      // NF4 stage: 32 codes of one row (half a block)
  float scale;
  uint4 a[4];      // adapter stage: 32 values of one row of A
};

__global__ __launch_bounds__(NT) void k_bwd_dx_nf4_gemm(DxParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sT[2][BT * BR];
  __shared__ __attribute__((aligned(16))) uint16_t sF[2][BF * BR];

  int64_t tt, tf;
  tile_of((p.M + BT - 1) / BT, (p.K + BF - 1) / BF, tt, tf);
  const int64_t m0 = tt * BT, k0 = tf * BF;
  const int64_t nkb = p.K / 64;                 // blocks per weight row
  const int64_t nred = (p.N + 63) / 64;         // reduction stages over the weight rows
  const int64_t niter = nred + p.rp / 64;
  const int t = threadIdx.x;

  TokenRegs TR;
  FeatRegs FR;

  // NF4 stage mapping: row n_local = t/4 (0..63), block (k0/64 + (t/2)%2), half t%2
  auto load = [&](int64_t it) {
    if (it < nred) {
      const int64_t nr0 = it * 64;
      load_tokens(TR, p.dY, p.N, m0, p.M, nr0, p.N);
      const int row = t >> 2, bsel = (t >> 1) & 1, half = t & 1;
      const int64_t n = nr0 + row;
      const int64_t kb = k0 / 64 + bsel;
      FR.code = make_uint4(0, 0, 0, 0);
      FR.scale = 0.0f;
      if (n < p.N && kb < nkb) {
        const int64_t blk = n * nkb + kb;
        FR.code = *reinterpret_cast<const uint4*>(p.w.codes + blk * kBlockBytes + half * 16);
        FR.scale = block_scale(p.w, blk);
      }
    } else {
      const int64_t j0 = (it - nred) * 64;
      load_tokens(TR, p.Gs, p.rp, m0, p.M, j0, p.rp);
      const int kr = t >> 1, jc = (t & 1) * 32;
      const int64_t k = k0 + kr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        FR.a[q] = make_uint4(0, 0, 0, 0);
        const int64_t j = j0 + jc + q * 8;
        if (k < p.K && j < p.r) FR.a[q] = *reinterpret_cast<const uint4*>(p.A + k * p.r + j);
      }
    }
  };

  auto store = [&](int64_t it, int buf) {
    store_tokens(TR, sT[buf]);
    if (it < nred) {
      const int row = t >> 2, bsel = (t >> 1) & 1, half = t & 1;
      const Planes pl = make_planes(p.tab, FR.scale);
      const uint32_t cw[4] = {FR.code.x, FR.code.y, FR.code.z, FR.code.w};
      const int kl0 = bsel * 64 + half * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = dequant8(pl, cw[q]);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kl = kl0 + q * 8 + e;
          const uint16_t h = (uint16_t)((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xFFFFu));
          sF[buf][swz(kl, row >> 3) + (row & 7)] = h;
        }
      }
    } else {
      const int kr = t >> 1, jc = (t & 1) * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint4*>(sF[buf] + swz(kr, (jc >> 3) + q)) = FR.a[q];
    }
  };

  Acc acc;
  acc_zero(acc);
  load(0);
  store(0, 0);
  __syncthreads();
  for (int64_t it = 0; it < niter; ++it) {
    const int buf = (int)(it & 1);
    if (it + 1 < niter) load(it + 1);
    mma_stage(acc, sT[buf], sF[buf]);
    if (it + 1 < niter) store(it + 1, buf ^ 1);
    __syncthreads();
  }
  store_out(acc, p.dX, p.K, m0, p.M, k0, p.K);
}

}  // namespace

hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const NF4View& w,
                          const uint16_t* Gs, int64_t rp, const uint16_t* A, int64_t r, uint16_t* dX,
                          hipStream_t s) {
  DxParams p{dY, M, K, N, w, Gs, rp, A, r, dX, nf4_table()};
  const int64_t tiles = ((M + BT - 1) / BT) * ((K + BF - 1) / BF);
  ProfScope ps("k_bwd_dx_nf4_gemm", s);
  hipLaunchKernelGGL(k_bwd_dx_nf4_gemm, dim3((unsigned)tiles), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
