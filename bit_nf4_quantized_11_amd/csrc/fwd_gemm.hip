// Fused forward for large token counts ("QLoRA: Efficient Finetuning of Quantized
// LLMs", section "The QLoRA layer, end to end": the weight is dequantized to bf16
// on the fly, used, and thrown away; y = x W + s (x L1) L2):
//
//   Y[M][N] = bf16( X[M][K] deq(W)^T + Ts[M][rp] B~ ),   B~(j, n) = B[j][n] (j < r), 0 otherwise
//
// Ts = bf16(s * X A) comes from the rank-r kernel.  The K/64 NF4 stages are
// followed by rp/64 adapter stages that accumulate into the same registers, so
// one bf16 rounding ends the whole sum.  In an NF4 stage each thread dequantizes
// half of one 64-weight block (its 16-entry scaled table is built in registers,
// the lookups are byte permutes) straight into the LDS feature tile.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace qlora {

namespace {

using namespace gemm;

struct FwdParams {
  const uint16_t* X;
  int64_t M, K, N;
  NF4View w;
  const uint16_t* Ts;
  int64_t rp;
  const uint16_t* B;
  int64_t r;
  uint16_t* Y;
  NF4Table tab;
};

struct FeatRegs {
  uint4 code;      // NF4 stage: 32 codes (half a block)
  float scale;
  uint4 b[4];      // adapter stage: 32 values of one row of B
};

__global__ __launch_bounds__(NT) void k_fwd_nf4_gemm(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sT[2][BT * BR];
  __shared__ __attribute__((aligned(16))) uint16_t sF[2][BF * BR];

  int64_t tt, tf;
  tile_of((p.M + BT - 1) / BT, (p.N + BF - 1) / BF, tt, tf);
  const int64_t m0 = tt * BT, n0 = tf * BF;
  const int64_t nkb = p.K / 64;
  const int64_t niter = nkb + p.rp / 64;
  const int t = threadIdx.x;

  TokenRegs TR;
  FeatRegs FR;

  auto load = [&](int64_t it) {
    if (it < nkb) {
      load_tokens(TR, p.X, p.K, m0, p.M, it * 64, p.K);
      const int row = t >> 1, half = t & 1;
      const int64_t n = n0 + row;
      FR.code = make_uint4(0, 0, 0, 0);
      FR.scale = 0.0f;
      if (n < p.N) {
        const int64_t blk = n * nkb + it;
        FR.code = *reinterpret_cast<const uint4*>(p.w.codes + blk * kBlockBytes + half * 16);
        FR.scale = block_scale(p.w, blk);
      }
    } else {
      const int64_t j0 = (it - nkb) * 64;
      load_tokens(TR, p.Ts, p.rp, m0, p.M, j0, p.rp);
      const int j = t >> 2, nc = (t & 3) * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        FR.b[q] = make_uint4(0, 0, 0, 0);
        const int64_t n = n0 + nc + q * 8;
        if (j0 + j < p.r && n < p.N) FR.b[q] = *reinterpret_cast<const uint4*>(p.B + (j0 + j) * p.N + n);
      }
    }
  };

  auto store = [&](int64_t it, int buf) {
    store_tokens(TR, sT[buf]);
    if (it < nkb) {
      const int row = t >> 1, half = t & 1;
      const Planes pl = make_planes(p.tab, FR.scale);
      const uint32_t cw[4] = {FR.code.x, FR.code.y, FR.code.z, FR.code.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(sF[buf] + swz(row, half * 4 + q)) = dequant8(pl, cw[q]);
    } else {
      // transpose B rows into feature-major LDS: sF[n][j]
      const int j = t >> 2, nc = (t & 3) * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w4[4] = {FR.b[q].x, FR.b[q].y, FR.b[q].z, FR.b[q].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int n = nc + q * 8 + e;
          const uint16_t v = (uint16_t)((e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xFFFFu));
          sF[buf][swz(n, j >> 3) + (j & 7)] = v;
        }
      }
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
  store_out(acc, p.Y, p.N, m0, p.M, n0, p.N);
}

}  // namespace

hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w,
                           const uint16_t* Ts, int64_t rp, const uint16_t* B, int64_t r, uint16_t* Y,
                           hipStream_t s) {
  FwdParams p{X, M, K, N, w, Ts, rp, B, r, Y, nf4_table()};
  const int64_t tiles = ((M + BT - 1) / BT) * ((N + BF - 1) / BF);
  ProfScope ps("k_fwd_nf4_gemm", s);
  hipLaunchKernelGGL(k_fwd_nf4_gemm, dim3((unsigned)tiles), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
