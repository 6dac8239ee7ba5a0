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
  uint64_t codes_bytes, absmax_bytes, c1_bytes;
  const uint16_t* Ts;
  int64_t rp;
  const uint16_t* B;
  int64_t r;
  uint16_t* Y;
  NF4Table tab;
};

struct WRegs {
  uint4 code;     // 32 codes (half a block)
  uint32_t c2;    // 8-bit block constant (double quant) or fp32 absmax bits
  float c1;
};

struct Stage {
  TokenRegs T;
  WRegs W;
};

template <bool DQ>
__global__ __launch_bounds__(NT) void k_fwd_nf4_gemm(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sT[2][BT * BR];
  __shared__ __attribute__((aligned(16))) uint16_t sF[2][BF * BR];

  int64_t tt, tf;
  tile_of((p.M + BT - 1) / BT, (p.N + BF - 1) / BF, tt, tf);
  const uint32_t m0 = (uint32_t)(tt * BT), n0 = (uint32_t)(tf * BF);
  const uint32_t nkb = (uint32_t)(p.K / 64);
  const int t = threadIdx.x;
  const int wrow = t >> 1, whalf = t & 1;
  const uint32_t wblk0 = (n0 + wrow) * nkb;   // first block of this thread's weight row

  const rsrc_t rX = make_rsrc(p.X, (uint64_t)p.M * p.K * 2);
  const rsrc_t rC = make_rsrc(p.w.codes, p.codes_bytes);
  const rsrc_t rA = make_rsrc(p.w.absmax, p.absmax_bytes);
  const rsrc_t rC1 = make_rsrc(p.w.c1, p.c1_bytes);
  constexpr bool dq = DQ;
  const float mu = dq ? *p.w.mu : 0.0f;

  auto load = [&](uint32_t it, Stage& S) {
    load_tokens(S.T, rX, (uint32_t)p.K, m0, it * 64);
    const uint32_t blk = wblk0 + it;
    S.W.code = ld16(rC, blk * kBlockBytes + whalf * 16);
    if constexpr (dq) {
      S.W.c2 = __builtin_amdgcn_raw_buffer_load_b8(rA, blk, 0, 0);
      S.W.c1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC1, (blk >> 8) * 4, 0, 0));
    } else {
      S.W.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, blk * 4, 0, 0);
      S.W.c1 = 0.0f;
    }
  };

  // MFMAs of the stage in LDS buffer `cb`, with the store of stage S into buffer `sb`
  // cut into pieces between the MFMA groups.
  auto compute_store = [&](Acc& acc, int cb, const Stage& S, int sb) {
    Frags F;
    Planes pl;
    const uint32_t cw[4] = {S.W.code.x, S.W.code.y, S.W.code.z, S.W.code.w};
    read_frags(F, sT[cb], sF[cb], 0);
    // piece 0
    mma_group(acc, F, 0);
    store_tokens_part(S.T, sT[sb], 0);
    store_tokens_part(S.T, sT[sb], 1);
    const float scale = dq ? __fadd_rn(__fmul_rn(e4m3_decode(S.W.c2), S.W.c1), mu) : __uint_as_float(S.W.c2);
    // piece 1
    mma_group(acc, F, 1);
    store_tokens_part(S.T, sT[sb], 2);
    store_tokens_part(S.T, sT[sb], 3);
    pl = make_planes(p.tab, scale);
    // piece 2
    mma_group(acc, F, 2);
    store_tokens_part(S.T, sT[sb], 4);
    store_tokens_part(S.T, sT[sb], 5);
    *reinterpret_cast<u32x4*>(sF[sb] + swzF(wrow, whalf * 4 + 0)) = dequant8(pl, cw[0]);
    // piece 3
    mma_group(acc, F, 3);
    store_tokens_part(S.T, sT[sb], 6);
    store_tokens_part(S.T, sT[sb], 7);
    *reinterpret_cast<u32x4*>(sF[sb] + swzF(wrow, whalf * 4 + 1)) = dequant8(pl, cw[1]);
    read_frags(F, sT[cb], sF[cb], 1);
    // piece 4
    mma_group(acc, F, 0);
    *reinterpret_cast<u32x4*>(sF[sb] + swzF(wrow, whalf * 4 + 2)) = dequant8(pl, cw[2]);
    // piece 5
    mma_group(acc, F, 1);
    *reinterpret_cast<u32x4*>(sF[sb] + swzF(wrow, whalf * 4 + 3)) = dequant8(pl, cw[3]);
    // pieces 6, 7
    mma_group(acc, F, 2);
    mma_group(acc, F, 3);
  };

  auto store_all = [&](const Stage& S, int sb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) store_tokens_part(S.T, sT[sb], i);
    const float scale = dq ? __fadd_rn(__fmul_rn(e4m3_decode(S.W.c2), S.W.c1), mu) : __uint_as_float(S.W.c2);
    const Planes pl = make_planes(p.tab, scale);
    const uint32_t cw[4] = {S.W.code.x, S.W.code.y, S.W.code.z, S.W.code.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(sF[sb] + swzF(wrow, whalf * 4 + q)) = dequant8(pl, cw[q]);
  };

  Acc acc;
  acc_zero(acc);
  Stage S0 = {}, S1 = {};
  load(0, S0);
  if (nkb > 1) load(1, S1);
  store_all(S0, 0);
  __syncthreads();
  // two stages per trip (stage it in buffer 0 with it+1 in S1, then it+1 in buffer 1 with
  // it+2 in S0); a single exit keeps the accumulators in one register set
  uint32_t it = 0;
  for (; it + 1 < nkb; it += 2) {
    if (it + 2 < nkb) load(it + 2, S0);
    compute_store(acc, 0, S1, 1);
    __syncthreads();
    if (it + 3 < nkb) load(it + 3, S1);
    compute_store(acc, 1, S0, 0);
    __syncthreads();
  }
  if (it < nkb) {   // odd number of stages: the last one is in buffer 0
    mma_stage(acc, sT[0], sF[0]);
    __syncthreads();
  }

  // adapter stages: Ts [M][rp] against B rows (transposed into the feature-major tile)
  const rsrc_t rTs = make_rsrc(p.Ts, (uint64_t)p.M * p.rp * 2);
  const rsrc_t rB = make_rsrc(p.B, (uint64_t)p.r * p.N * 2);
  for (uint32_t j0 = 0; j0 < (uint32_t)p.rp; j0 += 64) {
    TokenRegs T;
    load_tokens(T, rTs, (uint32_t)p.rp, m0, j0);
    const int j = t >> 2, nc = (t & 3) * 32;
    uint4 b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = ld16(rB, ((j0 + j) * (uint32_t)p.N + n0 + nc + q * 8) * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) store_tokens_part(T, sT[0], i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w4[4] = {b[q].x, b[q].y, b[q].z, b[q].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = nc + q * 8 + e;
        sF[0][swzF(n, j >> 3) + (j & 7)] = (uint16_t)((e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xFFFFu));
      }
    }
    __syncthreads();
    mma_stage(acc, sT[0], sF[0]);
    __syncthreads();
  }
  store_out(acc, p.Y, p.N, m0, p.M, n0, p.N);
}

}  // namespace

hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w,
                           const uint16_t* Ts, int64_t rp, const uint16_t* B, int64_t r, uint16_t* Y,
                           hipStream_t s) {
  const uint64_t nblk = (uint64_t)N * K / 64;
  FwdParams p{X, M, K, N, w, nblk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
              Ts, rp, B, r, Y, nf4_table()};
  const int64_t tiles = ((M + BT - 1) / BT) * ((N + BF - 1) / BF);
  ProfScope ps("k_fwd_nf4_gemm", s);
  if (w.dq)
    hipLaunchKernelGGL(k_fwd_nf4_gemm<true>, dim3((unsigned)tiles), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(k_fwd_nf4_gemm<false>, dim3((unsigned)tiles), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
