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
  uint64_t codes_bytes, absmax_bytes, c1_bytes;
  const uint16_t* Gs;
  int64_t rp;
  const uint16_t* A;
  int64_t r;
  uint16_t* dX;
  NF4Table tab;
};

struct WRegs {
  uint4 code;     // 32 codes: half of block (n, kb)
  uint32_t c2;
  float c1;
  uint32_t live;  // the weight row exists (n < N)
};

struct Stage {
  TokenRegs T;
  WRegs W;
};

template <bool DQ>
__global__ __launch_bounds__(NT) void k_bwd_dx_nf4_gemm(DxParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sT[2][BT * BR];
  __shared__ __attribute__((aligned(16))) uint16_t sF[2][BF * BR];

  int64_t tt, tf;
  tile_of((p.M + BT - 1) / BT, (p.K + BF - 1) / BF, tt, tf);
  const uint32_t m0 = (uint32_t)(tt * BT), k0 = (uint32_t)(tf * BF);
  const uint32_t nkb = (uint32_t)(p.K / 64);
  const uint32_t N = (uint32_t)p.N;
  const uint32_t nred = (N + 63) / 64;   // reduction stages over the weight rows
  const int t = threadIdx.x;
  // NF4 stage mapping: weight row t/4 of the stage, block k0/64 + (t/2)%2, half t%2
  const int wrow = t >> 2, wbsel = (t >> 1) & 1, whalf = t & 1;
  const uint32_t wkb = k0 / 64 + wbsel;
  const int kl0 = wbsel * 64 + whalf * 32;   // first feature row of this thread in sF

  const rsrc_t rD = make_rsrc(p.dY, (uint64_t)p.M * p.N * 2);
  const rsrc_t rC = make_rsrc(p.w.codes, p.codes_bytes);
  const rsrc_t rA = make_rsrc(p.w.absmax, p.absmax_bytes);
  const rsrc_t rC1 = make_rsrc(p.w.c1, p.c1_bytes);
  constexpr bool dq = DQ;
  const float mu = dq ? *p.w.mu : 0.0f;

  auto load = [&](uint32_t it, Stage& S) {
    load_tokens(S.T, rD, N, m0, it * 64);
    const uint32_t n = it * 64 + wrow;
    const uint32_t blk = n * nkb + wkb;
    S.W.code = ld16(rC, blk * kBlockBytes + whalf * 16);
    if constexpr (dq) {
      S.W.c2 = __builtin_amdgcn_raw_buffer_load_b8(rA, blk, 0, 0);
      S.W.c1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC1, (blk >> 8) * 4, 0, 0));
    } else {
      S.W.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, blk * 4, 0, 0);
      S.W.c1 = 0.0f;
    }
    S.W.live = n < N;
  };

  // rows past the last weight row must contribute exact zeros (the token operand there
  // holds the next token row's values): code 7 is the exact-zero level, scale 0
  auto scale_of = [&](const Stage& S) -> float {
    const float s = dq ? __fadd_rn(__fmul_rn(e4m3_decode(S.W.c2), S.W.c1), mu) : __uint_as_float(S.W.c2);
    return S.W.live ? s : 0.0f;
  };
  auto codes_of = [&](const Stage& S, uint32_t q) -> uint32_t {
    const uint32_t c = q == 0 ? S.W.code.x : q == 1 ? S.W.code.y : q == 2 ? S.W.code.z : S.W.code.w;
    return S.W.live ? c : 0x77777777u;
  };
  // dequantize 8 weights (k = kl0 + 8q .. +7 of row wrow) and write them transposed
  auto put8 = [&](const Planes& pl, uint32_t cw, int q, int sb) {
    const u32x4 v = dequant8(pl, cw);
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kl = kl0 + q * 8 + e;
      sF[sb][swzF(kl, wrow >> 3) + (wrow & 7)] = (uint16_t)((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xFFFFu));
    }
  };

  auto compute_store = [&](Acc& acc, int cb, const Stage& S, int sb) {
    Frags F;
    Planes pl;
    read_frags(F, sT[cb], sF[cb], 0);
    mma_group(acc, F, 0);
    store_tokens_part(S.T, sT[sb], 0);
    store_tokens_part(S.T, sT[sb], 1);
    const float scale = scale_of(S);
    mma_group(acc, F, 1);
    store_tokens_part(S.T, sT[sb], 2);
    store_tokens_part(S.T, sT[sb], 3);
    pl = make_planes(p.tab, scale);
    mma_group(acc, F, 2);
    store_tokens_part(S.T, sT[sb], 4);
    store_tokens_part(S.T, sT[sb], 5);
    put8(pl, codes_of(S, 0), 0, sb);
    mma_group(acc, F, 3);
    store_tokens_part(S.T, sT[sb], 6);
    store_tokens_part(S.T, sT[sb], 7);
    put8(pl, codes_of(S, 1), 1, sb);
    read_frags(F, sT[cb], sF[cb], 1);
    mma_group(acc, F, 0);
    put8(pl, codes_of(S, 2), 2, sb);
    mma_group(acc, F, 1);
    put8(pl, codes_of(S, 3), 3, sb);
    mma_group(acc, F, 2);
    mma_group(acc, F, 3);
  };

  auto store_all = [&](const Stage& S, int sb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) store_tokens_part(S.T, sT[sb], i);
    const Planes pl = make_planes(p.tab, scale_of(S));
#pragma unroll
    for (int q = 0; q < 4; ++q) put8(pl, codes_of(S, q), q, sb);
  };

  Acc acc;
  acc_zero(acc);
  Stage S0 = {}, S1 = {};
  load(0, S0);
  if (nred > 1) load(1, S1);
  store_all(S0, 0);
  __syncthreads();
  // two stages per trip (stage it in buffer 0 with it+1 in S1, then it+1 in buffer 1 with
  // it+2 in S0); a single exit keeps the accumulators in one register set
  uint32_t it = 0;
  for (; it + 1 < nred; it += 2) {
    if (it + 2 < nred) load(it + 2, S0);
    compute_store(acc, 0, S1, 1);
    __syncthreads();
    if (it + 3 < nred) load(it + 3, S1);
    compute_store(acc, 1, S0, 0);
    __syncthreads();
  }
  if (it < nred) {   // odd number of stages: the last one is in buffer 0
    mma_stage(acc, sT[0], sF[0]);
    __syncthreads();
  }

  // adapter stages: Gs [M][rp] against A rows (already feature-major: A is [K][r])
  const rsrc_t rG = make_rsrc(p.Gs, (uint64_t)p.M * p.rp * 2);
  const rsrc_t rAd = make_rsrc(p.A, (uint64_t)p.K * p.r * 2);
  for (uint32_t j0 = 0; j0 < (uint32_t)p.rp; j0 += 64) {
    TokenRegs T;
    load_tokens(T, rG, (uint32_t)p.rp, m0, j0);
    const int kr = t >> 1, jc = (t & 1) * 32;
    uint4 a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = ld16(rAd, ((k0 + kr) * (uint32_t)p.r + j0 + jc + q * 8) * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) store_tokens_part(T, sT[0], i);
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(sF[0] + swzF(kr, (jc >> 3) + q)) = a[q];
    __syncthreads();
    mma_stage(acc, sT[0], sF[0]);
    __syncthreads();
  }
  store_out(acc, p.dX, p.K, m0, p.M, k0, p.K);
}

}  // namespace

hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const NF4View& w,
                          const uint16_t* Gs, int64_t rp, const uint16_t* A, int64_t r, uint16_t* dX,
                          hipStream_t s) {
  const uint64_t nblk = (uint64_t)N * K / 64;
  DxParams p{dY, M, K, N, w, nblk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
             Gs, rp, A, r, dX, nf4_table()};
  const int64_t tiles = ((M + BT - 1) / BT) * ((K + BF - 1) / BF);
  ProfScope ps("k_bwd_dx_nf4_gemm", s);
  if (w.dq)
    hipLaunchKernelGGL(k_bwd_dx_nf4_gemm<true>, dim3((unsigned)tiles), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(k_bwd_dx_nf4_gemm<false>, dim3((unsigned)tiles), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace qlora
