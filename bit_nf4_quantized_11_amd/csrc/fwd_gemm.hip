// Fused forward for large token counts ("QLoRA: Efficient Finetuning of Quantized
// LLMs", section "The QLoRA layer, end to end": every product runs in bf16 on a
// weight decoded from its 4-bit storage, and no bf16 copy of the weight is kept;
// y = x W + s (x L1) L2):
//
//   Y[M][N] = bf16( X[M][K] deq(W)^T + Ts[M][rp] B~ ),   B~(j, n) = B[j][n] (j < r), 0 otherwise
//
// Ts = bf16(s * X A) comes from the rank-r kernel.  The K/64 NF4 stages are
// followed by rp/64 adapter stages that accumulate into the same registers, so
// one bf16 rounding ends the whole sum.  In an NF4 stage each thread dequantizes a
// quarter of one 64-weight block (the block's scaled 16-entry table is built by the
// four threads of the block together, the lookups are byte permutes) straight into
// the LDS feature tile.
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
  // split mode: K-slices of `spl` stages, fp32 partials [split][M][npad], no adapter stages
  float* partial;
  int64_t npad;
  uint32_t spl;
};

struct WRegs {
  uint2 code;     // 16 codes (a quarter of a block)
  uint32_t c2;    // 8-bit block constant (double quant) or fp32 absmax bits
  float c1;
};

struct Stage {
  TokenRegs T;
  WRegs W;
};

// BM: 0 for blocks of 64 (one block per row per stage), 1 for 128 and 256 (a block spans
// 2 or 4 stages), 2 for 32 (two blocks per row per stage: the two halves of a quad use
// different scales, so each lane builds the whole 16-entry table itself).
// SPLIT: a workgroup covers stages [spl s, spl (s + 1)) of its tile's reduction and writes
// fp32 partial sums (few tokens: the K-slices give the GPU enough workgroups); the adapter
// term and the final sum come from the weight-streaming path's epilogue.
template <bool DQ, int BM, bool SPLIT>
__global__ __launch_bounds__(NT) void k_fwd_nf4_gemm(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  uint16_t* const sT[2] = {smem, smem + TILE_T};
  uint16_t* const sF[2] = {smem + 2 * TILE_T, smem + 2 * TILE_T + TILE_F};

  int64_t tt, tf;
  const int64_t tiles_t = (p.M + BT - 1) / BT, tiles_f = (p.N + BF - 1) / BF;
  const uint32_t split = SPLIT ? (uint32_t)(blockIdx.x / (tiles_t * tiles_f)) : 0u;
  tile_of(tiles_t, tiles_f, tt, tf, SPLIT ? (int64_t)blockIdx.x - (int64_t)split * tiles_t * tiles_f : -1);
  const uint32_t m0 = (uint32_t)(tt * BT), n0 = (uint32_t)(tf * BF);
  const uint32_t nkb_all = (uint32_t)(p.K / 64);
  const uint32_t it0 = SPLIT ? split * p.spl : 0u;                       // first stage
  const uint32_t nkb = SPLIT ? min(nkb_all, it0 + p.spl) - it0 : nkb_all;   // stages of this workgroup
  const int t = threadIdx.x;
  // weight row t/4 of the tile, quarter t%4 of its block (groups 2q and 2q+1 -> chunks
  // 2q, 2q+1 of the LDS row); rows past N read as zero (their outputs are not stored)
  const int wrow = t >> 2, wq = t & 3;
  const uint32_t wblk0 = (n0 + wrow) * nkb_all;
  const uint32_t code_off = wblk0 * kBlockBytes + wq * 8;

  const TokenSrc xs = token_src(p.X, (uint64_t)p.M * p.K * 2, (uint32_t)p.K, m0);
  const rsrc_t rC = make_rsrc(p.w.codes, p.codes_bytes);
  const rsrc_t rA = make_rsrc(p.w.absmax, p.absmax_bytes);
  const rsrc_t rC1 = make_rsrc(p.w.c1, p.c1_bytes);
  constexpr bool dq = DQ;
  const float mu = dq ? *p.w.mu : 0.0f;
  const QuadLevels lev = quad_levels(p.tab);

  const uint32_t bsh = (uint32_t)(p.w.bshift - 6);   // BM == 1: 64-chunks per block, log2
  auto load = [&](uint32_t it, Stage& S) {
    load_tokens(S.T, xs, it * 64);
    S.W.code = ld8(rC, code_off, it * kBlockBytes);
    if constexpr (BM == 0) {
      if constexpr (dq) {
        S.W.c2 = __builtin_amdgcn_raw_buffer_load_b8(rA, wblk0, it, 0);
        S.W.c1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC1, ((wblk0 + it) >> 8) * 4, 0, 0));
      } else {
        S.W.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, wblk0 * 4, it * 4, 0);
        S.W.c1 = 0.0f;
      }
    } else {
      // block of this thread's 16 weights
      const uint32_t sb = BM == 1 ? (wblk0 + it) >> bsh : ((wblk0 + it) << 1) + (uint32_t)(wq >> 1);
      if constexpr (dq) {
        S.W.c2 = __builtin_amdgcn_raw_buffer_load_b8(rA, sb, 0, 0);
        S.W.c1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC1, (sb >> 8) * 4, 0, 0));
      } else {
        S.W.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, sb * 4, 0, 0);
        S.W.c1 = 0.0f;
      }
    }
  };
  auto planes = [&](float scale) -> Planes {
    if constexpr (BM == 2)
      return make_planes(p.tab, scale);
    else
      return quad_planes(lev, scale);
  };

  auto scale_of = [&](const Stage& S) -> float {
    return dq ? __fadd_rn(__fmul_rn(e4m3_decode(S.W.c2), S.W.c1), mu) : __uint_as_float(S.W.c2);
  };
  auto put = [&](const Planes& pl, uint32_t cw, int d, int sb) {
    *reinterpret_cast<u32x4*>(sF[sb] + swzF(wrow, 2 * wq + d)) = dequant8(pl, cw);
  };

  // This wave's MFMAs of the stage in LDS buffer `cb`, with the store of stage S into
  // buffer `sb` cut into pieces between the MFMA groups.
  const int kh = wave_k();
  auto compute_store = [&](Acc& acc, int cb, const Stage& S, int sb) {
    Frags Fa, Fb;
    read_frags(Fa, sT[cb], sF[cb], 2 * kh);
    read_frags(Fb, sT[cb], sF[cb], 2 * kh + 1);
    mma_group(acc, Fa, 0);
    store_tokens_part(S.T, sT[sb], 0);
    store_tokens_part(S.T, sT[sb], 1);
    const float scale = scale_of(S);
    mma_group(acc, Fa, 1);
    store_tokens_part(S.T, sT[sb], 2);
    store_tokens_part(S.T, sT[sb], 3);
    const Planes pl = planes(scale);
    mma_group(acc, Fb, 0);
    put(pl, S.W.code.x, 0, sb);
    mma_group(acc, Fb, 1);
    put(pl, S.W.code.y, 1, sb);
    interleave_mfma_valu();
  };

  auto store_all = [&](const Stage& S, int sb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) store_tokens_part(S.T, sT[sb], i);
    const Planes pl = planes(scale_of(S));
    put(pl, S.W.code.x, 0, sb);
    put(pl, S.W.code.y, 1, sb);
  };

  Acc acc;
  acc_zero(acc);
  Stage S0, S1;
  // Prefetch loads are unconditional (a stage index past the end is clamped to the last
  // stage and the data is never stored): a load under a branch would make the compiler
  // wait for every load in flight where the branch rejoins.
  const uint32_t last = it0 + nkb - 1;
  load(it0, S0);
  load(min(it0 + 1, last), S1);
  store_all(S0, 0);
  __syncthreads();
  // two stages per trip (stage it in buffer 0 with it+1 in S1, then it+1 in buffer 1 with
  // it+2 in S0); a single exit keeps the accumulators in one register set
  uint32_t it = 0;
  for (; it + 1 < nkb; it += 2) {
    load(min(it0 + it + 2, last), S0);
    compute_store(acc, 0, S1, 1);
    __syncthreads();
    load(min(it0 + it + 3, last), S1);
    compute_store(acc, 1, S0, 0);
    __syncthreads();
  }
  if (it < nkb) {   // odd number of stages: the last one is in buffer 0
    mma_stage<false>(acc, sT[0], sF[0]);
    __syncthreads();
  }

  if constexpr (SPLIT) {
    if (combine_halves(acc, smem))
      store_out_f32(acc, p.partial + (int64_t)split * p.M * p.npad, p.npad, m0, p.M, n0, p.N);
    return;
  }

  // adapter stages: Ts [M][rp] against rows of B, kept as stored ([j][n]) in the natural
  // tile and read with transposing loads.  Rows j >= r lie past the end of B and read zero.
  const TokenSrc ts = token_src(p.Ts, (uint64_t)p.M * p.rp * 2, (uint32_t)p.rp, m0);
  const rsrc_t rB = make_rsrc(p.B, (uint64_t)p.r * p.N * 2);
  const int bj = t >> 3, be = t & 7;
  for (uint32_t j0 = 0; j0 < (uint32_t)p.rp; j0 += 64) {
    TokenRegs T;
    load_tokens(T, ts, j0);
    const uint32_t boff = ((j0 + bj) * (uint32_t)p.N + n0 + be * 16) * 2;
    const uint4 b0 = ld16(rB, boff), b1 = ld16(rB, boff + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) store_tokens_part(T, sT[0], i);
    *reinterpret_cast<uint4*>(sF[0] + swzN(bj, 2 * be)) = b0;
    *reinterpret_cast<uint4*>(sF[0] + swzN(bj, 2 * be + 1)) = b1;
    __syncthreads();
    mma_stage<true>(acc, sT[0], sF[0]);
    __syncthreads();
  }
  if (combine_halves(acc, smem)) store_out(acc, p.Y, p.N, m0, p.M, n0, p.N);
}

}  // namespace

hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w,
                           const uint16_t* Ts, int64_t rp, const uint16_t* B, int64_t r, uint16_t* Y,
                           hipStream_t s) {
  // 64-element code chunks, and blocks (one constant each; in is a multiple of the block size)
  const uint64_t nchunk = (uint64_t)N * K / 64, nblk = ((uint64_t)N * K) >> w.bshift;
  FwdParams p{X, M, K, N, w, nchunk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
              Ts, rp, B, r, Y, nf4_table(w.cb), nullptr, 0, 0};
  const int64_t tiles = ((M + BT - 1) / BT) * ((N + BF - 1) / BF);
  const int bm = w.bshift == 6 ? 0 : w.bshift > 6 ? 1 : 2;
  ProfScope ps("k_fwd_nf4_gemm", s);
  const dim3 grid((unsigned)tiles), block(NT);
  if (w.dq) {
    if (bm == 0) hipLaunchKernelGGL((k_fwd_nf4_gemm<true, 0, false>), grid, block, 0, s, p);
    else if (bm == 1) hipLaunchKernelGGL((k_fwd_nf4_gemm<true, 1, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_fwd_nf4_gemm<true, 2, false>), grid, block, 0, s, p);
  } else {
    if (bm == 0) hipLaunchKernelGGL((k_fwd_nf4_gemm<false, 0, false>), grid, block, 0, s, p);
    else if (bm == 1) hipLaunchKernelGGL((k_fwd_nf4_gemm<false, 1, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_fwd_nf4_gemm<false, 2, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_gemm_split(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w, int stages,
                                 float* partial, int64_t npad, hipStream_t s) {
  const uint64_t nchunk = (uint64_t)N * K / 64, nblk = ((uint64_t)N * K) >> w.bshift;
  const uint32_t nkb = (uint32_t)(K / 64);
  const uint32_t spl = (uint32_t)stages;
  FwdParams p{X, M, K, N, w, nchunk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
              nullptr, 0, nullptr, 0, nullptr, nf4_table(w.cb), partial, npad, spl};
  const int64_t tiles = ((M + BT - 1) / BT) * ((N + BF - 1) / BF);
  const int64_t used = (nkb + spl - 1) / spl;   // splits that get at least one stage
  ProfScope ps("k_fwd_nf4_gemm", s);
  const dim3 grid((unsigned)(tiles * used)), block(NT);
  const int bm = w.bshift == 6 ? 0 : w.bshift > 6 ? 1 : 2;
  if (w.dq) {
    if (bm == 0) hipLaunchKernelGGL((k_fwd_nf4_gemm<true, 0, true>), grid, block, 0, s, p);
    else if (bm == 1) hipLaunchKernelGGL((k_fwd_nf4_gemm<true, 1, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_fwd_nf4_gemm<true, 2, true>), grid, block, 0, s, p);
  } else {
    if (bm == 0) hipLaunchKernelGGL((k_fwd_nf4_gemm<false, 0, true>), grid, block, 0, s, p);
    else if (bm == 1) hipLaunchKernelGGL((k_fwd_nf4_gemm<false, 1, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_fwd_nf4_gemm<false, 2, true>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace qlora
