// Backward input gradient ("QLoRA: Efficient Finetuning of Quantized LLMs",
// section "The QLoRA layer, end to end": the input gradient is a product with the
// transposed frozen weight, so the 4-bit weight is decoded a second time in the backward):
//
//   dX[M][K] = bf16( dY[M][N] deq(W) + Gs[M][rp] A~^T ),  A~(k, j) = A[k][j] (j < r), 0 otherwise
//
// with Gs = bf16(s * dY B^T) from the rank-r kernel.  The reduction runs over the
// weight's rows n while each stored row is contiguous along k, so a stage (64 weight
// rows x 128 columns) is dequantized into the natural LDS tile as stored and the
// MFMA operand is gathered with transposing LDS reads.  The adapter stages use the
// feature-major tile: A is [K][r].
//
// Split mode (few tokens, few column tiles): a workgroup covers a slice of the reduction
// stages, skips the adapter stages and writes fp32 partials; k_dx_split_epilogue sums the
// slices in order, adds Gs A~^T and rounds once.  When the rank-r kernel left G as split-K
// partials, the epilogue also forms Gs from them (no reduce launch) and stores it for dA.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"
#include "lora_tile.h"

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
  // split mode: slices of `spl` stages, fp32 partials [split][M][K], no adapter stages
  float* partial;
  uint32_t spl;
  // split mode: the first nlora workgroups compute the split-K partials of G = dY B^T instead
  LoraProblem lg;
  int nlora;
};

struct WRegs {
  uint2 code;     // 16 codes: a quarter of block (n, kb)
  uint32_t c2;
  float c1;
};

struct Stage {
  TokenRegs T;
  WRegs W;
};

// RAGGED: N % 64 != 0, the last stage's token columns past N are masked to zero.
// BM: 0 for blocks of 64, 1 for 128 and 256 (a block spans two or four 64-column
// halves of a row), 2 for 32 (two blocks per quad: each lane builds its own table).
template <bool DQ, bool RAGGED, int BM, bool SPLIT>
__global__ __launch_bounds__(NT) void k_bwd_dx_nf4_gemm(DxParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
  uint16_t* const sT[2] = {smem, smem + TILE_T};
  uint16_t* const sF[2] = {smem + 2 * TILE_T, smem + 2 * TILE_T + TILE_F};

  int64_t bid = blockIdx.x;
  if constexpr (SPLIT) {
    // the first nlora workgroups compute G's partials (independent of the dX slices: the
    // epilogue adds both; measured, placing them after the dX workgroups is slower)
    if (bid < p.nlora) {
      lora_tile::tile_kc512(p.lg, bid, smem);
      return;
    }
    bid -= p.nlora;
  }
  const int64_t tiles_t = (p.M + BT - 1) / BT, tiles_f = (p.K + BF - 1) / BF;
  const uint32_t split = SPLIT ? (uint32_t)(bid / (tiles_t * tiles_f)) : 0u;
  int64_t tt, tf;
  tile_of(tiles_t, tiles_f, tt, tf, SPLIT ? bid - (int64_t)split * tiles_t * tiles_f : -1);
  const uint32_t m0 = (uint32_t)(tt * BT), k0 = (uint32_t)(tf * BF);
  const uint32_t nkb = (uint32_t)(p.K / 64);
  const uint32_t N = (uint32_t)p.N;
  const uint32_t nred_all = (N + 63) / 64;   // reduction stages over the weight rows
  const uint32_t it0 = SPLIT ? split * p.spl : 0u;                            // first stage
  const uint32_t nred = SPLIT ? min(nred_all, it0 + p.spl) - it0 : nred_all;   // stages of this workgroup
  const int t = threadIdx.x;
  // NF4 stage mapping: weight row t/8 of the stage, block k0/64 + b (b = (t/4)%2), quarter
  // q = t%4 (groups 2q, 2q+1 -> chunks 8b+2q, 8b+2q+1 of the natural row).  Rows past N
  // read as zero codes and scale mu; the token operand is zero there.  Columns past K
  // belong to outputs that are not stored.
  const int wrow = t >> 3, wb = (t >> 2) & 1, wq = t & 3;
  const uint32_t wblk0 = (uint32_t)wrow * nkb + k0 / 64 + wb;   // block of this thread in stage 0
  const uint32_t stage_blks = 64 * nkb;                          // blocks per 64-row stage

  const TokenSrc ds = token_src(p.dY, (uint64_t)p.M * p.N * 2, N, m0);
  const rsrc_t rC = make_rsrc(p.w.codes, p.codes_bytes);
  const rsrc_t rA = make_rsrc(p.w.absmax, p.absmax_bytes);
  const rsrc_t rC1 = make_rsrc(p.w.c1, p.c1_bytes);
  constexpr bool dq = DQ;
  const float mu = dq ? *p.w.mu : 0.0f;
  const QuadLevels lev = quad_levels(p.tab);

  const uint32_t bsh = (uint32_t)(p.w.bshift - 6);   // BM == 1: 64-chunks per block, log2
  auto load = [&](uint32_t it, Stage& S) {
    if constexpr (RAGGED)
      load_tokens_edge(S.T, ds, it * 64, N);
    else
      load_tokens(S.T, ds, it * 64);
    const uint32_t blk = wblk0 + it * stage_blks;   // 64-element chunk of this thread's weights
    S.W.code = ld8(rC, blk * kBlockBytes + wq * 8);
    // block of this thread's 16 weights
    const uint32_t sb = BM == 0 ? blk : BM == 1 ? blk >> bsh : (blk << 1) + (uint32_t)(wq >> 1);
    if constexpr (dq) {
      S.W.c2 = __builtin_amdgcn_raw_buffer_load_b8(rA, sb, 0, 0);
      S.W.c1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC1, (sb >> 8) * 4, 0, 0));
    } else {
      S.W.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, sb * 4, 0, 0);
      S.W.c1 = 0.0f;
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
    *reinterpret_cast<u32x4*>(sF[sb] + swzN(wrow, 8 * wb + 2 * wq + d)) = dequant8(pl, cw);
  };

  const int kh = wave_k();
  auto compute_store = [&](Acc& acc, int cb, const Stage& S, int sb) {
    Frags Fa, Fb;
    read_frags_natural(Fa, sT[cb], sF[cb], 2 * kh);
    read_frags_natural(Fb, sT[cb], sF[cb], 2 * kh + 1);
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
  const uint32_t last = it0 + nred - 1;
  load(it0, S0);
  load(min(it0 + 1, last), S1);
  store_all(S0, 0);
  __syncthreads();
  // two stages per trip (stage it in buffer 0 with it+1 in S1, then it+1 in buffer 1 with
  // it+2 in S0); a single exit keeps the accumulators in one register set
  uint32_t it = 0;
  for (; it + 1 < nred; it += 2) {
    load(min(it0 + it + 2, last), S0);
    compute_store(acc, 0, S1, 1);
    __syncthreads();
    load(min(it0 + it + 3, last), S1);
    compute_store(acc, 1, S0, 0);
    __syncthreads();
  }
  if (it < nred) {   // odd number of stages: the last one is in buffer 0
    mma_stage<true>(acc, sT[0], sF[0]);
    __syncthreads();
  }

  if constexpr (SPLIT) {
    if (combine_halves(acc, smem))
      store_out_f32(acc, p.partial + (int64_t)split * p.M * p.K, p.K, m0, p.M, k0, p.K);
    return;
  }

  // adapter stages: Gs [M][rp] against rows of A (feature-major: A is [K][r]).  Columns
  // j >= r of a row of A hold the next row's values; Gs is zero there.
  const TokenSrc gs = token_src(p.Gs, (uint64_t)p.M * p.rp * 2, (uint32_t)p.rp, m0);
  const rsrc_t rAd = make_rsrc(p.A, (uint64_t)p.K * p.r * 2);
  for (uint32_t j0 = 0; j0 < (uint32_t)p.rp; j0 += 64) {
    TokenRegs T;
    load_tokens(T, gs, j0);
    const uint32_t aoff = ((k0 + wrow * 2 + wb) * (uint32_t)p.r + j0 + wq * 16) * 2;
    const uint4 a0 = ld16(rAd, aoff), a1 = ld16(rAd, aoff + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) store_tokens_part(T, sT[0], i);
    *reinterpret_cast<uint4*>(sF[0] + swzF(wrow * 2 + wb, 2 * wq)) = a0;
    *reinterpret_cast<uint4*>(sF[0] + swzF(wrow * 2 + wb, 2 * wq + 1)) = a1;
    __syncthreads();
    mma_stage<false>(acc, sT[0], sF[0]);
    __syncthreads();
  }
  if (combine_halves(acc, smem)) store_out(acc, p.dX, p.K, m0, p.M, k0, p.K);
}

// dX[m][i] = bf16( sum over slices of partial[slice][m][i] + sum_{j<r} Gs[m][j] A[i][j] ):
// the split GEMM's slices in order, then the adapter term, rounded once.  A workgroup
// covers 64 columns i of one 16-token group (blockIdx.y); thread t takes column t % 64 for
// the tokens t / 64 + 4 q of the group.  Rows i0..i0+63 of A are one contiguous run of
// 64 r values: loaded coalesced and kept transposed in LDS ([j][64]); the group's rows of
// Gs are kept as fp32.  All loads are issued before any is used.
// Sums over the (at most 16) tokens of one group for the adapter gradients: thread t keeps the
// 16 token values of its column of one operand in registers (zero past the group) and reads the
// other operand's 16 values as four broadcast 16-byte LDS reads from a transposed [row][16]
// tile; the tokens are added in order.
__device__ __forceinline__ float dot16(const float* __restrict__ row16, const float (&v)[16]) {
  float sum = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 a = *reinterpret_cast<const float4*>(row16 + 4 * q);
    sum = __builtin_fmaf(a.x, v[4 * q + 0], sum);
    sum = __builtin_fmaf(a.y, v[4 * q + 1], sum);
    sum = __builtin_fmaf(a.z, v[4 * q + 2], sum);
    sum = __builtin_fmaf(a.w, v[4 * q + 3], sum);
  }
  return sum;
}

// dB[j][o0 + oo] = fl32(s * sum_m T[m][j] dY[m][o0 + oo]) for j < r: T transposed in LDS
// ([j][16]), each thread one column oo (its 16 dY values in registers) and the rows j of its
// wave, consecutive threads on consecutive columns.
__device__ __forceinline__ void grad_dB_block(const GradFold& g, int64_t M, int64_t r, int64_t o0, float* sTt,
                                              float* sY) {
  const int t = threadIdx.x;
  const int Mg = (int)M;
  // every load is issued before the first LDS store: T (at most 16 x 256 values, 16 per
  // thread) and the 16 x 64 values of dY (4 per thread)
  uint16_t tv[16], yv[4];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = t + 256 * k, m = e / (int)r;
    tv[k] = e < 16 * (int)r && m < Mg ? g.T[e] : (uint16_t)0;   // T[m][j] at m r + j = e
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = t + 256 * k, m = e >> 6, oo = e & 63;
    yv[k] = m < Mg && o0 + oo < g.N ? g.dY[m * g.N + o0 + oo] : (uint16_t)0;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int e = t + 256 * k, m = e / (int)r, j = e - m * (int)r;
    if (e < 16 * (int)r) sTt[j * 16 + m] = bf16_to_f32(tv[k]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) sY[t + 256 * k] = bf16_to_f32(yv[k]);
  __syncthreads();
  const int oo = t & 63;
  float y[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) y[m] = sY[m * 64 + oo];
  for (int j = t >> 6; j < (int)r; j += 4) {
    const float sum = dot16(sTt + j * 16, y);
    if (o0 + oo < g.N) g.dB[j * g.N + o0 + oo] = __fmul_rn(g.scale, sum);
  }
}

__global__ __launch_bounds__(256) void k_dx_split_epilogue(const float* __restrict__ partial, int splits, int64_t M,
                                                          int64_t K, const uint16_t* __restrict__ Gs, int64_t rp,
                                                          const uint16_t* __restrict__ A, int64_t r,
                                                          uint16_t* __restrict__ dX, GFold gf, GradFold gr) {
  __shared__ __attribute__((aligned(16))) float sG[16 * 256];
  __shared__ __attribute__((aligned(16))) uint16_t sA[256 * 64];
  const int t = threadIdx.x;
  const int c = t & 63, mq = t >> 6;
  if (gr.dA && (int64_t)blockIdx.x >= K / 64) {   // a dB workgroup (one token group)
    grad_dB_block(gr, M, r, ((int64_t)blockIdx.x - K / 64) * 64, sG, reinterpret_cast<float*>(sA));
    return;
  }
  const int64_t i0 = (int64_t)blockIdx.x * 64;   // K is a multiple of 64: every column exists
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  const int Mg = (int)min<int64_t>(16, M - m0);
  const int mcap = Mg - 1;
  partial += m0 * K + i0 + c;   // row m of the group: partial[(sp M + m) K]

  // weight partials of the first 8 slices (slice indices past the end repeat the last one, unused)
  float v[8][4];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int sp = min(u, splits - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[u][q] = partial[((int64_t)sp * M + min(mq + 4 * q, mcap)) * K];
  }
  // A[i0..i0+63][0..r): 8 r pieces of 16 bytes, at most 8 per thread; pieces past the run
  // get an offset past the end of A and read zero
  const rsrc_t rA = make_rsrc(A, (uint64_t)K * r * 2);
  const int apieces = (int)r * 8;
  const uint32_t abase = (uint32_t)(i0 * r * 2), aend = (uint32_t)(K * r * 2);
  uint4 av[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int idx = t + 256 * u;
    av[u] = ld16(rA, idx < apieces ? abase + (uint32_t)idx * 16 : aend);
  }
  // dA: this block's 64 columns of X for the (at most 16) tokens, four per thread (8 bytes of
  // one row; rows past the tokens read zero), loaded now so they arrive with the rest
  uint2 xv = make_uint2(0u, 0u);
  if (gr.dA) {
    const int m = t >> 4, il = (t & 15) * 4;
    const rsrc_t rX = make_rsrc(gr.X, (uint64_t)M * K * 2);
    xv = gemm::ld8(rX, m < Mg ? (uint32_t)((m * K + i0 + il) * 2) : (uint32_t)(M * K * 2));
  }
  // Gs rows of the group: Mg rp values, at most 2 pieces per thread (when Gs is in memory)
  const rsrc_t rG = make_rsrc(Gs, (uint64_t)M * rp * 2);
  const int gpieces = gf.partial ? 0 : Mg * (int)rp / 8;
  const uint32_t gbase = (uint32_t)(m0 * rp * 2), gend = (uint32_t)(M * rp * 2);
  uint4 gv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = t + 256 * u;
    gv[u] = ld16(rG, idx < gpieces ? gbase + (uint32_t)idx * 16 : gend);
  }
  if (gf.partial) {
    // G from the split-K partials of the rank-r kernel ([tile][split][64][64] fp32, tile =
    // (m / 64) tiles_j + j / 64), summed in split order, scaled and rounded as the reduce
    // kernel would; the first column block of each token group also stores Gs for dA.
    const int ent = Mg * (int)rp;
    for (int e = t; e < ent; e += 256) {
      const int m = e / (int)rp, j = e - m * (int)rp;
      const int64_t row = m0 + m;
      const float* base = gf.partial + (((row >> 6) * gf.tiles_j + (j >> 6)) * gf.splits) * 4096 + (row & 63) * 64 + (j & 63);
      float pv[8];
      float sum = 0.0f;
      for (int s0 = 0; s0 < gf.splits; s0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) pv[u] = base[(int64_t)min(s0 + u, gf.splits - 1) * 4096];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < gf.splits) sum = s0 + u == 0 ? pv[u] : __fadd_rn(sum, pv[u]);
      }
      const uint32_t gb = j < (int)r ? f32_to_bf16_bits(__fmul_rn(gf.scale, sum)) : 0u;
      sG[m * 256 + j] = bf16_to_f32(gb);
      if (blockIdx.x == 0) gf.Gs_out[row * rp + j] = (uint16_t)gb;
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int idx = t + 256 * u;
    if (idx < apieces) {
      const int e = idx * 8, il = e / (int)r, j = e - il * (int)r;   // r % 8 == 0: a piece stays in its row
      const uint32_t w[4] = {av[u].x, av[u].y, av[u].z, av[u].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) sA[(j + k) * 64 + il] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = t + 256 * u;
    if (idx < gpieces) {
      const int e = idx * 8, m = e / (int)rp, j = e - m * (int)rp;
      const uint32_t w[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) sG[m * 256 + j + k] = bf16_to_f32((uint16_t)(w[k >> 1] >> (16 * (k & 1))));
    }
  }
  __syncthreads();
  float acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[q] = v[0][q];
#pragma unroll
    for (int u = 1; u < 8; ++u)
      if (u < splits) acc[q] = __fadd_rn(acc[q], v[u][q]);
  }
  for (int sp = 8; sp < splits; ++sp) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __fadd_rn(acc[q], partial[((int64_t)sp * M + min(mq + 4 * q, mcap)) * K]);
  }
  // Gs A~^T from LDS, four adapter columns at a time (r is a multiple of 8).  Rows of sG
  // past the group are never written; their sums are not stored.
  float lora[4] = {0.f, 0.f, 0.f, 0.f};
  for (int jj = 0; jj < (int)r; jj += 4) {
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = bf16_to_f32(sA[(jj + i) * 64 + c]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 g = *reinterpret_cast<const float4*>(sG + (mq + 4 * q) * 256 + jj);
      lora[q] = __builtin_fmaf(g.x, a[0], lora[q]);
      lora[q] = __builtin_fmaf(g.y, a[1], lora[q]);
      lora[q] = __builtin_fmaf(g.z, a[2], lora[q]);
      lora[q] = __builtin_fmaf(g.w, a[3], lora[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = mq + 4 * q;
    if (m < Mg) dX[(m0 + m) * K + i0 + c] = (uint16_t)f32_to_bf16_bits(__fadd_rn(acc[q], lora[q]));
  }
  if (gr.dA) {
    // dA[i0 + il][j] = sum over the tokens of X[m][i0 + il] Gs[m][j] (Gs in sG; the group holds
    // every token): X transposed in LDS ([il][16], sA is free again), each thread one column j
    // (its 16 Gs values in registers) and the rows il of its wave, consecutive threads on
    // consecutive j
    float* const sXt = reinterpret_cast<float*>(sA);
    __syncthreads();
    {
      const int m = t >> 4, il = (t & 15) * 4;
      sXt[(il + 0) * 16 + m] = bf16_to_f32(xv.x & 0xFFFFu);
      sXt[(il + 1) * 16 + m] = bf16_to_f32(xv.x >> 16);
      sXt[(il + 2) * 16 + m] = bf16_to_f32(xv.y & 0xFFFFu);
      sXt[(il + 3) * 16 + m] = bf16_to_f32(xv.y >> 16);
    }
    __syncthreads();
    for (int jb = 0; jb < (int)r; jb += 64) {
      const int j = jb + (t & 63);
      float g[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) g[m] = m < Mg && j < (int)r ? sG[m * 256 + j] : 0.0f;
      if (j < (int)r)
        for (int il = t >> 6; il < 64; il += 4) gr.dA[(i0 + il) * r + j] = dot16(sXt + il * 16, g);
    }
  }
}

// dispatch over the template flags (DQ, RAGGED, BM, SPLIT)
template <int BM, bool SPLIT>
void launch_dx_variant(bool dq, bool ragged, int bm, dim3 grid, dim3 block, const DxParams& p, hipStream_t s) {
  if constexpr (BM < 2) {
    if (bm != BM) return launch_dx_variant<BM + 1, SPLIT>(dq, ragged, bm, grid, block, p, s);
  }
  if (dq && !ragged)
    hipLaunchKernelGGL((k_bwd_dx_nf4_gemm<true, false, BM, SPLIT>), grid, block, 0, s, p);
  else if (dq)
    hipLaunchKernelGGL((k_bwd_dx_nf4_gemm<true, true, BM, SPLIT>), grid, block, 0, s, p);
  else if (!ragged)
    hipLaunchKernelGGL((k_bwd_dx_nf4_gemm<false, false, BM, SPLIT>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((k_bwd_dx_nf4_gemm<false, true, BM, SPLIT>), grid, block, 0, s, p);
}

}  // namespace

hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const NF4View& w,
                          const uint16_t* Gs, int64_t rp, const uint16_t* A, int64_t r, uint16_t* dX,
                          hipStream_t s) {
  // 64-element code chunks, and blocks (one constant each; in is a multiple of the block size)
  const uint64_t nchunk = (uint64_t)N * K / 64, nblk = ((uint64_t)N * K) >> w.bshift;
  DxParams p{dY, M, K, N, w, nchunk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
             Gs, rp, A, r, dX, nf4_table(w.cb), nullptr, 0, LoraProblem{}, 0};
  const int64_t tiles = ((M + BT - 1) / BT) * ((K + BF - 1) / BF);
  ProfScope ps("k_bwd_dx_nf4_gemm", s);
  const dim3 grid((unsigned)tiles), block(NT);
  const bool ragged = (N % 64) != 0;
  const int bm = w.bshift == 6 ? 0 : w.bshift > 6 ? 1 : 2;
  launch_dx_variant<0, false>(w.dq != 0, ragged, bm, grid, block, p, s);
  return hipGetLastError();
}

hipError_t launch_dx_gemm_split(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const NF4View& w, int stages,
                                float* partial, hipStream_t s, const LoraProblem* g_partials) {
  const uint64_t nchunk = (uint64_t)N * K / 64, nblk = ((uint64_t)N * K) >> w.bshift;
  const uint32_t spl = (uint32_t)stages;
  DxParams p{dY, M, K, N, w, nchunk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
             nullptr, 0, nullptr, 0, nullptr, nf4_table(w.cb), partial, spl, LoraProblem{}, 0};
  if (g_partials) {
    // both operands contiguous along the reduction, split-K partials only
    if (g_partials->g.a_sk != 1 || g_partials->g.b_sk != 1 || g_partials->splits < 2 || !g_partials->partial)
      return hipErrorInvalidValue;
    p.lg = *g_partials;
    p.nlora = (int)(g_partials->tiles_i * g_partials->tiles_j * g_partials->splits);
  }
  const int64_t tiles = ((M + BT - 1) / BT) * ((K + BF - 1) / BF);
  const int64_t nred = (N + 63) / 64;
  const int64_t used = (nred + spl - 1) / spl;   // slices, each with at least one stage
  ProfScope ps("k_bwd_dx_nf4_gemm", s);
  const dim3 grid((unsigned)(p.nlora + tiles * used)), block(NT);
  const bool ragged = (N % 64) != 0;
  const int bm = w.bshift == 6 ? 0 : w.bshift > 6 ? 1 : 2;
  launch_dx_variant<0, true>(w.dq != 0, ragged, bm, grid, block, p, s);
  return hipGetLastError();
}

hipError_t launch_dx_split_epilogue(const float* partial, int splits, int64_t M, int64_t K, const uint16_t* Gs,
                                    int64_t rp, const uint16_t* A, int64_t r, uint16_t* dX, const GFold& gf,
                                    hipStream_t s, const GradFold* grads) {
  if (grads && M > 16) return hipErrorInvalidValue;   // the gradients need every token in one group
  const GradFold gr = grads ? *grads : GradFold{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0.0f};
  const int64_t nb = K / 64 + (grads ? (grads->N + 63) / 64 : 0);
  ProfScope ps("k_dx_split_epilogue", s);
  const dim3 grid((unsigned)nb, (unsigned)((M + 15) / 16)), block(256);
  hipLaunchKernelGGL(k_dx_split_epilogue, grid, block, 0, s, partial, splits, M, K, Gs, rp, A, r, dX, gf, gr);
  return hipGetLastError();
}

}  // namespace qlora
