// Forward for few tokens (M <= 64), where the layer is bound by streaming the
// packed weight from HBM ("QLoRA: Efficient Finetuning of Quantized LLMs",
// section "The QLoRA layer, end to end": the products run in bf16 on a weight
// decoded from 4-bit storage in registers, never written back; y = x W + s (x L1) L2).
//
// Two launches:
//   k_fwd_nf4_gemv      one grid of two kinds of workgroups:
//                        * weight workgroups: one slice of 2048 reduction indices (32 blocks)
//                          x a contiguous range of 16-row groups, fp32 partial sums of
//                          X deq(W)^T into partial[slice][m][n];
//                        * adapter workgroups: 64 columns of A x one slice of 2048 rows,
//                          fp32 partial sums of X A into tpartial[slice][m][j];
//   k_gemv_epilogue     T = sum of its partials (in slice order), Ts = bf16(s T),
//                       Y = bf16( sum of the weight partials (in slice order) + Ts B ).
//
// Weight workgroup (8 waves): wave w owns blocks 4w .. 4w+3 of the slice in every row;
// lane l takes row l % 16 of the current row group and block 4w + l / 16 of it, so one
// lane dequantizes one whole 64-weight block per row group (its scaled 16-entry table is
// built in registers, the lookups are byte permutes) and one v_mfma_f32_16x16x32_bf16
// takes 8 weights from each of the wave's 4 blocks: 8 MFMAs per row group.  The MFMA's
// reduction index is a permutation of k, applied identically to the token operand.  That
// operand depends only on the wave's blocks, not on the row, so it is loaded once into
// registers (8 x 16 bytes per lane) and the wave then streams row group after row group:
// packed codes and block constants run four row groups ahead in a ring of registers.
// After each row group the eight waves' 16 x 16 partial tiles meet in LDS (two buffers,
// one barrier) and are summed in wave order.  Batches of up to 64 tokens run as 2 or 4
// groups of 16 (TG): each lane dequantizes its block once per row group and feeds it to
// TG x 8 MFMAs, holding TG token operands in registers (one workgroup per CU then).
// Adapter workgroups and the epilogue take one 16-token group each.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

namespace qlora {

namespace {

using gemm::i16x4;
using gemm::ld16;
using gemm::make_rsrc;
using gemm::rsrc_t;

constexpr int GT = 512;           // threads per workgroup (8 waves)
constexpr int WBLK = 4;           // blocks per wave in each row (one per 16-lane group)
constexpr int SLB = 8 * WBLK;     // blocks per weight slice
constexpr int RGR = 16;           // rows per row group
constexpr int GROWS = 64;         // adapter columns per adapter workgroup
constexpr int ACH = 64;           // rows of A per LDS chunk (8 KiB)
constexpr int XAS = 72;           // X chunk row stride in the adapter workgroups (64 + 8 padding)
constexpr int KA = 2048;          // rows of A per adapter slice beside the weight pass
constexpr int kSlotsPerCU = 1;    // resident workgroups per CU the grid is sized for (TG = 1)
constexpr int RG_ROUND = 4;       // row groups x token groups per round (one LDS hand-over each)

// LDS: weight groups use two buffers of RG_ROUND [8 waves][64 lanes] float4 tiles; adapter
// groups two A chunks, two X chunks and the [4][64] float4 hand-over area of waves 4..7.
constexpr size_t kLdsWeight = 2 * RG_ROUND * 8 * 64 * 16;
constexpr size_t kLdsAdapter = 2 * ACH * 64 * 2 + 2 * 16 * XAS * 2 + 4 * 64 * 16;

struct GemvParams {
  const uint16_t* X;
  int64_t M, K, N;
  NF4View w;
  uint64_t codes_bytes, absmax_bytes, c1_bytes;
  const uint16_t* A;
  int64_t r;
  float* partial;       // weight partials [splits][M][npad]
  float* tpartial;      // adapter partials [asplits][M][rp]
  int64_t npad;         // rgroups * 16
  int64_t rp;
  int splits;           // weight slices of SLB blocks
  int64_t rgroups;      // 16-row groups
  int64_t rranges;      // weight workgroups per slice (contiguous ranges of row groups)
  int64_t agroups;      // adapter workgroups per adapter slice
  int asplits;
  int ka;               // rows of A per adapter slice (a multiple of 64)
  int ngr;              // 16-token groups
  NF4Table tab;
};

// Natural [ACH][64] tile of A: row k = 128 bytes of eight 16-byte chunks; chunk q of row
// k sits at q ^ 2 f(k), f(k) = ((k >> 1) & 1) | ((k >> 2) & 2), which keeps the
// transposing reads (4 rows x 32 bytes per 16 lanes, two such row quads 8 apart per 32
// lanes) and the row stores (2 rows x 8 chunks per 16 lanes) conflict-free.
__device__ __forceinline__ int apos(int k, int q) {
  const int f = ((k >> 1) & 1) | ((k >> 2) & 2);
  return k * 64 + ((q ^ (f << 1)) << 3);
}

// ---- weight workgroup: slice `slice` of the reduction, row groups [rg_beg, rg_end) ----
// BM: 0 for blocks of 64 (one block per lane), 1 for 128 and 256 (neighbouring lanes share
// a block), 2 for 32 (two blocks per lane: two constants and two tables).
template <bool DQ, int BM, int TG>
__device__ __forceinline__ void weight_group(const GemvParams& p, int bid, uint8_t* lds) {
  float4* const red = reinterpret_cast<float4*>(lds);          // [2][RG_ROUND][8][64]
  const int rranges = (int)p.rranges;
  const int slice = bid / rranges, rr = bid - slice * rranges;
  const int64_t G = p.rgroups;
  const int rg_beg = (int)((rr * G) / rranges);
  const int n_it = (int)(((rr + 1) * G) / rranges) - rg_beg;   // workgroup-uniform
  const int M = (int)p.M, N = (int)p.N;
  const int nkb = (int)(p.K / 64);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int row = lane & 15, g = lane >> 4;
  const int kb = slice * SLB + wave * WBLK + g;     // this lane's block in every row
  const bool kvalid = kb < nkb;
  const uint32_t kbc = (uint32_t)(kvalid ? kb : nkb - 1);   // clamped; its scale is zero

  // token operand of the 8 MFMAs of token group tg: X[16 tg + row][64 kb + 8c .. +7] (zero
  // past M or past K)
  u32x4 xr[TG][8];
  {
    const rsrc_t rX = make_rsrc(p.X, (uint64_t)p.M * p.K * 2);
    const uint32_t xend = (uint32_t)(p.M * p.K * 2);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int m = tg * 16 + row;
      const uint32_t xo = (uint32_t)(m * (int)p.K + kb * 64) * 2;
      const bool xin = m < M && kvalid;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 v = ld16(rX, xin ? xo + c * 16 : xend);
        xr[tg][c] = u32x4{v.x, v.y, v.z, v.w};
      }
    }
  }
  const rsrc_t rC = make_rsrc(p.w.codes, p.codes_bytes);
  const rsrc_t rA = make_rsrc(p.w.absmax, p.absmax_bytes);
  const rsrc_t rC1 = make_rsrc(p.w.c1, p.c1_bytes);
  constexpr bool dq = DQ;
  const float mu = dq ? *p.w.mu : 0.0f;

  struct WStep {
    uint4 c0, c1;     // the 32 code bytes of the lane's 64 weights
    uint32_t c2;      // double quant: the aligned dword holding the lane's 8-bit block
                      // constant (blocks of 32: both constants); else the fp32 absmax bits
                      // (blocks of 32: the first)
    uint32_t c2b;     // double quant: bit offset of the constant in c2; blocks of 32
                      // without double quant: the second fp32 absmax
    float c1f;        // group scale
  };
  const uint32_t bsh = (uint32_t)(p.w.bshift - 6);   // BM == 1: 64-chunks per block, log2
  // row group rg_beg + i: row n = 16 (rg_beg + i) + row, block kbc of that row; rows past N
  // read past the end of the buffers and get zeros (their sums are not stored)
  auto load = [&](int i, WStep& S) {
    const uint32_t n = (uint32_t)((rg_beg + i) * RGR + row);
    const uint32_t blk = n * (uint32_t)nkb + kbc;   // 64-element chunk
    S.c0 = ld16(rC, blk * kBlockBytes);
    S.c1 = ld16(rC, blk * kBlockBytes + 16);
    // first block of the chunk (blocks of 32: blocks 2 blk and 2 blk + 1, one group of 256)
    const uint32_t sb = BM == 0 ? blk : BM == 1 ? blk >> bsh : blk << 1;
    if constexpr (dq) {
      // a whole dword (the constants buffer holds a multiple of 4 bytes for every weight the
      // linear calls take): a byte-sized load would be carried between rounds as a narrow
      // value that the compiler widens right after the load, waiting for it there
      S.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, sb & ~3u, 0, 0);
      S.c2b = (sb & 3u) * 8u;
      S.c1f = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC1, (sb >> 8) * 4, 0, 0));
    } else {
      if constexpr (BM == 2) {
        S.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, sb * 4, 0, 0);
        S.c2b = __builtin_amdgcn_raw_buffer_load_b32(rA, sb * 4 + 4, 0, 0);
      } else {
        S.c2 = __builtin_amdgcn_raw_buffer_load_b32(rA, sb * 4, 0, 0);
        S.c2b = 0;
      }
      S.c1f = 0.0f;
    }
  };
  // The wave works in rounds of R row groups (R x TG accumulator tiles), loading the codes
  // of the next round while it computes this one, and the eight waves' tiles meet in LDS
  // once per round.  acc[v] of lane l holds row 4 (l / 16) + v, token l % 16 of a tile.
  constexpr int R = RG_ROUND / TG;
  constexpr int TILES = R * TG;                                  // tiles per wave and round
  // reduction mapping: thread t sums rows t % 16 of tokens (t / 16) % 16 of tiles t / 256,
  // t / 256 + 2, ... (so a wave stores 64 consecutive rows of four tokens)
  const int rrow = t & 15, rtok = (t >> 4) & 15, rt0 = t >> 8;
  const int roff = ((rrow >> 2) * 16 + rtok) * 4 + (rrow & 3);   // float offset inside a tile
  // partials through a buffer resource: an offset past its end drops the store, so the
  // reduction needs no branch (a branch around the stores would make the compiler lose track
  // of the loads in flight and wait for all of them at the next round)
  const uint32_t pbytes = (uint32_t)(p.splits * p.M * p.npad * 4);
  const rsrc_t rP = make_rsrc(p.partial, pbytes);
  const uint32_t pbase = (uint32_t)((slice * p.M + rtok) * p.npad + rrow) * 4u;
  // one row group: dequantize the lane's block, TG x 8 MFMAs.  The scheduling barriers and the
  // empty asm keep each row group's work in place: left free, the compiler moves arithmetic
  // on the next round's freshly loaded codes ahead and so waits for loads issued a moment
  // earlier.
  auto step = [&](const WStep& S, f32x4 (&acc)[TG]) {
    __builtin_amdgcn_sched_barrier(0);
    u32x4 q0 = {S.c0.x, S.c0.y, S.c0.z, S.c0.w}, q1 = {S.c1.x, S.c1.y, S.c1.z, S.c1.w};
    uint32_t c2 = S.c2, c2b = S.c2b;
    float c1f = S.c1f;
    asm volatile("" : "+v"(q0), "+v"(q1), "+v"(c2), "+v"(c2b), "+v"(c1f));
    if constexpr (dq) c2 >>= c2b;
    // v_cvt_f32_fp8 reads byte 0 of its operand (the lane's constant; blocks of 32: the first)
    const float sc = dq ? __fadd_rn(__fmul_rn(e4m3_decode(c2), c1f), mu) : __uint_as_float(c2);
    const Planes pl = make_planes(p.tab, kvalid ? sc : 0.0f);
    const uint32_t cw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) acc[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BM == 2) {
      // code words 0..3 hold the first block of 32, 4..7 the second (its table is built once
      // the first one is done with, so the two never occupy registers together)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 wv = dequant8(pl, cw[c]);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) acc[tg] = mfma16(wv, xr[tg][c], acc[tg]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const float sc2 = dq ? __fadd_rn(__fmul_rn(e4m3_decode_byte1(c2), c1f), mu) : __uint_as_float(c2b);
      const Planes pl2 = make_planes(p.tab, kvalid ? sc2 : 0.0f);
#pragma unroll
      for (int c = 4; c < 8; ++c) {
        const u32x4 wv = dequant8(pl2, cw[c]);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) acc[tg] = mfma16(wv, xr[tg][c], acc[tg]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const u32x4 wv = dequant8(pl, cw[c]);
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) acc[tg] = mfma16(wv, xr[tg][c], acc[tg]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // eight waves' tiles of round q (row groups q R .. q R + R - 1) meet in LDS buffer q % 2
  auto hand_over = [&](int q, const f32x4 (&acc)[R][TG]) {
    const int g0 = q * R;
    float4* const buf = red + (q & 1) * (TILES * 512);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int tg = 0; tg < TG; ++tg)
        buf[(r * TG + tg) * 512 + wave * 64 + lane] = make_float4(acc[r][tg][0], acc[r][tg][1], acc[r][tg][2],
                                                                  acc[r][tg][3]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TILES / 2; ++u) {
      const int tile = rt0 + 2 * u, r = tile / TG, tg = tile - r * TG;
      const int n = (rg_beg + g0 + r) * RGR + rrow;
      const bool ok = g0 + r < n_it && tg * 16 + rtok < M && n < N;
      const float* b = reinterpret_cast<const float*>(buf + tile * 512) + roff;
      float sum = b[0];
#pragma unroll
      for (int w = 1; w < 8; ++w) sum = __fadd_rn(sum, b[w * 256]);
      const uint32_t off = pbase + (uint32_t)(tg * 16 * p.npad + (rg_beg + g0 + r) * RGR) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rP, ok ? off : pbytes, 0, 0);
    }
  };
  // Row groups are loaded RING ahead (a ring of register sets, one round of 4 row groups of
  // work: RING / R rounds in flight), and a ring cycle runs without branches (a branch around a
  // row group's work would make the compiler wait for every load in flight where it rejoins):
  // the codes of row group i + RING are loaded right after row group i has used its registers.
  // A load index past the end is clamped to the last row group (loaded again, never used).
  constexpr int RING = 4;
  static_assert(RING % R == 0, "whole rounds per ring cycle");
  const int last = max(n_it - 1, 0);
  const int ncyc = n_it / RING;
  WStep S[RING];
  // the first loads in the order the loop issues them (slot by slot): the compiler's wait
  // counts at the loop head must hold on entry as well as around the loop
#pragma unroll
  for (int d = 0; d < RING; ++d) {
    load(min(d, last), S[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int c = 0; c < ncyc; ++c) {
#pragma unroll
    for (int q = 0; q < RING / R; ++q) {
      f32x4 acc[R][TG];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int d = q * R + r;
        step(S[d], acc[r]);
        load(min(c * RING + d + RING, last), S[d]);
      }
      hand_over(c * (RING / R) + q, acc);
    }
  }
  // the last n_it % RING row groups (workgroup-uniform branches)
  const int i0 = ncyc * RING;
#pragma unroll
  for (int q = 0; q < RING / R; ++q) {
    if (i0 + q * R < n_it) {
      f32x4 acc[R][TG];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (i0 + q * R + r < n_it) {
          step(S[q * R + r], acc[r]);
        } else {
#pragma unroll
          for (int tg = 0; tg < TG; ++tg) acc[r][tg] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      hand_over(ncyc * (RING / R) + q, acc);
    }
  }
}

// ---- adapter workgroup: columns j0.. of A over a slice of ka rows; A is [K][r], columns
// past r read zero.  Loads run in groups of 4 chunks (of 64 rows), one group ahead; each
// chunk of A and of X is stored to LDS (two buffers) and taken by waves 0..3 (first 32 rows)
// and 4..7 (the rest).
__device__ __forceinline__ void adapter_group(const GemvParams& p, int bid, uint8_t* lds) {
  uint16_t* const sAb = reinterpret_cast<uint16_t*>(lds);      // [2][ACH * 64]
  uint16_t* const sXa = sAb + 2 * ACH * 64;                    // [2][16][XAS]
  float4* const sAcc = reinterpret_cast<float4*>(sXa + 2 * 16 * XAS);   // [4][64]
  const int nsp = p.asplits;
  const int tgi = bid % p.ngr;                                 // this workgroup's 16-token group
  const int rest = bid / p.ngr;
  const int grp = rest / nsp;
  const int split = rest - grp * nsp;
  const int m0 = tgi * 16;
  const int kb_beg = split * (p.ka / 64);
  const int nkb = (int)(p.K / 64);
  const int nkb_s = min(nkb, kb_beg + p.ka / 64) - kb_beg;      // blocks (64-row chunks) in this slice
  const int M = min((int)p.M - m0, 16);      // tokens of this group
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wq = wave & 3, par = wave >> 2;
  const int row = lane & 15, g = lane >> 4;
  const int xrow = row < M ? row : row % M;   // token rows past the group repeat real rows (outputs unused)
  const rsrc_t rX = make_rsrc(p.X, (uint64_t)p.M * p.K * 2);
  const uint32_t xend = (uint32_t)(p.M * p.K * 2);
  const int j0 = grp * GROWS;
  const rsrc_t rAd = make_rsrc(p.A, (uint64_t)p.K * p.r * 2);
  const uint32_t aend = (uint32_t)(p.K * p.r * 2);
  const int lr = t >> 3, lq = t & 7;                 // A load mapping: row lr, chunk lq
  const bool col_ok = j0 + lq * 8 < p.r;
  const bool xload = t < M * 8;                      // X load mapping: token t / 8, chunk t % 8
  const int xm = t >> 3;
  const int j = lane & 15, jc = wq * 16 + (j & 3) * 4;
  const int kr = par * 32 + g * 8 + (j >> 2);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // chunks cb .. cb+3 into registers; chunks past the slice read zero (never stored)
  auto load4 = [&](int cb, uint4 (&va)[4], uint4 (&vx)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = cb + u;
      const int k = (kb_beg + c) * 64 + lr;
      va[u] = ld16(rAd, col_ok && c < nkb_s ? (uint32_t)((k * (int)p.r + j0 + lq * 8) * 2) : aend);
      vx[u] = ld16(rX, xload && c < nkb_s ? (uint32_t)(((m0 + xm) * (int)p.K + (kb_beg + c) * 64 + lq * 8) * 2)
                                         : xend);
    }
  };
  auto proc4 = [&](int cb, const uint4 (&va)[4], const uint4 (&vx)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (cb + u < nkb_s) {   // uniform
        const int buf = (cb + u) & 1;
        uint16_t* sAc = sAb + buf * (ACH * 64);
        uint16_t* sXc = sXa + buf * (16 * XAS);
        *reinterpret_cast<uint4*>(sAc + apos(lr, lq)) = va[u];
        *reinterpret_cast<uint4*>(sXc + (xload ? xm * XAS + lq * 8 : 15 * XAS + 64)) = vx[u];
        __syncthreads();
        // operand A: rows = columns jc = 16 (wave % 4) + l % 16 of A, 8 consecutive k per lane group
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(sAc + apos(kr, jc >> 3) + (jc & 7)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(sAc + apos(kr + 4, jc >> 3) + (jc & 7)));
        const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
        u32x4 wa;
        wa.x = a.x; wa.y = a.y; wa.z = b.x; wa.w = b.y;
        const u32x4 xb = *reinterpret_cast<const u32x4*>(sXc + xrow * XAS + par * 32 + g * 8);
        acc = mfma16(wa, xb, acc);
      }
    }
  };
  // two groups of four chunks in flight: the loads of the next group are issued before the
  // current one is processed
  uint4 a0[4], x0[4], a1[4], x1[4];
  load4(0, a0, x0);
  for (int cb = 0; cb < nkb_s; cb += 8) {
    load4(cb + 4, a1, x1);
    proc4(cb, a0, x0);
    load4(cb + 8, a0, x0);
    proc4(cb + 4, a1, x1);
  }
  // waves 4..7 hand their sums to waves 0..3; acc[v] = C[column 4 g + v of the wave][token l % 16]
  if (par) sAcc[wq * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (!par && row < M) {
    const float4 o = sAcc[wq * 64 + lane];
    const int64_t n = (int64_t)grp * GROWS + wq * 16 + 4 * g;
    float* dst = p.tpartial + ((int64_t)split * p.M + m0 + row) * p.rp + n;
    *reinterpret_cast<float4*>(dst) = make_float4(__fadd_rn(acc[0], o.x), __fadd_rn(acc[1], o.y),
                                                  __fadd_rn(acc[2], o.z), __fadd_rn(acc[3], o.w));
  }
}

// Workgroups [0, agroups * asplits) are adapter workgroups, the rest weight workgroups.
// DQ: block constants are double-quantized (8-bit code, c1 per 256 blocks, mu).
template <bool DQ, int BM, int TG>
__global__ __launch_bounds__(GT) void k_fwd_nf4_gemv(GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int n_adapter = (int)(p.agroups * p.asplits) * p.ngr;
  if ((int)blockIdx.x < n_adapter)
    adapter_group(p, (int)blockIdx.x, lds);
  else
    weight_group<DQ, BM, TG>(p, (int)blockIdx.x - n_adapter, lds);
}

// Y[m][n] = bf16( sum over slices of partial[slice][m][n] + sum_j Ts[m][j] B[j][n] ),
// Ts = bf16(s T), T = sum over adapter slices of tpartial[slice][m][j] (formed again by every
// workgroup: 16 r values); column block 0 also writes T_save = bf16(T).  A workgroup covers
// 64 columns of one 16-token group (blockIdx.y); thread t takes column t % 64 for the tokens
// m = t / 64 + 4 q of the group.  The loads of the first 8
// slices of both sums and of B are all issued before any of them is used, so the common case
// waits for memory once; sums run in slice order.
__global__ __launch_bounds__(256) void k_gemv_epilogue(const float* __restrict__ partial, int splits,
                                                       const float* __restrict__ tpartial, int asplits, int64_t M,
                                                       int64_t N, int64_t npad, int64_t rp,
                                                       const uint16_t* __restrict__ B, int64_t r, float scale,
                                                       uint16_t* __restrict__ Y, uint16_t* __restrict__ T_save) {
  __shared__ __attribute__((aligned(16))) float sTs[16 * 256];
  __shared__ __attribute__((aligned(16))) uint16_t sB[256 * 64];
  const int t = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int c = t & 63, mq = t >> 6;
  const int64_t n = n0 + c;
  const int64_t nc = n < N ? n : N - 1;          // clamped column: every load stays inside the partials
  const int64_t m0 = (int64_t)blockIdx.y * 16;   // first token of the group
  const int Mg = (int)min<int64_t>(16, M - m0);  // tokens of the group
  const int mcap = Mg - 1;
  const int MR = (int)(Mg * rp);                 // T entries of the group (at most 16 x 256)
  partial += m0 * npad;                          // row m of the group: partial[(sp M + m) npad + n]
  tpartial += m0 * rp;                           // tpartial[sp M rp + m rp + j]
  Y += m0 * N;
  if (T_save) T_save += m0 * r;

  // weight partials of the first 8 slices (slice indices past the end repeat the last one, unused)
  float v[8][4];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int sp = min(u, splits - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[u][q] = partial[((int64_t)sp * M + min(mq + 4 * q, mcap)) * npad + nc];
  }
  // rows j < r of B for the 64 columns: rp * 8 chunks of 16 bytes, at most 8 per thread
  // (buffer loads: chunks outside B get an offset past its end and read zero, no branch)
  const rsrc_t rB = make_rsrc(B, (uint64_t)r * N * 2);
  const uint32_t bend = (uint32_t)(r * N * 2);
  uint4 bv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int idx = t + 256 * u;
    const int jj = idx >> 3, q = idx & 7;
    const bool ok = idx < (int)rp * 8 && jj < r && n0 + q * 8 < N;
    bv[u] = ld16(rB, ok ? (uint32_t)((jj * N + n0 + q * 8) * 2) : bend);
  }
  // T entries idx = t + 256 u, four at a time, over the adapter slices in order (8 slices per pass)
  for (int e0 = 0; e0 < MR; e0 += 4 * 256) {
    float ts[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < asplits; s0 += 8) {
      float tv[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sp = min(s0 + u, asplits - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[u][e] = tpartial[(int64_t)sp * M * rp + min(e0 + e * 256 + t, MR - 1)];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (s0 + u < asplits) ts[e] = __fadd_rn(ts[e], tv[u][e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = e0 + e * 256 + t;
      if (idx < MR) {
        const int m = idx / (int)rp, jj = idx - m * (int)rp;
        sTs[m * 256 + jj] = jj < r ? bf16_to_f32(f32_to_bf16_bits(__fmul_rn(scale, ts[e]))) : 0.0f;
        if (T_save && blockIdx.x == 0 && jj < r) T_save[m * r + jj] = (uint16_t)f32_to_bf16_bits(ts[e]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int idx = t + 256 * u;
    if (idx < (int)rp * 8) *reinterpret_cast<uint4*>(sB + (idx >> 3) * 64 + (idx & 7) * 8) = bv[u];
  }
  __syncthreads();
  if (n >= N) return;
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
    for (int q = 0; q < 4; ++q)
      acc[q] = __fadd_rn(acc[q], partial[((int64_t)sp * M + min(mq + 4 * q, mcap)) * npad + n]);
  }
  // s T B from LDS, four adapter rows at a time (rp is a multiple of 64; rows past r are zero)
  float lora[4] = {0.f, 0.f, 0.f, 0.f};
  for (int jj = 0; jj < (int)rp; jj += 4) {
    float b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = bf16_to_f32(sB[(jj + i) * 64 + c]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 tq = *reinterpret_cast<const float4*>(sTs + (mq + 4 * q) * 256 + jj);
      lora[q] = __builtin_fmaf(tq.x, b[0], lora[q]);
      lora[q] = __builtin_fmaf(tq.y, b[1], lora[q]);
      lora[q] = __builtin_fmaf(tq.z, b[2], lora[q]);
      lora[q] = __builtin_fmaf(tq.w, b[3], lora[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = mq + 4 * q;
    if (m < Mg) Y[m * N + n] = (uint16_t)f32_to_bf16_bits(__fadd_rn(acc[q], lora[q]));
  }
}

// dispatch over the template flags (DQ, BM, TG)
template <int TG>
void launch_gemv_variant(bool dq, int bm, int tg, dim3 grid, size_t lds, const GemvParams& p, hipStream_t s) {
  if constexpr (TG < 4) {
    if (tg != TG) return launch_gemv_variant<TG * 2>(dq, bm, tg, grid, lds, p, s);
  }
  const dim3 block(GT);
  if (dq) {
    if (bm == 0) hipLaunchKernelGGL((k_fwd_nf4_gemv<true, 0, TG>), grid, block, lds, s, p);
    else if (bm == 1) hipLaunchKernelGGL((k_fwd_nf4_gemv<true, 1, TG>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((k_fwd_nf4_gemv<true, 2, TG>), grid, block, lds, s, p);
  } else {
    if (bm == 0) hipLaunchKernelGGL((k_fwd_nf4_gemv<false, 0, TG>), grid, block, lds, s, p);
    else if (bm == 1) hipLaunchKernelGGL((k_fwd_nf4_gemv<false, 1, TG>), grid, block, lds, s, p);
    else hipLaunchKernelGGL((k_fwd_nf4_gemv<false, 2, TG>), grid, block, lds, s, p);
  }
}

}  // namespace

// Weight slices of SLB blocks, each split into contiguous ranges of 16-row groups, and
// adapter slices of KA rows of A.  The grid fills kSlotsPerCU workgroups per CU in one round.
// adapters_only (a launch of X A alone): slices of at least 256 rows, as many as it takes for
// the adapter workgroups to reach about one per CU.
GemvPlan gemv_plan(int64_t M, int64_t K, int64_t N, int64_t rp, bool adapters_only) {
  const int64_t nkb = K / 64;
  const int64_t Mm = std::max<int64_t>(M, 1);
  GemvPlan pl;
  pl.ngr = (int)((Mm + 15) / 16);
  pl.tg = pl.ngr == 1 ? 1 : pl.ngr == 2 ? 2 : 4;
  const int64_t slots = 256 * (pl.tg == 1 ? kSlotsPerCU : 1);   // TG > 1: 256 VGPRs, one per CU
  pl.splits = (int)((nkb + SLB - 1) / SLB);
  pl.rgroups = (N + RGR - 1) / RGR;
  pl.npad = pl.rgroups * RGR;
  pl.agroups = rp / GROWS;
  int64_t ka = KA;
  if (adapters_only) {
    const int64_t want = std::max<int64_t>(1, 256 / (pl.agroups * pl.ngr));
    ka = std::max<int64_t>(256, ((K + want - 1) / want + 255) / 256 * 256);
  }
  pl.ka = (int)std::min<int64_t>(ka, (K + 63) / 64 * 64);
  pl.asplits = (int)((K + pl.ka - 1) / pl.ka);
  const int64_t aw = pl.agroups * pl.asplits * pl.ngr;
  pl.rranges = std::max<int64_t>(1, std::min<int64_t>(pl.rgroups, (slots - aw) / pl.splits));
  pl.tpart = (size_t)pl.splits * Mm * pl.npad;
  return pl;
}

size_t gemv_partial_floats(const GemvPlan& pl, int64_t M) {
  return pl.tpart + (size_t)pl.asplits * M * pl.agroups * GROWS;
}

hipError_t launch_gemv(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w, const uint16_t* A,
                       int64_t r, const GemvPlan& pl, float* partial, hipStream_t s, bool adapters_only) {
  // 64-element code chunks, and blocks (one constant each; in is a multiple of the block size)
  const uint64_t nchunk = (uint64_t)N * K / 64, nblk = ((uint64_t)N * K) >> w.bshift;
  GemvParams p{X, M, K, N, w, nchunk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
               A, r, partial, partial + pl.tpart, pl.npad, pl.agroups * GROWS, pl.splits, pl.rgroups,
               pl.rranges, pl.agroups, pl.asplits, pl.ka, pl.ngr, nf4_table(w.cb)};
  // X A alone: the TG = 1 code (the adapter workgroups do not depend on TG) and their LDS only
  const size_t lds = adapters_only ? kLdsAdapter : std::max(kLdsWeight, kLdsAdapter);
  ProfScope ps("k_fwd_nf4_gemv", s);
  const int64_t n_adapter = pl.agroups * pl.asplits * pl.ngr;
  const dim3 grid((unsigned)((adapters_only ? 0 : pl.rranges * pl.splits) + n_adapter));
  const int bm = w.bshift == 6 ? 0 : w.bshift > 6 ? 1 : 2;
  launch_gemv_variant<1>(w.dq != 0, bm, adapters_only ? 1 : pl.tg, grid, lds, p, s);
  return hipGetLastError();
}

hipError_t launch_gemv_epilogue(const float* partial, const GemvPlan& pl, int64_t M, int64_t N, const uint16_t* B,
                                int64_t r, float scale, uint16_t* Y, uint16_t* T_save, hipStream_t s) {
  ProfScope ps("k_gemv_epilogue", s);
  hipLaunchKernelGGL(k_gemv_epilogue, dim3((unsigned)((N + 63) / 64), (unsigned)pl.ngr), dim3(256), 0, s, partial,
                     pl.splits,
                     partial + pl.tpart, pl.asplits, M, N, pl.npad, pl.agroups * GROWS, B, r, scale, Y, T_save);
  return hipGetLastError();
}

}  // namespace qlora
