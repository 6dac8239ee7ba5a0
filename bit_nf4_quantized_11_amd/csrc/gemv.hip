// Forward for few tokens (M <= 16), where the layer is bound by streaming the
// packed weight from HBM ("QLoRA: Efficient Finetuning of Quantized LLMs",
// section "The QLoRA layer, end to end": the weight is dequantized to bf16 on the
// fly, used, and thrown away; y = x W + s (x L1) L2).
//
// Two launches:
//   k_fwd_nf4_gemv      one grid of two kinds of workgroups:
//                        * weight workgroups: 64 weight rows x one slice of the reduction,
//                          fp32 partial sums of X deq(W)^T into partial[split][m][n];
//                        * adapter workgroups: 64 columns of A x one slice of 2048 rows,
//                          fp32 partial sums of X A into tpartial[slice][m][j];
//   k_gemv_epilogue     T = sum of its partials (in slice order), Ts = bf16(s T),
//                       Y = bf16( sum of the weight partials (in split order) + Ts B ).
//
// Weight workgroup (8 waves): wave w owns rows 16 (w % 4) .. +15 of the group and the
// steps of parity w / 4; lane l takes row l % 16 and, in each of its steps of 4 blocks,
// block (step*4 + l/16) of that row: one lane dequantizes one whole 64-weight block (its
// scaled 16-entry table is built once per block in registers, the lookups are byte
// permutes).  One v_mfma_f32_16x16x32_bf16 then takes 8 weights from each of the 4
// blocks, so 8 MFMAs consume a step.  The MFMA's reduction index is a permutation of k,
// applied identically to the token operand, which is read from the slice of X staged in
// LDS.  Loads of the packed weight run four steps ahead; the two waves of a row group add
// their sums through LDS at the end.
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
constexpr int GROWS = 64;         // weight rows (or adapter columns) per workgroup
constexpr int GMAX_X = 16384;     // max elements of the staged X slice (M * slice length): 32 KiB
constexpr int ACH = 64;           // rows of A per LDS chunk (8 KiB)
constexpr int XAS = 72;           // X chunk row stride in the adapter workgroups (64 + 8 padding)
constexpr int KA = 2048;          // rows of A per adapter slice

struct GemvParams {
  const uint16_t* X;
  int64_t M, K, N;
  NF4View w;
  uint64_t codes_bytes, absmax_bytes, c1_bytes;
  const uint16_t* A;
  int64_t r;
  float* partial;       // weight partials [splits][M][npad]
  float* tpartial;      // adapter partials [asplits][M][rp]
  int64_t npad;         // wgroups * 64
  int64_t rp;
  int64_t kbps;         // blocks per weight slice (multiple of 4)
  int splits;
  int64_t wgroups;      // weight workgroups per slice
  int64_t agroups;      // adapter workgroups per adapter slice
  int64_t ka;           // rows of A per adapter slice (multiple of 64, at most 512 and kbps * 64)
  int asplits;
  NF4Table tab;
};

// X slice in LDS: row m of rc 16-byte chunks plus one chunk of padding, so the 16 token
// rows read by one MFMA operand fetch (same chunk) fall in distinct banks.
__device__ __forceinline__ int xrow_elems(int rc) { return (rc + 1) * 8; }

// Natural [ACH][64] tile of A: row k = 128 bytes of eight 16-byte chunks; chunk q of row
// k sits at q ^ 2 f(k), f(k) = ((k >> 1) & 1) | ((k >> 2) & 2), which keeps the
// transposing reads (4 rows x 32 bytes per 16 lanes, two such row quads 8 apart per 32
// lanes) and the row stores (2 rows x 8 chunks per 16 lanes) conflict-free.
__device__ __forceinline__ int apos(int k, int q) {
  const int f = ((k >> 1) & 1) | ((k >> 2) & 2);
  return k * 64 + ((q ^ (f << 1)) << 3);
}

// Dynamic LDS: the X slice (M padded rows), then the A chunk (adapter groups) or the decoded
// block scales of the group (weight groups); a static 4 KiB area carries the accumulators of
// waves 4..7 to waves 0..3.
// DQ: block constants are double-quantized (8-bit code, c1 per 256 blocks, mu).
template <bool DQ>
__global__ __launch_bounds__(GT) void k_fwd_nf4_gemv(GemvParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];
  __shared__ float4 sAcc[4 * 64];
  const int rc = (int)(p.kbps * 8);                           // 16-byte chunks of the slice
  const int xre = xrow_elems(rc);
  uint16_t* const sX = smem_dyn;
  uint16_t* const sA = smem_dyn + (int)p.M * xre;              // adapter groups
  float* const sS = reinterpret_cast<float*>(sA);              // weight groups: [64][kbps] scales

  // workgroups [0, agroups * asplits) are adapter workgroups, the rest weight workgroups
  const int nkb = (int)(p.K / 64);
  const int n_adapter = (int)(p.agroups * p.asplits);
  const bool adapter = (int)blockIdx.x < n_adapter;
  const int bid = adapter ? (int)blockIdx.x : (int)blockIdx.x - n_adapter;
  const int nsp = adapter ? p.asplits : p.splits;
  const int grp = bid / nsp;
  const int split = bid - grp * nsp;
  const int kbu = adapter ? KA / 64 : (int)p.kbps;             // blocks per slice of this kind
  const int kb_beg = split * kbu;
  const int nkb_s = min(nkb, kb_beg + kbu) - kb_beg;           // blocks in this slice
  const int M = (int)p.M;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform: loop bounds stay scalar
  const int wq = wave & 3, par = wave >> 2;
  const int row = lane & 15, g = lane >> 4;
  const int xrow = row < M ? row : row % M;   // token rows past M repeat real rows (outputs unused)

  // stage X[0..M)[slice] (chunks past the slice end are zero)
  const rsrc_t rX = make_rsrc(p.X, (uint64_t)p.M * p.K * 2);
  const uint32_t xend = (uint32_t)(p.M * p.K * 2);
  auto stage_x = [&]() {
    const int total = M * rc;
    for (int base = 0; base < total; base += 4 * GT) {   // 4 loads in flight per thread
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * GT + t;
        const int m = idx / rc, c = idx - m * rc;
        const bool in = idx < total && c < nkb_s * 8;
        v[u] = ld16(rX, in ? (uint32_t)((m * (int)p.K + kb_beg * 64 + c * 8) * 2) : xend);
      }
      // stores are unconditional (lanes past the end write the padding chunk of row 0): a
      // store under a branch leaves its load "pending" for the compiler, which then waits
      // for it on every later reuse of the register
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = base + u * GT + t;
        const int m = idx / rc, c = idx - m * rc;
        *reinterpret_cast<uint4*>(sX + (idx < total ? m * xre + c * 8 : rc * 8)) = v[u];
      }
    }
    __syncthreads();
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* xbase = sX + xrow * xre;

  if (!adapter) {
    // ---- weight workgroup ----
    const uint32_t n = (uint32_t)(grp * GROWS + wq * 16 + row);   // rows past N read as zero (OOB)
    const rsrc_t rC = make_rsrc(p.w.codes, p.codes_bytes);
    const rsrc_t rA = make_rsrc(p.w.absmax, p.absmax_bytes);
    const rsrc_t rC1 = make_rsrc(p.w.c1, p.c1_bytes);
    constexpr bool dq = DQ;
    const float mu = dq ? *p.w.mu : 0.0f;
    const uint32_t rowblk = n * (uint32_t)nkb + (uint32_t)kb_beg;
    const int nsteps = (nkb_s + 3) / 4;
    const int my_steps = (nsteps - par + 1) / 2;   // steps par, par + 2, ...
    const int kbps = (int)p.kbps;

    // block scales of the group's 64 rows x this slice, decoded once into LDS
    // ("doubleDequant": s' = fl32(fl32(dec(c2) c1) + mu)); rows past N read zero constants
    auto stage_scales = [&]() {
      const int total = GROWS * nkb_s;
      for (int base = 0; base < total; base += 4 * GT) {
        uint32_t c2[4];
        float c1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int idx = min(base + u * GT + t, total - 1);
          const int rr = idx / nkb_s, kb = idx - rr * nkb_s;
          const uint32_t blk = (uint32_t)(grp * GROWS + rr) * (uint32_t)nkb + (uint32_t)(kb_beg + kb);
          if constexpr (dq) {
            c2[u] = __builtin_amdgcn_raw_buffer_load_b8(rA, blk, 0, 0);
            c1[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC1, (blk >> 8) * 4, 0, 0));
          } else {
            c2[u] = __builtin_amdgcn_raw_buffer_load_b32(rA, blk * 4, 0, 0);
            c1[u] = 0.0f;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // unconditional: lanes past the end write the spare slot
          const int idx = base + u * GT + t;
          const int rr = idx / nkb_s, kb = idx - rr * nkb_s;
          sS[idx < total ? rr * kbps + kb : GROWS * kbps] =
              dq ? __fadd_rn(__fmul_rn(e4m3_decode(c2[u]), c1[u]), mu) : __uint_as_float(c2[u]);
        }
      }
    };
    const float* srow = sS + (wq * 16 + row) * kbps;

    struct WStep {
      uint4 c0, c1;
    };
    // this wave's k-th step: block kb_beg + 4 (par + 2k) + g of row n, clamped to the last
    // block of the slice (its contribution is then dropped by a zero scale)
    auto load = [&](int k, WStep& S) {
      const int kbl = min(4 * (par + 2 * k) + g, nkb_s - 1);
      const uint32_t blk = rowblk + (uint32_t)kbl;
      S.c0 = ld16(rC, blk * kBlockBytes);
      S.c1 = ld16(rC, blk * kBlockBytes + 16);
    };
    // The scheduling barriers and the empty asm keep each step's work inside its step: left
    // free, the compiler moves arithmetic on the next step's freshly loaded codes ahead and
    // so waits for loads issued a moment earlier.
    auto compute = [&](int k, const WStep& S) {
      __builtin_amdgcn_sched_barrier(0);
      const int kb = 4 * (par + 2 * k) + g;
      const uint16_t* xp = xbase + kb * 64;
      const float sraw = srow[kb];                 // kb < kbps: inside the scale tile
      const float sc = kb < nkb_s ? sraw : 0.0f;
      u32x4 q0 = {S.c0.x, S.c0.y, S.c0.z, S.c0.w}, q1 = {S.c1.x, S.c1.y, S.c1.z, S.c1.w};
      asm volatile("" : "+v"(q0), "+v"(q1));
      const Planes pl = make_planes(p.tab, sc);
      const uint32_t cw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc = mfma16(dequant8(pl, cw[c]), *reinterpret_cast<const u32x4*>(xp + c * 8), acc);
      __builtin_amdgcn_sched_barrier(0);
    };
    // four steps in flight per wave (a ring of four register sets)
    WStep S0, S1, S2, S3;
    const int last = max(my_steps - 1, 0);
    load(0, S0);
    load(min(1, last), S1);
    load(min(2, last), S2);
    load(min(3, last), S3);
    stage_scales();
    stage_x();
    int k = 0;
    for (; k + 3 < my_steps; k += 4) {
      compute(k, S0);
      load(min(k + 4, last), S0);
      compute(k + 1, S1);
      load(min(k + 5, last), S1);
      compute(k + 2, S2);
      load(min(k + 6, last), S2);
      compute(k + 3, S3);
      load(min(k + 7, last), S3);
    }
    if (k < my_steps) compute(k, S0);
    if (k + 1 < my_steps) compute(k + 1, S1);
    if (k + 2 < my_steps) compute(k + 2, S2);
  } else {
    // ---- adapter workgroup: columns j0.. of A over a slice of rows (one block = 64 rows of
    // A per chunk); A is [K][r], columns past r read zero.  Loads run 4 chunks at a time; each
    // chunk of A and of X is stored to LDS (two buffers) and taken by waves 0..3 (first 32
    // rows) and 4..7 (the rest).
    uint16_t* const sAb = smem_dyn;                            // [2][ACH * 64]
    uint16_t* const sXa = smem_dyn + 2 * ACH * 64;             // [2][16][XAS]
    const int j0 = grp * GROWS;
    const rsrc_t rAd = make_rsrc(p.A, (uint64_t)p.K * p.r * 2);
    const uint32_t aend = (uint32_t)(p.K * p.r * 2);
    const int lr = t >> 3, lq = t & 7;                 // A load mapping: row lr, chunk lq
    const bool col_ok = j0 + lq * 8 < p.r;
    const bool xload = t < M * 8;                      // X load mapping: token t / 8, chunk t % 8
    const int xm = t >> 3;
    const int j = lane & 15, jc = wq * 16 + (j & 3) * 4;
    const int kr = par * 32 + g * 8 + (j >> 2);
    for (int cb = 0; cb < nkb_s; cb += 4) {
      uint4 va[4], vx[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = cb + u;
        const int k = (kb_beg + c) * 64 + lr;
        va[u] = ld16(rAd, col_ok && c < nkb_s ? (uint32_t)((k * (int)p.r + j0 + lq * 8) * 2) : aend);
        vx[u] = ld16(rX, xload && c < nkb_s ? (uint32_t)((xm * (int)p.K + (kb_beg + c) * 64 + lq * 8) * 2) : xend);
      }
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
    }
  }

  // waves 4..7 hand their sums to waves 0..3; acc[v] = C[row 4 g + v of the wave][token l % 16]
  if (par) sAcc[wq * 64 + lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (!par && row < M) {
    const float4 o = sAcc[wq * 64 + lane];
    const int64_t n = (int64_t)grp * GROWS + wq * 16 + 4 * g;
    float* dst = adapter ? p.tpartial + ((int64_t)split * p.M + row) * p.rp + n
                         : p.partial + ((int64_t)split * p.M + row) * p.npad + n;
    *reinterpret_cast<float4*>(dst) = make_float4(__fadd_rn(acc[0], o.x), __fadd_rn(acc[1], o.y),
                                                  __fadd_rn(acc[2], o.z), __fadd_rn(acc[3], o.w));
  }
}

// sum of partial[split][m][col] over the splits, in split order; loads issued 8 at a time
__device__ __forceinline__ float split_sum(const float* __restrict__ partial, int splits, int64_t stride) {
  float sum = 0.0f;
  int sp = 0;
  for (; sp + 8 <= splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[(int64_t)(sp + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum = __fadd_rn(sum, v[u]);
  }
  for (; sp < splits; ++sp) sum = __fadd_rn(sum, partial[(int64_t)sp * stride]);
  return sum;
}

// Y[m][n] = bf16( sum over splits of partial[split][m][n] + sum_j Ts[m][j] B[j][n] ),
// Ts = bf16(s T), T = sum over adapter slices of tpartial[slice][m][j] (formed again by every
// workgroup: there are few slices); block 0 also writes T_save = bf16(T).  A workgroup covers
// 64 columns; B's rows for them are staged in LDS; thread t takes column t % 64 for the
// tokens m = t / 64 (mod 4).
__global__ __launch_bounds__(256) void k_gemv_epilogue(const float* __restrict__ partial, int splits,
                                                       const float* __restrict__ tpartial, int asplits, int64_t M,
                                                       int64_t N, int64_t npad, int64_t rp,
                                                       const uint16_t* __restrict__ B, int64_t r, float scale,
                                                       uint16_t* __restrict__ Y, uint16_t* __restrict__ T_save) {
  __shared__ float sTs[16 * 256];
  __shared__ __attribute__((aligned(16))) uint16_t sB[256 * 64];
  const int t = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  // B rows j < r, columns n0.. (8-column chunks past N or rows past r read as zero)
  for (int idx = t; idx < (int)rp * 8; idx += 256) {
    const int jj = idx >> 3, q = idx & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (jj < r && n0 + q * 8 < N) v = *reinterpret_cast<const uint4*>(B + jj * N + n0 + q * 8);
    *reinterpret_cast<uint4*>(sB + jj * 64 + q * 8) = v;
  }
  for (int base = 0; base < (int)(M * rp); base += 4 * 256) {   // four independent sums in flight
    float sum[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + u * 256 + t;
      sum[u] = idx < (int)(M * rp) ? split_sum(tpartial + idx, asplits, M * rp) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + u * 256 + t;
      if (idx < (int)(M * rp)) {
        const int m = idx / (int)rp, jj = idx - m * (int)rp;
        sTs[m * 256 + jj] = jj < r ? bf16_to_f32(f32_to_bf16_bits(__fmul_rn(scale, sum[u]))) : 0.0f;
        if (T_save && blockIdx.x == 0 && jj < r) T_save[m * r + jj] = (uint16_t)f32_to_bf16_bits(sum[u]);
      }
    }
  }
  __syncthreads();
  const int c = t & 63, mq = t >> 6;
  const int64_t n = n0 + c;
  if (n >= N) return;
  // sums over the splits in split order, the loads of 4 splits x 4 tokens in flight together
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, lora[4] = {0.f, 0.f, 0.f, 0.f};
  const int mcap = (int)M - 1;
  int sp = 0;
  for (; sp + 4 <= splits; sp += 4) {
    float v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) v[u][q] = partial[((int64_t)(sp + u) * M + min(mq + 4 * q, mcap)) * npad + n];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __fadd_rn(acc[q], v[u][q]);
  }
  for (; sp < splits; ++sp) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __fadd_rn(acc[q], partial[((int64_t)sp * M + min(mq + 4 * q, mcap)) * npad + n]);
  }
  for (int jj = 0; jj < (int)r; ++jj) {
    const float b = bf16_to_f32(sB[jj * 64 + c]);
#pragma unroll
    for (int q = 0; q < 4; ++q) lora[q] = __builtin_fmaf(sTs[(mq + 4 * q) * 256 + jj], b, lora[q]);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = mq + 4 * q;
    if (m < M) Y[m * N + n] = (uint16_t)f32_to_bf16_bits(__fadd_rn(acc[q], lora[q]));
  }
}

}  // namespace

// Weight slices of whole 4-block steps and adapter slices of up to 512 rows of A.  Three
// workgroups are resident per CU (768 on the chip): the grid is sized to fill whole rounds of
// those slots (one round when the X slice fits, else as many full rounds as the LDS cap on
// the X slice, GMAX_X elements, needs).
GemvPlan gemv_plan(int64_t M, int64_t K, int64_t N, int64_t rp) {
  constexpr int64_t kSlots = 768;
  const int64_t nkb = K / 64;
  const int64_t Mm = std::max<int64_t>(M, 1);
  GemvPlan pl;
  pl.wgroups = (N + GROWS - 1) / GROWS;
  pl.agroups = rp / GROWS;
  pl.npad = pl.wgroups * GROWS;
  const int64_t aw = pl.agroups * ((K + KA - 1) / KA);
  const int64_t kb_cap = std::max<int64_t>(4, (GMAX_X / (Mm * 64)) / 4 * 4);   // LDS for the X slice
  const int64_t s_min = (nkb + kb_cap - 1) / kb_cap;
  const int64_t rounds = std::max<int64_t>(1, (pl.wgroups * s_min + aw + kSlots - 1) / kSlots);
  int64_t s = std::max<int64_t>(s_min, (rounds * kSlots - aw) / pl.wgroups);
  s = std::max<int64_t>(1, std::min<int64_t>(s, nkb));
  int64_t kbps = (nkb + s - 1) / s;
  kbps = std::min<int64_t>((kbps + 3) / 4 * 4, kb_cap);
  pl.kb_per_split = kbps;
  pl.splits = (int)((nkb + kbps - 1) / kbps);
  pl.ka = KA;
  pl.asplits = (int)((K + KA - 1) / KA);
  pl.tpart = (size_t)pl.splits * Mm * pl.npad;
  return pl;
}

size_t gemv_partial_floats(const GemvPlan& pl, int64_t M) {
  return pl.tpart + (size_t)pl.asplits * M * pl.agroups * GROWS;
}

hipError_t launch_gemv(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w, const uint16_t* A,
                       int64_t r, const GemvPlan& pl, float* partial, hipStream_t s) {
  const uint64_t nblk = (uint64_t)N * K / 64;
  GemvParams p{X, M, K, N, w, nblk * kBlockBytes, w.dq ? nblk : nblk * 4, w.dq ? ((nblk + 255) / 256) * 4 : 0,
               A, r, partial, partial + pl.tpart, pl.npad, pl.agroups * GROWS, pl.kb_per_split, pl.splits,
               pl.wgroups, pl.agroups, pl.ka, pl.asplits, nf4_table()};
  // weight groups: X slice, then the block scales; adapter groups: two A chunks and two X chunks
  const size_t lds = std::max<size_t>((size_t)M * (pl.kb_per_split * 8 + 1) * 16 + (size_t)(GROWS * pl.kb_per_split + 4) * 4,
                                      (size_t)2 * ACH * 64 * 2 + (size_t)2 * 16 * XAS * 2);
  ProfScope ps("k_fwd_nf4_gemv", s);
  const dim3 grid((unsigned)(pl.wgroups * pl.splits + pl.agroups * pl.asplits));
  if (w.dq)
    hipLaunchKernelGGL(k_fwd_nf4_gemv<true>, grid, dim3(GT), lds, s, p);
  else
    hipLaunchKernelGGL(k_fwd_nf4_gemv<false>, grid, dim3(GT), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_gemv_epilogue(const float* partial, const GemvPlan& pl, int64_t M, int64_t N, const uint16_t* B,
                                int64_t r, float scale, uint16_t* Y, uint16_t* T_save, hipStream_t s) {
  ProfScope ps("k_gemv_epilogue", s);
  hipLaunchKernelGGL(k_gemv_epilogue, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, s, partial, pl.splits,
                     partial + pl.tpart, pl.asplits, M, N, pl.npad, pl.agroups * GROWS, B, r, scale, Y, T_save);
  return hipGetLastError();
}

}  // namespace qlora
