// Small rank-r products of the adapter path ("QLoRA: Efficient Finetuning of
// Quantized LLMs", section "The QLoRA layer, end to end", the one-layer listing):
//   T = X L1 (forward), G = dY L2^T, dL1 = s X^T G, dL2 = s T^T dY (backward).
// Each has one dimension equal to the rank r (<= 256): the output is small and the
// reduction long.  The reduction is split over workgroups, each writing its fp32
// partial tile; a second kernel adds the partials in split order (so the result
// does not depend on timing) and writes the bf16 / fp32 outputs.  The hand-off goes
// through a kernel boundary: on this GPU each XCD has its own L2, and an in-kernel
// device-scope fence would write back and invalidate it.
//
// Tiles are 64 x 64, 64 deep per step, on v_mfma_f32_16x16x32_bf16, with both operand
// tiles double-buffered in LDS; the loads of up to eight steps are in flight at once.  An operand stored contiguously along the reduction ("KC") is kept as
// [row][k] and read with 16-byte LDS loads; one stored contiguously along its row index
// is kept as stored ([k][row]) and read with transposing loads (ds_read_b64_tr_b16).
// Loads go through raw buffer resources with explicit masks: elements past the ends of
// the reduction or of the rows read as zero.
#include "common.h"
#include "gemm_core.h"
#include "kernels.h"

#include <algorithm>

namespace qlora {

namespace {

using gemm::i16x4;
using gemm::ld16;
using gemm::make_rsrc;
using gemm::rsrc_t;

constexpr int TI = 64, TJ = 64, TK = 64;
constexpr int CH = 8;   // steps per batch of loads (even: the LDS buffer of step q is q % 2)

// [row][k] tile (128-byte rows of eight 16-byte chunks): chunk c of row r at c ^ ((r >> 1) & 7);
// 16 consecutive rows of one chunk (a fragment read) and 2 rows x 8 chunks (a store) are
// conflict-free.
__device__ __forceinline__ int kcpos(int row, int c) { return row * 64 + ((c ^ ((row >> 1) & 7)) << 3); }
// [k][row] tile: chunk q of k-row k at q ^ 2 f(k), f(k) = ((k >> 1) & 1) | ((k >> 2) & 2):
// transposing reads (4 k-rows x 32 bytes per 16 lanes, two such quads 8 apart per 32 lanes)
// and stores (2 k-rows x 8 chunks) are conflict-free.
__device__ __forceinline__ int trpos(int k, int q) {
  const int f = ((k >> 1) & 1) | ((k >> 2) & 2);
  return k * 64 + ((q ^ (f << 1)) << 3);
}

// One operand of a product: element (o, k) (o = row index i or column index j) at
// P[o * ld + k] when KC, else P[k * ld + o]; o < nout, k < K.
struct Operand {
  rsrc_t r;
  uint32_t end;
  int64_t ld, nout;
};

template <bool KC>
__device__ __forceinline__ void load_panel(uint4 (&v)[2], const Operand& op, int64_t o0, int64_t k0, int64_t kend) {
  const int t = threadIdx.x;
  const int lr = t >> 3, lc = t & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int mr = lr + 32 * h;
    int64_t o, k;
    if constexpr (KC) {
      o = o0 + mr;
      k = k0 + lc * 8;
    } else {
      k = k0 + mr;
      o = o0 + lc * 8;
    }
    const bool valid = o < op.nout && k < kend;   // nout % 8 == 0 (!KC), kend % 8 == 0 (KC)
    const int64_t off = KC ? (o * op.ld + k) * 2 : (k * op.ld + o) * 2;
    v[h] = ld16(op.r, valid ? (uint32_t)off : op.end);
  }
}

template <bool KC>
__device__ __forceinline__ void store_panel(const uint4 (&v)[2], uint16_t* __restrict__ lds) {
  const int t = threadIdx.x;
  const int lr = t >> 3, lc = t & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    *reinterpret_cast<uint4*>(lds + (KC ? kcpos(lr + 32 * h, lc) : trpos(lr + 32 * h, lc))) = v[h];
}

// 16x16x32 operand: rows ob + lane % 16, reduction ks*32 + 8 (lane / 16) .. +7
template <bool KC>
__device__ __forceinline__ u32x4 read_frag(const uint16_t* __restrict__ lds, int ob, int ks) {
  const int lane = threadIdx.x & 63;
  if constexpr (KC) {
    return *reinterpret_cast<const u32x4*>(lds + kcpos(ob + (lane & 15), ks * 4 + (lane >> 4)));
  } else {
    const int j = lane & 15, G = lane >> 4;
    const int kr = ks * 32 + G * 8 + (j >> 2);
    const int col = ob + (j & 3) * 4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds + trpos(kr, col >> 3) + (col & 7)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds + trpos(kr + 4, col >> 3) + (col & 7)));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    u32x4 o;
    o.x = a.x; o.y = a.y; o.z = b.x; o.w = b.y;
    return o;
  }
}

__device__ __forceinline__ void epi_write(const LoraEpi& ep, int64_t I, int64_t J, int64_t i, int64_t j, float sum) {
  if (i >= I) return;
  if (j < J) {
    if (ep.out_a) ep.out_a[i * ep.lda + j] = (uint16_t)f32_to_bf16_bits(__fmul_rn(ep.scale_a, sum));
    if (ep.out_b) ep.out_b[i * ep.ldb + j] = (uint16_t)f32_to_bf16_bits(__fmul_rn(ep.scale_b, sum));
    if (ep.out_f) ep.out_f[i * J + j] = __fmul_rn(ep.scale_f, sum);
  } else if (ep.out_b && j < ep.ldb) {
    ep.out_b[i * ep.ldb + j] = 0;   // zero padding up to the padded rank
  }
}

template <bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) void k_lora_gemm(LoraProblem p0, LoraProblem p1, int nprob) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][TI * TK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][TJ * TK];

  // which problem, tile and split this workgroup owns
  int64_t wg = blockIdx.x;
  const int64_t n0 = p0.tiles_i * p0.tiles_j * p0.splits;
  const LoraProblem& P = (nprob > 1 && wg >= n0) ? p1 : p0;
  if (nprob > 1 && wg >= n0) wg -= n0;
  const SmallGemm& g = P.g;
  const int split = (int)(wg % P.splits);
  const int64_t tile = wg / P.splits;
  const int64_t ti = tile / P.tiles_j, tj = tile - ti * P.tiles_j;
  const int64_t i0 = ti * TI, j0 = tj * TJ;
  const int64_t kbeg = (int64_t)split * P.k_per_split;
  const int64_t kend = min(g.K, kbeg + P.k_per_split);
  const int nsteps = (int)((kend - kbeg + TK - 1) / TK);

  // operand extents (largest element index + 1) bound the buffer resources
  const uint64_t a_ext = (uint64_t)((g.I - 1) * g.a_si + (g.K - 1) * g.a_sk + 1);
  const uint64_t b_ext = (uint64_t)((g.K - 1) * g.b_sk + (g.J - 1) * g.b_sj + 1);
  const Operand oa{make_rsrc(g.A, a_ext * 2), (uint32_t)(a_ext * 2), A_KC ? g.a_si : g.a_sk, g.I};
  const Operand ob{make_rsrc(g.B, b_ext * 2), (uint32_t)(b_ext * 2), B_KC ? g.b_sj : g.b_sk, g.J};

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wi = wave & 1, wj = wave >> 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The loads of up to CH steps are issued together (a step past the split's end reads
  // zeros without touching memory), so a workgroup waits for memory once per CH steps;
  // the LDS tiles are double-buffered with one barrier per step.
  for (int c0 = 0; c0 < nsteps; c0 += CH) {
    uint4 va[CH][2], vb[CH][2];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int64_t k = kbeg + (int64_t)(c0 + q) * TK;
      load_panel<A_KC>(va[q], oa, i0, k, kend);
      load_panel<B_KC>(vb[q], ob, j0, k, kend);
    }
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (c0 + q >= nsteps) break;
      const int cb = q & 1;
      store_panel<A_KC>(va[q], sA[cb]);
      store_panel<B_KC>(vb[q], sB[cb]);
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 af[2], bfr[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) af[a] = read_frag<A_KC>(sA[cb], wi * 32 + a * 16, ks);
#pragma unroll
        for (int b = 0; b < 2; ++b) bfr[b] = read_frag<B_KC>(sB[cb], wj * 32 + b * 16, ks);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
      }
    }
  }

  // acc[a][b][v] = C[i = wi*32 + a*16 + 4*(lane/16) + v][j = wj*32 + b*16 + lane%16]
  if (P.splits == 1) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          epi_write(P.ep, g.I, g.J, i0 + wi * 32 + a * 16 + 4 * (lane >> 4) + v, j0 + wj * 32 + b * 16 + (lane & 15),
                    acc[a][b][v]);
    return;
  }
  // split reduction: every split stores its whole 64x64 partial tile (zeros past the edges)
  float* part = P.partial + (tile * P.splits + split) * (TI * TJ);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        part[(wi * 32 + a * 16 + 4 * (lane >> 4) + v) * TJ + wj * 32 + b * 16 + (lane & 15)] = acc[a][b][v];
}

// Four consecutive outputs of one row: a single 8-byte (bf16) or 16-byte (fp32) store where
// the destination is aligned, else element stores.
__device__ __forceinline__ void store4_bf16(uint16_t* dst, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  if ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(a | (b << 16), c | (d << 16));
  } else {
    dst[0] = (uint16_t)a; dst[1] = (uint16_t)b; dst[2] = (uint16_t)c; dst[3] = (uint16_t)d;
  }
}

__device__ __forceinline__ void epi_write4(const LoraEpi& ep, int64_t I, int64_t J, int64_t i, int64_t j,
                                           const float4& v) {
  if (i >= I) return;
  if (j + 4 > J) {   // the rank's ragged edge (and padding columns up to ldb)
    epi_write(ep, I, J, i, j + 0, v.x);
    epi_write(ep, I, J, i, j + 1, v.y);
    epi_write(ep, I, J, i, j + 2, v.z);
    epi_write(ep, I, J, i, j + 3, v.w);
    return;
  }
  auto bf = [](float sc, float x) { return f32_to_bf16_bits(__fmul_rn(sc, x)); };
  if (ep.out_a)
    store4_bf16(ep.out_a + i * ep.lda + j, bf(ep.scale_a, v.x), bf(ep.scale_a, v.y), bf(ep.scale_a, v.z),
                bf(ep.scale_a, v.w));
  if (ep.out_b)
    store4_bf16(ep.out_b + i * ep.ldb + j, bf(ep.scale_b, v.x), bf(ep.scale_b, v.y), bf(ep.scale_b, v.z),
                bf(ep.scale_b, v.w));
  if (ep.out_f) {
    float* dst = ep.out_f + i * J + j;
    const float4 o = make_float4(__fmul_rn(ep.scale_f, v.x), __fmul_rn(ep.scale_f, v.y), __fmul_rn(ep.scale_f, v.z),
                                 __fmul_rn(ep.scale_f, v.w));
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
      *reinterpret_cast<float4*>(dst) = o;
    } else {
      dst[0] = o.x; dst[1] = o.y; dst[2] = o.z; dst[3] = o.w;
    }
  }
}

// Sum of the split partials in split order, then the outputs.  Four consecutive
// elements of a tile row per thread.  S (2, 4, 8 or 16) bounds the splits of both problems:
// every thread issues exactly S loads (indices past the last split repeat it, unused) before
// the first add, so it waits for memory once.
template <int S>
__global__ __launch_bounds__(256) void k_lora_reduce(LoraProblem p0, LoraProblem p1, int nprob) {
  const int64_t per = p0.tiles_i * p0.tiles_j * (TI * TJ / 4);
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool second = nprob > 1 && idx >= per;
  const LoraProblem& P = second ? p1 : p0;
  if (second) idx -= per;
  if (idx >= P.tiles_i * P.tiles_j * (TI * TJ / 4)) return;
  const int64_t tile = idx / (TI * TJ / 4);
  const int e = (int)(idx - tile * (TI * TJ / 4)) * 4;
  const int64_t ti = tile / P.tiles_j, tj = tile - ti * P.tiles_j;
  const float* base = P.partial + tile * P.splits * (TI * TJ) + e;
  float4 v[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp)
    v[sp] = *reinterpret_cast<const float4*>(base + min(sp, P.splits - 1) * (TI * TJ));
  float4 sum = v[0];
#pragma unroll
  for (int sp = 1; sp < S; ++sp) {
    if (sp < P.splits) {
      sum.x = __fadd_rn(sum.x, v[sp].x);
      sum.y = __fadd_rn(sum.y, v[sp].y);
      sum.z = __fadd_rn(sum.z, v[sp].z);
      sum.w = __fadd_rn(sum.w, v[sp].w);
    }
  }
  epi_write4(P.ep, P.g.I, P.g.J, ti * TI + e / TJ, tj * TJ + e % TJ, sum);
}

}  // namespace

LoraProblem lora_problem(const SmallGemm& g, const LoraEpi& ep, int max_splits) {
  LoraProblem p;
  p.g = g;
  p.ep = ep;
  p.tiles_i = (g.I + TI - 1) / TI;
  p.tiles_j = (g.J + TJ - 1) / TJ;
  const int64_t tiles = p.tiles_i * p.tiles_j;
  const int64_t ksteps = (g.K + TK - 1) / TK;
  int64_t s = (256 + tiles - 1) / tiles;   // about one workgroup per compute unit
  if (s > ksteps / 4) s = ksteps / 4;      // keep at least 4 steps per split
  if (s > max_splits) s = max_splits;
  if (s > kMaxLoraSplits) s = kMaxLoraSplits;
  if (s < 1) s = 1;
  int64_t kps = (ksteps + s - 1) / s * TK;
  p.splits = (int)((g.K + kps - 1) / kps);
  if (p.splits < 1) p.splits = 1;
  p.k_per_split = kps;
  p.partial = nullptr;
  return p;
}

size_t lora_partial_floats(const LoraProblem& p) {
  return p.splits > 1 ? (size_t)(p.tiles_i * p.tiles_j * p.splits) * TI * TJ : 0;
}

hipError_t launch_lora(const LoraProblem& p0, const LoraProblem* p1, const char* name, hipStream_t s) {
  const int64_t n = p0.tiles_i * p0.tiles_j * p0.splits + (p1 ? p1->tiles_i * p1->tiles_j * p1->splits : 0);
  const bool akc = p0.g.a_sk == 1, bkc = p0.g.b_sk == 1;
  const LoraProblem q1 = p1 ? *p1 : p0;
  const int nprob = p1 ? 2 : 1;
  ProfScope ps(name, s);
  if (akc && bkc)
    hipLaunchKernelGGL((k_lora_gemm<true, true>), dim3((unsigned)n), dim3(256), 0, s, p0, q1, nprob);
  else if (akc && !bkc)
    hipLaunchKernelGGL((k_lora_gemm<true, false>), dim3((unsigned)n), dim3(256), 0, s, p0, q1, nprob);
  else if (!akc && bkc)
    hipLaunchKernelGGL((k_lora_gemm<false, true>), dim3((unsigned)n), dim3(256), 0, s, p0, q1, nprob);
  else
    hipLaunchKernelGGL((k_lora_gemm<false, false>), dim3((unsigned)n), dim3(256), 0, s, p0, q1, nprob);
  return hipGetLastError();
}

hipError_t launch_lora_reduce(const LoraProblem& p0, const LoraProblem* p1, const char* name, hipStream_t s) {
  const LoraProblem q1 = p1 ? *p1 : p0;
  const int nprob = p1 ? 2 : 1;
  const int64_t n = (p0.tiles_i * p0.tiles_j + (p1 ? p1->tiles_i * p1->tiles_j : 0)) * (TI * TJ / 4);
  const int most = std::max(p0.splits, p1 ? p1->splits : 1);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  ProfScope ps(name, s);
  if (most <= 2) hipLaunchKernelGGL(k_lora_reduce<2>, grid, block, 0, s, p0, q1, nprob);
  else if (most <= 4) hipLaunchKernelGGL(k_lora_reduce<4>, grid, block, 0, s, p0, q1, nprob);
  else if (most <= 8) hipLaunchKernelGGL(k_lora_reduce<8>, grid, block, 0, s, p0, q1, nprob);
  else hipLaunchKernelGGL(k_lora_reduce<kMaxLoraSplits>, grid, block, 0, s, p0, q1, nprob);
  return hipGetLastError();
}

}  // namespace qlora
