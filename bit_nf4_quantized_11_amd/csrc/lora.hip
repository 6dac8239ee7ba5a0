// Small rank-r products of the adapter path ("QLoRA: Efficient Finetuning of
// Quantized LLMs", section "The QLoRA layer, end to end", the one-layer listing):
//   T = X L1 (forward), G = dY L2^T, dL1 = s X^T G, dL2 = s T^T dY (backward).
// Each has one dimension equal to the rank r (<= 256): the output is small and the
// reduction long.  The reduction is split over workgroups, each writing its fp32
// partial tile; a second kernel adds the partials in split order (so the result
// does not depend on timing) and writes the bf16 / fp32 outputs.  The hand-off goes
// through a kernel boundary: on this GPU each XCD has its own L2, and an in-kernel
// device-scope fence would write back and invalidate it.  Tiles are 64 x 64, 64 deep per step, on
// v_mfma_f32_16x16x32_bf16; both operands go through LDS with the reduction
// index contiguous, whatever their layout in memory, and the next step's tiles are
// prefetched into registers while the current step computes.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int TI = 64, TJ = 64, TK = 64, LDK = TK + 8;   // LDS row: 72 bf16 = 144 bytes

// 64 rows x 64 reduction elements of an operand, staged per thread as two 8-element
// vectors.  K_CONTIG: vectors along the reduction; otherwise along the rows.
template <bool K_CONTIG>
struct Tile {
  uint4 v[2];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ P, int64_t s_row, int64_t s_k, int64_t row0,
                                       int64_t nrow, int64_t k0, int64_t kend) {
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v[h] = make_uint4(0, 0, 0, 0);
      if (K_CONTIG) {
        const int row = (t >> 3) + 32 * h, kc = (t & 7) * 8;
        const int64_t gr = row0 + row, gk = k0 + kc;
        if (gr < nrow && gk < kend) v[h] = *reinterpret_cast<const uint4*>(P + gr * s_row + gk);   // kend % 8 == 0
      } else {
        const int k = (t >> 3) + 32 * h, rc = (t & 7) * 8;
        const int64_t gk = k0 + k, gr = row0 + rc;
        if (gk < kend && gr < nrow) v[h] = *reinterpret_cast<const uint4*>(P + gk * s_k + gr);   // nrow % 8 == 0
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* __restrict__ lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (K_CONTIG) {
        const int row = (t >> 3) + 32 * h, kc = (t & 7) * 8;
        *reinterpret_cast<uint4*>(lds + row * LDK + kc) = v[h];
      } else {
        const int k = (t >> 3) + 32 * h, rc = (t & 7) * 8;
        const uint32_t w[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lds[(rc + 2 * e) * LDK + k] = (uint16_t)(w[e] & 0xFFFFu);
          lds[(rc + 2 * e + 1) * LDK + k] = (uint16_t)(w[e] >> 16);
        }
      }
    }
  }
};

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
  __shared__ __attribute__((aligned(16))) uint16_t sA[TI * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[TJ * LDK];

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

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wi = wave & 1, wj = wave >> 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  Tile<A_KC> ta;
  Tile<B_KC> tb;
  if (kbeg < kend) {
    ta.load(g.A, A_KC ? g.a_si : g.a_sk, A_KC ? 1 : g.a_sk, i0, g.I, kbeg, kend);
    tb.load(g.B, B_KC ? g.b_sj : g.b_sk, B_KC ? 1 : g.b_sk, j0, g.J, kbeg, kend);
  }
  for (int64_t k0 = kbeg; k0 < kend; k0 += TK) {
    ta.store(sA);
    tb.store(sB);
    __syncthreads();
    if (k0 + TK < kend) {   // prefetch the next step while this one computes
      ta.load(g.A, A_KC ? g.a_si : g.a_sk, A_KC ? 1 : g.a_sk, i0, g.I, k0 + TK, kend);
      tb.load(g.B, B_KC ? g.b_sj : g.b_sk, B_KC ? 1 : g.b_sk, j0, g.J, k0 + TK, kend);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *reinterpret_cast<const u32x4*>(sA + (wi * 32 + a * 16 + (lane & 15)) * LDK + ks * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bfr[b] = *reinterpret_cast<const u32x4*>(sB + (wj * 32 + b * 16 + (lane & 15)) * LDK + ks * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
    }
    __syncthreads();
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

// Sum of the split partials in split order, then the outputs.  Four consecutive
// elements of a tile row per thread.
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
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp = 0; sp < P.splits; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(base + sp * (TI * TJ));
    sum.x = __fadd_rn(sum.x, v.x);
    sum.y = __fadd_rn(sum.y, v.y);
    sum.z = __fadd_rn(sum.z, v.z);
    sum.w = __fadd_rn(sum.w, v.w);
  }
  const int64_t i = ti * TI + e / TJ, j = tj * TJ + e % TJ;
  epi_write(P.ep, P.g.I, P.g.J, i, j + 0, sum.x);
  epi_write(P.ep, P.g.I, P.g.J, i, j + 1, sum.y);
  epi_write(P.ep, P.g.I, P.g.J, i, j + 2, sum.z);
  epi_write(P.ep, P.g.I, P.g.J, i, j + 3, sum.w);
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
  if (s > ksteps / 2) s = ksteps / 2;      // keep at least 2 steps per split
  if (s > max_splits) s = max_splits;
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
  ProfScope ps(name, s);
  hipLaunchKernelGGL(k_lora_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p0, q1, nprob);
  return hipGetLastError();
}

}  // namespace qlora
