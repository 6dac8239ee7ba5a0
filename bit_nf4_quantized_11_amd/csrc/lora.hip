// Small rank-r products of the adapter path ("QLoRA: Efficient Finetuning of
// Quantized LLMs", section "The QLoRA layer, end to end", the one-layer listing):
//   T = X L1 (forward), G = dY L2^T, dL1 = s X^T G, dL2 = s T^T dY (backward).
// Each has one dimension equal to the rank r (<= 256), so the output is small and
// the reduction long: split-K over the reduction into fp32 partials, then a
// reduction kernel that sums the splits in a fixed order (deterministic) and
// writes bf16 and/or fp32 results.  Tiles of 64 x 64 x 32 on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16), both operands staged through LDS with the
// reduction index contiguous, whichever layout the operand has in memory.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int TI = 64, TJ = 64, TK = 32, LDK = TK + 8;   // LDS row: 40 bf16 = 80 bytes

// Stage a 64 x 32 tile (rows = i or j, columns = k) into LDS, k contiguous.
// src(row, k) = P[row * s_row + k * s_k]; exactly one stride is 1 (template).
template <bool K_CONTIG>
__device__ __forceinline__ void stage(uint16_t* __restrict__ lds, const uint16_t* __restrict__ P, int64_t s_row,
                                      int64_t s_k, int64_t row0, int64_t nrow, int64_t k0, int64_t kend) {
  const int t = threadIdx.x;
  if (K_CONTIG) {
    const int row = t >> 2, kc = (t & 3) * 8;
    const int64_t gr = row0 + row, gk = k0 + kc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gr < nrow && gk < kend) v = *reinterpret_cast<const uint4*>(P + gr * s_row + gk);   // kend % 8 == 0
    *reinterpret_cast<uint4*>(lds + row * LDK + kc) = v;
  } else {
    const int k = t >> 3, rc = (t & 7) * 8;
    const int64_t gk = k0 + k, gr = row0 + rc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gk < kend && gr < nrow) v = *reinterpret_cast<const uint4*>(P + gk * s_k + gr);       // nrow % 8 == 0
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lds[(rc + 2 * e) * LDK + k] = (uint16_t)(w[e] & 0xFFFFu);
      lds[(rc + 2 * e + 1) * LDK + k] = (uint16_t)(w[e] >> 16);
    }
  }
}

template <bool A_KC, bool B_KC>
__global__ __launch_bounds__(256) void k_lora_splitk(SmallGemm g, float* __restrict__ partial, int64_t k_per_split) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[TI * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[TJ * LDK];
  const int64_t i0 = (int64_t)blockIdx.x * TI, j0 = (int64_t)blockIdx.y * TJ;
  const int split = blockIdx.z;
  const int64_t kbeg = split * k_per_split;
  const int64_t kend = min(g.K, kbeg + k_per_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wi = wave & 1, wj = wave >> 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kbeg; k0 < kend; k0 += TK) {
    // A(i,k): rows i, stride along k is a_sk; B(k,j): rows j, stride along k is b_sk
    stage<A_KC>(sA, g.A, g.a_si, g.a_sk, i0, g.I, k0, kend);
    stage<B_KC>(sB, g.B, g.b_sj, g.b_sk, j0, g.J, k0, kend);
    __syncthreads();
    u32x4 af[2], bfr[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
      af[a] = *reinterpret_cast<const u32x4*>(sA + (wi * 32 + a * 16 + (lane & 15)) * LDK + (lane >> 4) * 8);
#pragma unroll
    for (int b = 0; b < 2; ++b)
      bfr[b] = *reinterpret_cast<const u32x4*>(sB + (wj * 32 + b * 16 + (lane & 15)) * LDK + (lane >> 4) * 8);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = mfma16(af[a], bfr[b], acc[a][b]);
    __syncthreads();
  }
  // acc[a][b][v] = C[i = wi*32 + a*16 + 4*(lane/16) + v][j = wj*32 + b*16 + lane%16]
  float* out = partial + (int64_t)split * g.I * g.J;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + wi * 32 + a * 16 + 4 * (lane >> 4) + v;
        const int64_t j = j0 + wj * 32 + b * 16 + (lane & 15);
        if (i < g.I && j < g.J) out[i * g.J + j] = acc[a][b][v];
      }
}

__global__ __launch_bounds__(256) void k_lora_reduce(const float* __restrict__ partial, int splits, int64_t I,
                                                     int64_t J, uint16_t* __restrict__ out_a, int64_t lda,
                                                     float scale_a, uint16_t* __restrict__ out_b, int64_t ldb,
                                                     float scale_b, float* __restrict__ out_f, float scale_f) {
  const int64_t cols = out_b ? max(J, ldb) : J;
  const int64_t n = I * cols;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / cols, j = idx - i * cols;
    if (j >= J) {   // zero padding of the second bf16 output
      out_b[i * ldb + j] = 0;
      continue;
    }
    float sum = 0.0f;
    for (int s = 0; s < splits; ++s) sum = __fadd_rn(sum, partial[(int64_t)s * I * J + i * J + j]);
    if (out_a) out_a[i * lda + j] = (uint16_t)f32_to_bf16_bits(__fmul_rn(scale_a, sum));
    if (out_b) out_b[i * ldb + j] = (uint16_t)f32_to_bf16_bits(__fmul_rn(scale_b, sum));
    if (out_f) out_f[i * J + j] = __fmul_rn(scale_f, sum);
  }
}

int64_t k_per_split_for(const SmallGemm& g, int splits) {
  int64_t kps = (g.K + splits - 1) / splits;
  kps = (kps + TK - 1) / TK * TK;
  return kps;
}

}  // namespace

int small_gemm_splits(const SmallGemm& g) {
  const int64_t tiles = ((g.I + TI - 1) / TI) * ((g.J + TJ - 1) / TJ);
  const int64_t ksteps = (g.K + TK - 1) / TK;
  int64_t s = (512 + tiles - 1) / tiles;   // aim for about 512 workgroups
  if (s > ksteps / 4) s = ksteps / 4;      // keep at least 4 k-steps per split
  if (s > 16) s = 16;                      // bound the fp32 partial traffic
  if (s < 1) s = 1;
  return (int)s;
}

size_t small_gemm_partial_floats(const SmallGemm& g) {
  return (size_t)small_gemm_splits(g) * (size_t)g.I * (size_t)g.J;
}

hipError_t launch_small_gemm(const SmallGemm& g, float* partial, int splits, const char* name, hipStream_t s) {
  const int64_t kps = k_per_split_for(g, splits);
  const int used = (int)((g.K + kps - 1) / kps);
  // splits that would be empty still write zeros: launch them with an empty range
  dim3 grid((unsigned)((g.I + TI - 1) / TI), (unsigned)((g.J + TJ - 1) / TJ), (unsigned)splits);
  (void)used;
  const bool akc = g.a_sk == 1, bkc = g.b_sk == 1;
  ProfScope ps(name, s);
  if (akc && bkc)
    hipLaunchKernelGGL((k_lora_splitk<true, true>), grid, dim3(256), 0, s, g, partial, kps);
  else if (akc && !bkc)
    hipLaunchKernelGGL((k_lora_splitk<true, false>), grid, dim3(256), 0, s, g, partial, kps);
  else if (!akc && bkc)
    hipLaunchKernelGGL((k_lora_splitk<false, true>), grid, dim3(256), 0, s, g, partial, kps);
  else
    hipLaunchKernelGGL((k_lora_splitk<false, false>), grid, dim3(256), 0, s, g, partial, kps);
  return hipGetLastError();
}

hipError_t launch_small_reduce(const float* partial, int splits, int64_t I, int64_t J, uint16_t* out_a, int64_t lda,
                               float scale_a, uint16_t* out_b, int64_t ldb, float scale_b, float* out_f,
                               float scale_f, const char* name, hipStream_t s) {
  const int64_t cols = out_b ? (J > ldb ? J : ldb) : J;
  const int64_t n = I * cols;
  if (n <= 0) return hipSuccess;
  int64_t grid = (n + 255) / 256;
  if (grid > 8192) grid = 8192;
  ProfScope ps(name, s);
  hipLaunchKernelGGL(k_lora_reduce, dim3((unsigned)grid), dim3(256), 0, s, partial, splits, I, J, out_a, lda, scale_a,
                     out_b, ldb, scale_b, out_f, scale_f);
  return hipGetLastError();
}

}  // namespace qlora
