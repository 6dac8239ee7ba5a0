// Adapter merge ("QLoRA: quantising the part you are not training", section "What it
// costs": merging the adapter into the quantised base means requantising):
//   W'[n][k] = bf16( deq(W)[n][k] + s * sum_j A[k][j] B[j][n] ),
// the weight a plain linear layer would need to reproduce base + adapter.  The result is
// bf16 [out][in] and can be quantized again with qlora_quantize_nf4 (the requantization
// the page warns about).
//
// Arithmetic per element: d = fp32 fused multiply-add chain over j = 0..r-1 of A[k][j] B[j][n]
// (bf16 inputs, exact products), u = fl32(s d), W' = bf16_RNE(fl32(deq + u)) with deq the
// bf16 dequantized weight ("doubleDequant").  One workgroup per 64 x 64 tile: rows of B and
// of A^T for the tile staged in LDS, each thread 4 rows x 4 consecutive columns (one 64-element
// code chunk per row: the 4 codes of a thread are the low or high nibbles of one code dword).
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int MT = 256;      // threads
constexpr int RMAX = 256;    // largest rank

__global__ __launch_bounds__(MT) void k_merge_adapter(NF4View w, int64_t N, int64_t K, const uint16_t* __restrict__ A,
                                                      const uint16_t* __restrict__ B, int r, float scale,
                                                      uint16_t* __restrict__ out, NF4Table tab) {
  __shared__ __attribute__((aligned(16))) uint16_t sB[RMAX * 64];    // [j][n - n0]
  __shared__ __attribute__((aligned(16))) uint16_t sAt[RMAX * 64];   // [j][k - k0]
  __shared__ float lv[16];
  const int t = threadIdx.x;
  const int64_t tiles_k = K / 64;
  const int64_t n0 = (int64_t)(blockIdx.x / tiles_k) * 64, k0 = (int64_t)(blockIdx.x % tiles_k) * 64;
  if (t < 16) lv[t] = tab.level[t];
  // stage: B rows j, columns n0..n0+63 (zero past N); A rows k0..k0+63 transposed
  for (int idx = t; idx < r * 64; idx += MT) {
    const int j = idx >> 6, c = idx & 63;
    sB[j * 64 + c] = n0 + c < N ? B[(int64_t)j * N + n0 + c] : (uint16_t)0;
    sAt[j * 64 + c] = A[(k0 + c) * (int64_t)r + j];
  }
  __syncthreads();
  const int rn = (t >> 4) * 4, ck = (t & 15) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = 0.0f;
  for (int j = 0; j < r; ++j) {
    const uint2 bb = *reinterpret_cast<const uint2*>(sB + j * 64 + rn);
    const uint2 aa = *reinterpret_cast<const uint2*>(sAt + j * 64 + ck);
    const float b[4] = {bf16_to_f32(bb.x & 0xFFFFu), bf16_to_f32(bb.x >> 16), bf16_to_f32(bb.y & 0xFFFFu),
                        bf16_to_f32(bb.y >> 16)};
    const float a[4] = {bf16_to_f32(aa.x & 0xFFFFu), bf16_to_f32(aa.x >> 16), bf16_to_f32(aa.y & 0xFFFFu),
                        bf16_to_f32(aa.y >> 16)};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[i][c] = __builtin_fmaf(a[c], b[i], acc[i][c]);
  }
  // dequantize the thread's 4 weights of each of its 4 rows and add the adapter term
  const int g = ck >> 3, hi = (ck >> 2) & 1;     // code group of the 4 columns, low or high nibbles
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + rn + i;
    if (n >= N) continue;
    const int64_t chunk = n * tiles_k + k0 / 64;                 // 64-element code chunk
    const float s = block_scale(w, (n * K + k0 + ck) >> w.bshift);   // the 4 columns share a block
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(w.codes + chunk * kBlockBytes + g * 4);
    uint32_t o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t code = (cw >> (8 * c + 4 * hi)) & 15u;
      const float deq = bf16_to_f32(f32_to_bf16_bits(__fmul_rn(lv[code], s)));
      o[c] = f32_to_bf16_bits(__fadd_rn(deq, __fmul_rn(scale, acc[i][c])));
    }
    uint2 v;
    v.x = o[0] | (o[1] << 16);
    v.y = o[2] | (o[3] << 16);
    *reinterpret_cast<uint2*>(out + n * K + k0 + ck) = v;
  }
}

}  // namespace

hipError_t launch_merge_adapter(const NF4View& w, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int64_t r,
                                float scale, uint16_t* out, hipStream_t s) {
  const int64_t tiles = ((N + 63) / 64) * (K / 64);
  ProfScope ps("k_merge_adapter", s);
  hipLaunchKernelGGL(k_merge_adapter, dim3((unsigned)tiles), dim3(MT), 0, s, w, N, K, A, B, (int)r, scale, out,
                     nf4_table(w.cb));
  return hipGetLastError();
}

}  // namespace qlora
