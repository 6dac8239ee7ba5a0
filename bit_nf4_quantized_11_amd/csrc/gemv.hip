// Forward for few tokens (M <= 16), where the layer is bound by streaming the
// packed weight from HBM ("QLoRA: Efficient Finetuning of Quantized LLMs",
// section "The QLoRA layer, end to end").
//
// Each wave owns 16 weight rows; every lane holds one whole 64-weight block
// (32 bytes of codes, one 16-byte load pair), builds that block's scaled bf16
// table in registers once and dequantizes its 64 weights with byte permutes.
// The 4 lane groups of a wave hold 4 consecutive blocks, so one MFMA
// (v_mfma_f32_16x16x32_bf16) takes 8 weights from each of 4 blocks; 8 MFMAs
// consume the 4 blocks.  The MFMA's reduction index is therefore a permutation of
// k, applied identically to the token operand read from LDS (tokens beyond M are
// zero).  Result C[n][m] per wave; each split writes its fp32 partial sums, and an
// epilogue kernel adds the splits in split order, adds the adapter term
// Ts[M][rp] B and rounds to bf16 once.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int GT = 256;          // threads per workgroup (4 waves x 16 rows = 64 rows)
constexpr int GROWS = 64;
constexpr int GMAX_KS = 2048;    // max reduction length per split (LDS: 16 x 2048 bf16 = 64 KB)

struct GemvParams {
  const uint16_t* X;
  int64_t M, K, N;
  NF4View w;
  float* partial;       // [groups][splits][M][64]
  int64_t kb_per_split;
  int splits;
  NF4Table tab;
};

// token row m, 16-byte chunk c of a [16][ks] LDS tile, XOR-swizzled on the low 3 bits
__device__ __forceinline__ int xsw(int m, int c) { return (c ^ (m & 7)); }

__global__ __launch_bounds__(GT) void k_fwd_nf4_gemv(GemvParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[16 * GMAX_KS];
  const int64_t nkb = p.K / 64;
  const int64_t grp_id = (int64_t)blockIdx.x / p.splits;
  const int split = (int)((int64_t)blockIdx.x - grp_id * p.splits);
  const int64_t n0 = grp_id * GROWS;
  const int64_t kb_beg = split * p.kb_per_split;
  const int64_t kb_end = min(nkb, kb_beg + p.kb_per_split);
  const int64_t nkb_s = kb_end - kb_beg;
  const int64_t kcols = nkb_s * 64;
  const int chunks = (int)(kcols / 8);   // 16-byte chunks per token row
  const int t = threadIdx.x;

  // stage X[0..M)[kb_beg*64 .. kb_end*64) into LDS
  for (int idx = t; idx < (int)p.M * chunks; idx += GT) {
    const int m = idx / chunks, c = idx - m * chunks;
    const uint4 v = *reinterpret_cast<const uint4*>(p.X + (int64_t)m * p.K + kb_beg * 64 + c * 8);
    *reinterpret_cast<uint4*>(sX + m * (GMAX_KS) + (xsw(m, c & 7) | (c & ~7)) * 8) = v;
  }
  __syncthreads();

  const int lane = t & 63, wave = t >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int64_t n = n0 + wave * 16 + row;
  const bool row_ok = n < p.N;
  const bool tok_ok = row < p.M;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};

  for (int64_t kb4 = 0; kb4 < nkb_s; kb4 += 4) {
    const int64_t kbl = kb4 + grp;   // local block index of this lane
    uint4 c0 = make_uint4(0, 0, 0, 0), c1 = make_uint4(0, 0, 0, 0);
    float sc = 0.0f;
    const bool ok = row_ok && kbl < nkb_s;
    if (ok) {
      const int64_t blk = n * nkb + kb_beg + kbl;
      const uint4* src = reinterpret_cast<const uint4*>(p.w.codes + blk * kBlockBytes);
      c0 = src[0];
      c1 = src[1];
      sc = block_scale(p.w, blk);
    }
    const Planes pl = make_planes(p.tab, sc);
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 wa = ok ? dequant8(pl, cw[c]) : u32x4{0u, 0u, 0u, 0u};
      u32x4 xb = {0u, 0u, 0u, 0u};
      if (tok_ok && kbl < nkb_s) {
        const int ch = (int)(kbl * 8 + c);
        xb = *reinterpret_cast<const u32x4*>(sX + row * GMAX_KS + (xsw(row, ch & 7) | (ch & ~7)) * 8);
      }
      acc = mfma16(wa, xb, acc);
    }
  }
  // acc[v] = C[n = n0 + wave*16 + 4*grp + v][m = row]; this split's partial tile is [M][64]
  float* part = p.partial + (grp_id * p.splits + split) * p.M * GROWS;
  if (tok_ok) {
    const float4 o = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(part + row * GROWS + wave * 16 + 4 * grp) = o;
  }
}

// Y[m][n] = bf16( sum over splits (in order) + sum_j Ts[m][j] B[j][n] ); one thread per output
__global__ __launch_bounds__(256) void k_gemv_epilogue(const float* __restrict__ partial, int splits, int64_t M,
                                                       int64_t N, const uint16_t* __restrict__ Ts, int64_t rp,
                                                       const uint16_t* __restrict__ B, int64_t r,
                                                       uint16_t* __restrict__ Y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over [groups][M][64]
  const int64_t per_group = M * GROWS;
  const int64_t grp_id = idx / per_group;
  const int e = (int)(idx - grp_id * per_group);
  const int m = e / GROWS, nl = e - m * GROWS;
  const int64_t n = grp_id * GROWS + nl;
  if (n >= N) return;
  const float* base = partial + grp_id * splits * per_group + e;
  float sum = 0.0f;
  for (int sp = 0; sp < splits; ++sp) sum = __fadd_rn(sum, base[sp * per_group]);
  float lora = 0.0f;
  for (int64_t j = 0; j < r; ++j) lora = __builtin_fmaf(bf16_to_f32(Ts[m * rp + j]), bf16_to_f32(B[j * N + n]), lora);
  Y[m * N + n] = (uint16_t)f32_to_bf16_bits(__fadd_rn(sum, lora));
}

}  // namespace

// Blocks of the reduction per split: whole 4-block steps, at most GMAX_KS columns
// (the LDS token tile), and enough splits for about 1024 workgroups.
GemvPlan gemv_plan(int64_t K, int64_t N) {
  const int64_t nkb = K / 64;
  GemvPlan pl;
  pl.groups = (N + GROWS - 1) / GROWS;
  int64_t s = (1024 + pl.groups - 1) / pl.groups;
  if (s > nkb) s = nkb;
  if (s < 1) s = 1;
  int64_t kbps = (nkb + s - 1) / s;
  kbps = (kbps + 3) / 4 * 4;
  if (kbps * 64 > GMAX_KS) kbps = GMAX_KS / 64;
  pl.kb_per_split = kbps;
  pl.splits = (int)((nkb + kbps - 1) / kbps);
  return pl;
}

size_t gemv_partial_floats(const GemvPlan& pl, int64_t M) { return (size_t)(pl.groups * pl.splits * M * GROWS); }

hipError_t launch_gemv(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w, const GemvPlan& pl,
                       float* partial, hipStream_t s) {
  GemvParams p{X, M, K, N, w, partial, pl.kb_per_split, pl.splits, nf4_table()};
  ProfScope ps("k_fwd_nf4_gemv", s);
  hipLaunchKernelGGL(k_fwd_nf4_gemv, dim3((unsigned)(pl.groups * pl.splits)), dim3(GT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemv_epilogue(const float* partial, const GemvPlan& pl, int64_t M, int64_t N, const uint16_t* Ts,
                                int64_t rp, const uint16_t* B, int64_t r, uint16_t* Y, hipStream_t s) {
  const int64_t n = pl.groups * M * GROWS;
  ProfScope ps("k_gemv_epilogue", s);
  hipLaunchKernelGGL(k_gemv_epilogue, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, partial, pl.splits, M, N,
                     Ts, rp, B, r, Y);
  return hipGetLastError();
}

}  // namespace qlora
