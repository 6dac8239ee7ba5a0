// NF4 blockwise quantization, double quantization of the block constants, and
// the standalone doubleDequant.
//
// Sources ("QLoRA: Efficient Finetuning of Quantized LLMs"):
//   "Quantize in blocks, not all at once" -- absmax scale per 64 contiguous weights,
//       a value is normalized by multiplying it with c = 1/absmax ("Double quantization"
//       weighs other block sizes: 32, 128 and 256 are supported as format variants);
//   "NormalFloat: 4 bits for a bell curve" -- 16 levels, nearest level;
//   "Double quantization" -- block constants, mean subtracted, as 8-bit floats in
//       groups of 256 with one fp32 scale per group;
//   "The QLoRA layer, end to end" -- doubleDequant, inner step (scales) first.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

constexpr int kThreads = 256;
constexpr int kQuantThreads = 1024;   // quantize workgroups: at most kQuantSlots of them

// Code of a normalized weight: the number of thresholds below x, read off the encoder's bin
// table (see ThrLut in common.h) held in LDS as {threshold, base} pairs.
__device__ __forceinline__ uint32_t lut_encode(float x, const float2* __restrict__ lut) {
  const float2 e = lut[lut_bin(x)];
  return __float_as_uint(e.y) + (x > e.x ? 1u : 0u);
}

// L = block / 8 lanes per block, eight consecutive weights per lane (one 16-byte load, one
// code dword).  Lane 0 of each group writes the fp32 block constant and, for double
// quantization, adds its significand to a per-exponent histogram in LDS.  At the end the
// workgroup turns that histogram into the exact integer sum_E hist[E] << E (the sum of its
// constants times 2^134, see exact_mean) and writes it to its own slot of `sums` as kSumLimbs
// 64-bit words, word k holding the part of weight 2^(32 k) (each below 2^39, not carried):
// integer adds only, so the result does not depend on the order, and no slot needs clearing
// beforehand.  Blocks from nblk up to ncode_blk (the code buffer's padding to
// whole 64-element chunks) get zero codes and no constant.
template <int L>
__global__ __launch_bounds__(kQuantThreads) void k_nf4_quantize(const uint16_t* __restrict__ W, int64_t numel,
                                                                int64_t ncode_blk, uint8_t* __restrict__ codes,
                                                                float* __restrict__ absmax,
                                                                unsigned long long* __restrict__ sums, ThrLut lut) {
  __shared__ unsigned long long lhist[256];
  __shared__ unsigned long long limb[kSumLimbs];
  __shared__ float2 slut[kLutBins];
  const bool dq = sums != nullptr;
  if (dq && threadIdx.x < 256) lhist[threadIdx.x] = 0ull;
  if (dq && threadIdx.x < kSumLimbs) limb[threadIdx.x] = 0ull;
  if (threadIdx.x < kLutBins) slut[threadIdx.x] = make_float2(lut.t[threadIdx.x], __uint_as_float(lut.base[threadIdx.x]));
  __syncthreads();
  const int sub = threadIdx.x & (L - 1);
  const int64_t nblk = (numel + 8 * L - 1) / (8 * L);
  const int64_t stride = (int64_t)gridDim.x * (kQuantThreads / L);
  for (int64_t blk = (int64_t)blockIdx.x * (kQuantThreads / L) + (threadIdx.x / L); blk < ncode_blk; blk += stride) {
    const int64_t e0 = blk * (8 * L) + sub * 8;
    uint32_t h[8];
    if (e0 + 8 <= numel) {
      const uint4 v = *reinterpret_cast<const uint4*>(W + e0);
      h[0] = v.x & 0xFFFFu; h[1] = v.x >> 16; h[2] = v.y & 0xFFFFu; h[3] = v.y >> 16;
      h[4] = v.z & 0xFFFFu; h[5] = v.z >> 16; h[6] = v.w & 0xFFFFu; h[7] = v.w >> 16;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (e0 + i < numel) ? (uint32_t)W[e0 + i] : 0u;
    }
    // largest magnitude: on bf16 bit patterns the magnitude order is the integer order
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, h[i] & 0x7FFFu);
#pragma unroll
    for (int off = 1; off < L; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, L));
    if (m < 0x0080u) m = 0;   // below the smallest normal: a zero block
    const float a = bf16_to_f32(m);
    // correctly rounded fp32 reciprocal (a float64 quotient rounded to fp32 is exact-rounded)
    const float inv = m ? (float)(1.0 / (double)a) : 0.0f;
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = lut_encode(__fmul_rn(bf16_to_f32(h[i]), inv), slut);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= (c[i] | (c[i + 4] << 4)) << (8 * i);
    *reinterpret_cast<uint32_t*>(codes + (e0 >> 1)) = packed;
    if (sub == 0 && blk < nblk) {
      absmax[blk] = a;
      if (dq && m) atomicAdd(&lhist[m >> 7], (unsigned long long)((m & 0x7Fu) | 0x80u));
    }
  }
  if (dq) {
    __syncthreads();
    // bin E adds hist[E] << E: its low 64 bits over limbs E / 32 and E / 32 + 1, the bits shifted
    // out into limb E / 32 + 2 (E <= 254 keeps that below kSumLimbs); each limb collects at most
    // 96 terms below 2^32.  Exponent 255 (infinite or NaN weights) is left out.
    if (threadIdx.x < 255) {
      const unsigned long long v = lhist[threadIdx.x];
      if (v) {
        const int l0 = threadIdx.x >> 5, sh = threadIdx.x & 31;
        const unsigned long long lo = v << sh, hi = sh ? v >> (64 - sh) : 0ull;
        atomicAdd(&limb[l0], lo & 0xFFFFFFFFull);
        atomicAdd(&limb[l0 + 1], lo >> 32);
        if (hi) atomicAdd(&limb[l0 + 2], hi);
      }
    }
    __syncthreads();
    if (threadIdx.x < kSumLimbs) sums[(int64_t)blockIdx.x * kSumLimbs + threadIdx.x] = limb[threadIdx.x];
  }
}

// mu = fl32(S / nblk), S = the exact sum of all block constants rounded once to float64.  A
// constant with bf16 exponent field E and significand m (implicit bit included) is
// m * 2^(E - 134), so S * 2^134 is an integer: the sum of the quantize workgroups' slots, added
// word by word (word k weighs 2^(32 k)) and carried once, then rounded to nearest even.  Called by all kThreads threads of a workgroup; every thread gets mu.
__device__ float exact_mean(const unsigned long long* __restrict__ sums, int nslots, int64_t nblk) {
  constexpr int G = kThreads / kSumLimbs;   // 25 threads per limb
  __shared__ unsigned long long tot[kSumLimbs];
  __shared__ float mu_s;
  if (threadIdx.x < kSumLimbs) tot[threadIdx.x] = 0ull;
  __syncthreads();
  if (threadIdx.x < G * kSumLimbs) {
    // thread t adds limb t % kSumLimbs of slots t / kSumLimbs, + G, + 2 G, ... (at most
    // kQuantSlots slots);
    // threads read consecutive words; every load is issued before the first add
    constexpr int PER = (kQuantSlots + G - 1) / G;
    const int k = threadIdx.x % kSumLimbs, g = threadIdx.x / kSumLimbs;
    unsigned long long v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int sl = g + u * G;
      v[u] = sl < nslots ? sums[sl * kSumLimbs + k] : 0ull;
    }
    unsigned long long a = 0ull;
#pragma unroll
    for (int u = 0; u < PER; ++u) a += v[u];
    atomicAdd(&tot[k], a);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // limb sums are below 2^49 (at most kQuantSlots slots of words below 2^39): one carry pass
    // gives 32-bit limbs
    constexpr int NW = kSumLimbs / 2;   // 64-bit words
    unsigned long long acc[NW];
    unsigned long long carry = 0;
    for (int k = 0; k < kSumLimbs; ++k) {
      const unsigned long long t = tot[k] + carry;
      const unsigned long long l = t & 0xFFFFFFFFull;
      if (k & 1) acc[k >> 1] |= l << 32; else acc[k >> 1] = l;
      carry = t >> 32;
    }
    int top = -1;
    for (int k = NW - 1; k >= 0; --k)
      if (acc[k]) { top = k * 64 + 63 - __builtin_clzll(acc[k]); break; }
    double S = 0.0;
    if (top >= 0 && top <= 52) {
      S = __builtin_ldexp((double)acc[0], -134);
    } else if (top > 52) {
      const int low = top - 52;                      // lowest kept bit
      auto word_at = [&](int pos) -> unsigned long long {   // 64 bits starting at bit pos
        const int w = pos >> 6, off = pos & 63;
        unsigned long long v = acc[w] >> off;
        if (off && w + 1 < NW) v |= acc[w + 1] << (64 - off);
        return v;
      };
      unsigned long long mant = word_at(low) & ((1ull << 53) - 1ull);
      const int rpos = low - 1;
      const unsigned long long round = (acc[rpos >> 6] >> (rpos & 63)) & 1ull;
      unsigned long long sticky = 0;
      for (int k = 0; k < (rpos >> 6); ++k) sticky |= acc[k];
      if (rpos & 63) sticky |= acc[rpos >> 6] & ((1ull << (rpos & 63)) - 1ull);
      if (round && (sticky || (mant & 1ull))) mant += 1ull;
      S = __builtin_ldexp((double)mant, low - 134);
    }
    mu_s = (float)(S / (double)nblk);
  }
  __syncthreads();
  return mu_s;
}

// Groups of 256 block constants, one wave per group (4 constants per lane, a wave-wide
// max), grid-stride over the groups.  Each workgroup first forms mu from the slots itself
// (the same exact sum in every workgroup, so no launch of its own); the first one stores it.
// Then c1 = max |absmax - mu| / 448 and the E4M3 codes of the group.
__global__ __launch_bounds__(kThreads) void k_dq_encode(const float* __restrict__ absmax, int64_t nblk,
                                                        const unsigned long long* __restrict__ sums, int nslots,
                                                        float* __restrict__ mu_out, uint8_t* __restrict__ c2,
                                                        float* __restrict__ c1_out) {
  static_assert(kSuper == 4 * 64, "a group is one wave of 4 constants per lane");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nsup = (nblk + kSuper - 1) / kSuper;
  const int64_t j0 = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  // the constants of a group; entries past the end are marked and become mu (so x - mu = 0)
  auto load = [&](int64_t j, float (&x)[4], bool (&in)[4]) {
    const int64_t b0 = j * kSuper + lane * 4;
    if (b0 + 4 <= nblk) {
      const float4 a = *reinterpret_cast<const float4*>(absmax + b0);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
#pragma unroll
      for (int i = 0; i < 4; ++i) in[i] = true;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        in[i] = b0 + i < nblk;
        x[i] = in[i] ? absmax[b0 + i] : 0.0f;
      }
    }
  };
  // the first group's loads are in flight while mu is formed
  float x0[4] = {0.f, 0.f, 0.f, 0.f};
  bool in0[4] = {false, false, false, false};
  if (j0 < nsup) load(j0, x0, in0);
  const float mu = exact_mean(sums, nslots, nblk);
  if (blockIdx.x == 0 && threadIdx.x == 0) *mu_out = mu;
  for (int64_t j = j0; j < nsup; j += (int64_t)gridDim.x * (kThreads / 64)) {
    const int64_t b0 = j * kSuper + lane * 4;
    float x[4];
    bool in[4];
    if (j == j0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[i] = x0[i]; in[i] = in0[i]; }
    } else {
      load(j, x, in);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) if (!in[i]) x[i] = mu;   // past the end: x - mu = 0
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __fsub_rn(x[i], mu);
      m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    float c1 = (float)((double)__uint_as_float(m) / 448.0);
    if (c1 < 0x1p-126f) c1 = 0.0f;
    if (lane == 0) c1_out[j] = c1;
    const float inv = c1 != 0.0f ? (float)(1.0 / (double)c1) : 0.0f;
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= (c1 != 0.0f ? e4m3_encode(__fmul_rn(x[i], inv)) : 0u) << (8 * i);
    if (b0 + 4 <= nblk) {
      *reinterpret_cast<uint32_t*>(c2 + b0) = packed;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (b0 + i < nblk) c2[b0 + i] = (uint8_t)(packed >> (8 * i));
    }
  }
}

// doubleDequant of a whole tensor: one thread per group of 8 weights (4 code bytes).
__global__ __launch_bounds__(kThreads) void k_nf4_dequant(NF4View w, int64_t numel, uint16_t* __restrict__ out,
                                                          NF4Table tab) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = tab.level[threadIdx.x];
  __syncthreads();
  const int64_t ngroups = (numel + 7) >> 3;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < ngroups; g += (int64_t)gridDim.x * kThreads) {
    const int64_t blk = (g * 8) >> w.bshift;
    const float s = block_scale(w, blk);
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(w.codes + g * 4);
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = f32_to_bf16_bits(__fmul_rn(lv[(cw >> (8 * i)) & 15u], s));
      v[i + 4] = f32_to_bf16_bits(__fmul_rn(lv[(cw >> (8 * i + 4)) & 15u], s));
    }
    const int64_t e0 = g * 8;
    if (e0 + 8 <= numel) {
      uint4 o;
      o.x = v[0] | (v[1] << 16); o.y = v[2] | (v[3] << 16);
      o.z = v[4] | (v[5] << 16); o.w = v[6] | (v[7] << 16);
      *reinterpret_cast<uint4*>(out + e0) = o;
    } else {
      for (int i = 0; i < 8 && e0 + i < numel; ++i) out[e0 + i] = (uint16_t)v[i];
    }
  }
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

inline unsigned grid_for(int64_t work, int64_t per_block, unsigned cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

NF4Table nf4_table(int which) {
  NF4Table t;
  const float* l = codebook_levels_host(which);
  const float* th = codebook_thresholds_host(which);
  for (int i = 0; i < 16; ++i) t.level[i] = l[i];
  for (int i = 0; i < 15; ++i) t.thr[i] = th[i];
  t.pad_ = 0.0f;
  return t;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  ProfScope ps("k_fill_u32", s);
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n, 256, 4096)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

int quantize_grid(int64_t numel, int block) {
  const int64_t unit = block > 64 ? block : 64;   // the code buffer holds whole blocks and 64-chunks
  const int64_t ncode_blk = (numel + unit - 1) / unit * (unit / block);
  return (int)grid_for(ncode_blk, kQuantThreads / (block / 8), kQuantSlots);
}

hipError_t launch_quantize(const uint16_t* W, int64_t numel, int codebook, int block, uint8_t* codes,
                           float* absmax_f32, unsigned long long* sums, hipStream_t s) {
  const int64_t unit = block > 64 ? block : 64;
  const int64_t ncode_blk = (numel + unit - 1) / unit * (unit / block);
  const unsigned grid = (unsigned)quantize_grid(numel, block);
  const ThrLut& tab = thr_lut_host(codebook);
  ProfScope ps("k_nf4_quantize", s);
  if (block == 32)
    hipLaunchKernelGGL(k_nf4_quantize<4>, dim3(grid), dim3(kQuantThreads), 0, s, W, numel, ncode_blk, codes,
                       absmax_f32, sums, tab);
  else if (block == 64)
    hipLaunchKernelGGL(k_nf4_quantize<8>, dim3(grid), dim3(kQuantThreads), 0, s, W, numel, ncode_blk, codes,
                       absmax_f32, sums, tab);
  else if (block == 128)
    hipLaunchKernelGGL(k_nf4_quantize<16>, dim3(grid), dim3(kQuantThreads), 0, s, W, numel, ncode_blk, codes,
                       absmax_f32, sums, tab);
  else
    hipLaunchKernelGGL(k_nf4_quantize<32>, dim3(grid), dim3(kQuantThreads), 0, s, W, numel, ncode_blk, codes,
                       absmax_f32, sums, tab);
  return hipGetLastError();
}

hipError_t launch_dq_encode(const float* absmax_f32, int64_t nblk, const unsigned long long* sums, int nslots, float* mu,
                            uint8_t* c2, float* c1, hipStream_t s) {
  const int64_t nsup = (nblk + kSuper - 1) / kSuper;
  ProfScope ps("k_dq_encode", s);
  hipLaunchKernelGGL(k_dq_encode, dim3(grid_for(nsup, kThreads / 64, 1024)), dim3(kThreads), 0, s, absmax_f32, nblk,
                     sums, nslots, mu, c2, c1);
  return hipGetLastError();
}

hipError_t launch_dequant(const NF4View& w, int64_t numel, uint16_t* out, hipStream_t s) {
  const int64_t ngroups = (numel + 7) / 8;
  ProfScope ps("k_nf4_dequant", s);
  hipLaunchKernelGGL(k_nf4_dequant, dim3(grid_for(ngroups, kThreads, 16384)), dim3(kThreads), 0, s, w, numel, out,
                     nf4_table(w.cb));
  return hipGetLastError();
}

}  // namespace qlora
