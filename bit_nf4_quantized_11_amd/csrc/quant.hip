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

// Code of a normalized weight: the number of thresholds below x, read off the encoder's bin
// table (see ThrLut in common.h) held in LDS as {threshold, base} pairs.
__device__ __forceinline__ uint32_t lut_encode(float x, const float2* __restrict__ lut) {
  const float2 e = lut[lut_bin(x)];
  return __float_as_uint(e.y) + (x > e.x ? 1u : 0u);
}

// L = block / 8 lanes per block, eight consecutive weights per lane (one 16-byte load, one
// code dword).  Lane 0 of each group writes the fp32 block constant and, for double
// quantization, adds it to a per-exponent histogram from which the exact sum of all
// constants is rebuilt (integer adds: order-independent, hence deterministic).  Blocks
// from nblk up to ncode_blk (the code buffer's padding to whole 64-element chunks) get
// zero codes and no constant.
template <int L>
__global__ __launch_bounds__(kThreads) void k_nf4_quantize(const uint16_t* __restrict__ W, int64_t numel,
                                                           int64_t ncode_blk, uint8_t* __restrict__ codes,
                                                           float* __restrict__ absmax,
                                                           unsigned long long* __restrict__ hist, ThrLut lut) {
  __shared__ unsigned long long lhist[256];
  __shared__ float2 slut[kLutBins];
  const bool dq = hist != nullptr;
  if (dq) lhist[threadIdx.x] = 0ull;
  if (threadIdx.x < kLutBins) slut[threadIdx.x] = make_float2(lut.t[threadIdx.x], __uint_as_float(lut.base[threadIdx.x]));
  __syncthreads();
  const int sub = threadIdx.x & (L - 1);
  const int64_t nblk = (numel + 8 * L - 1) / (8 * L);
  const int64_t stride = (int64_t)gridDim.x * (kThreads / L);
  for (int64_t blk = (int64_t)blockIdx.x * (kThreads / L) + (threadIdx.x / L); blk < ncode_blk; blk += stride) {
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
    // one of kHistCopies global copies per workgroup, so the few busy bins do not
    // serialize every workgroup's atomics on one address
    __syncthreads();
    const unsigned long long v = lhist[threadIdx.x];
    if (v) atomicAdd(&hist[(blockIdx.x % kHistCopies) * 256 + threadIdx.x], v);
  }
}

// mu = fl32(S / nblk), S = the exact sum of all block constants rounded once to float64.
// hist[E] = sum of the 8-bit significands (implicit bit included) of the constants whose
// bf16 exponent field is E, so S = sum_E hist[E] * 2^(E - 134).  The exact integer
// sum_E hist[E] << E is built in 64-bit words, then rounded to nearest even.  Called by all
// kThreads threads of a workgroup; every thread gets mu.
__device__ float exact_mean(const unsigned long long* __restrict__ hist, int64_t nblk) {
  __shared__ unsigned long long tot[256];
  __shared__ unsigned long long nonzero[4];
  __shared__ float mu_s;
  {
    unsigned long long v = 0;
#pragma unroll 16
    for (int c = 0; c < kHistCopies; ++c) v += hist[c * 256 + threadIdx.x];
    tot[threadIdx.x] = v;
    const unsigned long long b = __ballot(v != 0ull);
    if ((threadIdx.x & 63) == 0) nonzero[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    constexpr int NW = 7;   // 448 bits: 2^254 * 2^64 fits
    unsigned long long acc[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) acc[k] = 0ull;
    // only the occupied exponent bins, in increasing order (bin 0 only ever holds zeros)
    for (int wv = 0; wv < 4; ++wv)
    for (unsigned long long bits = nonzero[wv]; bits; bits &= bits - 1ull) {
      const int E = wv * 64 + __builtin_ctzll(bits);
      if (E == 0 || E == 255) continue;
      const unsigned long long v = tot[E];
      const int w = E >> 6, sh = E & 63;
      const unsigned long long lo = v << sh;
      const unsigned long long hi = sh ? (v >> (64 - sh)) : 0ull;
      unsigned long long s = acc[w] + lo;
      unsigned long long carry = s < lo;
      acc[w] = s;
      s = acc[w + 1] + hi;
      unsigned long long c2 = s < hi;
      s += carry;
      c2 += (s < carry);
      acc[w + 1] = s;
      for (int k = w + 2; c2 && k < NW; ++k) {
        acc[k] += 1ull;
        c2 = (acc[k] == 0ull);
      }
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
// max), grid-stride over the groups.  Each workgroup first forms mu from the histogram itself
// (the same exact sum in every workgroup, so no launch of its own); the first one stores it.
// Then c1 = max |absmax - mu| / 448 and the E4M3 codes of the group.
__global__ __launch_bounds__(kThreads) void k_dq_encode(const float* __restrict__ absmax, int64_t nblk,
                                                        const unsigned long long* __restrict__ hist,
                                                        float* __restrict__ mu_out, uint8_t* __restrict__ c2,
                                                        float* __restrict__ c1_out) {
  static_assert(kSuper == 4 * 64, "a group is one wave of 4 constants per lane");
  const float mu = exact_mean(hist, nblk);
  if (blockIdx.x == 0 && threadIdx.x == 0) *mu_out = mu;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nsup = (nblk + kSuper - 1) / kSuper;
  for (int64_t j = (int64_t)blockIdx.x * (kThreads / 64) + wave; j < nsup; j += (int64_t)gridDim.x * (kThreads / 64)) {
    const int64_t b0 = j * kSuper + lane * 4;
    float x[4];
    if (b0 + 4 <= nblk) {
      const float4 a = *reinterpret_cast<const float4*>(absmax + b0);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = b0 + i < nblk ? absmax[b0 + i] : mu;   // past the end: x = 0
    }
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

hipError_t launch_quantize(const uint16_t* W, int64_t numel, int codebook, int block, uint8_t* codes,
                           float* absmax_f32, unsigned long long* hist, hipStream_t s) {
  const int64_t unit = block > 64 ? block : 64;   // the code buffer holds whole blocks and 64-chunks
  const int64_t ncode_blk = (numel + unit - 1) / unit * (unit / block);
  const unsigned grid = grid_for(ncode_blk, kThreads / (block / 8), 2048);
  const ThrLut& tab = thr_lut_host(codebook);
  ProfScope ps("k_nf4_quantize", s);
  if (block == 32)
    hipLaunchKernelGGL(k_nf4_quantize<4>, dim3(grid), dim3(kThreads), 0, s, W, numel, ncode_blk, codes, absmax_f32,
                       hist, tab);
  else if (block == 64)
    hipLaunchKernelGGL(k_nf4_quantize<8>, dim3(grid), dim3(kThreads), 0, s, W, numel, ncode_blk, codes, absmax_f32,
                       hist, tab);
  else if (block == 128)
    hipLaunchKernelGGL(k_nf4_quantize<16>, dim3(grid), dim3(kThreads), 0, s, W, numel, ncode_blk, codes, absmax_f32,
                       hist, tab);
  else
    hipLaunchKernelGGL(k_nf4_quantize<32>, dim3(grid), dim3(kThreads), 0, s, W, numel, ncode_blk, codes, absmax_f32,
                       hist, tab);
  return hipGetLastError();
}

hipError_t launch_dq_encode(const float* absmax_f32, int64_t nblk, const unsigned long long* hist, float* mu,
                            uint8_t* c2, float* c1, hipStream_t s) {
  const int64_t nsup = (nblk + kSuper - 1) / kSuper;
  ProfScope ps("k_dq_encode", s);
  hipLaunchKernelGGL(k_dq_encode, dim3(grid_for(nsup, kThreads / 64, 1024)), dim3(kThreads), 0, s, absmax_f32, nblk, hist, mu, c2,
                     c1);
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
