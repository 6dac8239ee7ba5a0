// AdamW step on the adapter parameters ("QLoRA: Efficient Finetuning of Quantized
// LLMs", section "Paged optimizers": the optimizer state exists only for the
// adapters, kept in fp32; the 4-bit base gets no gradient and no state).
//
// Decoupled weight decay, with the bias corrections folded into two host constants
// (the usual formulation of AdamW):
//   p <- p * (1 - lr * wd)
//   m <- b1 m + (1 - b1) g
//   v <- b2 v + (1 - b2) g^2
//   p <- p - (lr / (1 - b1^t)) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// in fp32, each product and sum rounded separately; the bf16 working copy the layer
// reads is bf16_RNE(p).  One pass over memory: 16 bytes read and 12 (+2) written per
// parameter, four parameters per thread and iteration.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

struct AdamConsts {
  float decay, b1, omb1, b2, omb2, step_size, bc2_sqrt, eps;
};

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, const AdamConsts& c) {
  p = __fmul_rn(p, c.decay);
  m = __fadd_rn(__fmul_rn(c.b1, m), __fmul_rn(c.omb1, g));
  v = __fadd_rn(__fmul_rn(c.b2, v), __fmul_rn(c.omb2, __fmul_rn(g, g)));
  const float denom = __fadd_rn(__fdiv_rn(__fsqrt_rn(v), c.bc2_sqrt), c.eps);
  p = __fsub_rn(p, __fmul_rn(c.step_size, __fdiv_rn(m, denom)));
}

__global__ __launch_bounds__(256) void k_adamw(float* __restrict__ param, uint16_t* __restrict__ pbf16,
                                               const float* __restrict__ grad, float* __restrict__ m,
                                               float* __restrict__ v, int64_t n, AdamConsts c) {
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 p = reinterpret_cast<float4*>(param)[i];
    const float4 g = reinterpret_cast<const float4*>(grad)[i];
    float4 mm = reinterpret_cast<float4*>(m)[i];
    float4 vv = reinterpret_cast<float4*>(v)[i];
    adam_one(p.x, g.x, mm.x, vv.x, c);
    adam_one(p.y, g.y, mm.y, vv.y, c);
    adam_one(p.z, g.z, mm.z, vv.z, c);
    adam_one(p.w, g.w, mm.w, vv.w, c);
    reinterpret_cast<float4*>(param)[i] = p;
    reinterpret_cast<float4*>(m)[i] = mm;
    reinterpret_cast<float4*>(v)[i] = vv;
    if (pbf16) {
      uint2 b;
      b.x = f32_to_bf16_bits(p.x) | (f32_to_bf16_bits(p.y) << 16);
      b.y = f32_to_bf16_bits(p.z) | (f32_to_bf16_bits(p.w) << 16);
      reinterpret_cast<uint2*>(pbf16)[i] = b;
    }
  }
  // the last n % 4 parameters
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t j = n4 * 4 + t;
  if (t < (n & 3)) {
    float p = param[j], mm = m[j], vv = v[j];
    adam_one(p, grad[j], mm, vv, c);
    param[j] = p;
    m[j] = mm;
    v[j] = vv;
    if (pbf16) pbf16[j] = (uint16_t)f32_to_bf16_bits(p);
  }
}

}  // namespace

hipError_t launch_adamw(float* param, uint16_t* param_bf16, const float* grad, float* m, float* v, int64_t n,
                        int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  AdamConsts c;
  c.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  c.b1 = beta1;
  c.omb1 = (float)(1.0 - (double)beta1);
  c.b2 = beta2;
  c.omb2 = (float)(1.0 - (double)beta2);
  c.step_size = (float)((double)lr / (1.0 - std::pow((double)beta1, (double)step)));
  c.bc2_sqrt = (float)std::sqrt(1.0 - std::pow((double)beta2, (double)step));
  c.eps = eps;
  const int64_t n4 = (n + 3) / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  ProfScope ps("k_adamw", s);
  hipLaunchKernelGGL(k_adamw, dim3((unsigned)blocks), dim3(256), 0, s, param, param_bf16, grad, m, v, n, c);
  return hipGetLastError();
}

}  // namespace qlora
