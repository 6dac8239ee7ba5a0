// Internal launch interface between the host layer (api.cpp) and the kernels.
// Every launcher validates nothing: the host layer has already checked shapes,
// pointers and workspace.  All return hipGetLastError() of their launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "qlora.h"

namespace qlora {

// Host-side NF4 table (computed once, see codebook.cpp).
const float* nf4_levels_host();
const float* nf4_thresholds_host();
constexpr int kNumCodebooks = 3;   // NF4, FP4, INT4
const float* codebook_levels_host(int which);
const float* codebook_thresholds_host(int which);
NF4Table nf4_table(int which);
// The encoder's bin table of a codebook (computed once per codebook, see codebook.cpp).
const ThrLut& thr_lut_host(int which);

// Argument checks of qlora_linear_fwd other than the workspace (api.cpp).
qlora_status linear_fwd_check(const uint16_t* X, int64_t M, const qlora_nf4* w, const uint16_t* A, const uint16_t* B,
                              int32_t r, const uint16_t* Y, const uint16_t* T_save);

// Optional per-launch timing (api.cpp).
struct ProfScope {
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  int slot_;
  hipStream_t s_;
};

// ---- quantize / dequantize (quant.hip) --------------------------------------------------
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
// workgroups of the quantize launch (<= kQuantSlots): the number of exact-sum slots it writes
int quantize_grid(int64_t numel, int block);
// sums: kSumLimbs x quantize_grid() 64-bit words (double quantization), or NULL
hipError_t launch_quantize(const uint16_t* W, int64_t numel, int codebook, int block, uint8_t* codes,
                           float* absmax_f32, unsigned long long* sums, hipStream_t s);
// mu from the quantize workgroups' exact sums (every workgroup forms it; the first stores it),
// then c1 and the E4M3 codes of every group of 256 block constants
hipError_t launch_dq_encode(const float* absmax_f32, int64_t nblk, const unsigned long long* sums, int nslots, float* mu,
                            uint8_t* c2, float* c1, hipStream_t s);
hipError_t launch_dequant(const NF4View& w, int64_t numel, uint16_t* out, hipStream_t s);

// ---- small rank-r products (lora.hip) ----------------------------------------------------
// C[I][J] = sum_k A(i,k) B(k,j); A(i,k) = A[i*a_si + k*a_sk] (one of the two strides is 1),
// B(k,j) = B[k*b_sk + j*b_sj] (one of the two strides is 1).
struct SmallGemm {
  const uint16_t* A;
  int64_t a_si, a_sk;
  const uint16_t* B;
  int64_t b_sk, b_sj;
  int64_t I, J, K;
};
// Outputs of a product (any may be NULL):
//   out_a[i*lda + j] = bf16(scale_a * C)                     (j < J)
//   out_b[i*ldb + j] = bf16(scale_b * C) for j < J, 0 for J <= j < ldb
//   out_f[i*J + j]   = scale_f * C
struct LoraEpi {
  uint16_t* out_a;
  int64_t lda;
  float scale_a;
  uint16_t* out_b;
  int64_t ldb;
  float scale_b;
  float* out_f;
  float scale_f;
};
struct LoraProblem {
  SmallGemm g;
  LoraEpi ep;
  int64_t tiles_i, tiles_j, k_per_split;
  int splits;
  float* partial;        // splits > 1: tiles * splits * 64*64 floats of workspace
};
constexpr int kMaxLoraSplits = 16;   // the reduce kernel sums at most this many partials
LoraProblem lora_problem(const SmallGemm& g, const LoraEpi& ep, int max_splits);
size_t lora_partial_floats(const LoraProblem& p);
// one launch for p0, or for p0 and p1 together (same operand layouts); with splits > 1
// the partials are summed and written out by launch_lora_reduce
hipError_t launch_lora(const LoraProblem& p0, const LoraProblem* p1, const char* name, hipStream_t s);
hipError_t launch_lora_reduce(const LoraProblem& p0, const LoraProblem* p1, const char* name, hipStream_t s);

// ---- fused forward, large M (fwd_gemm.hip) ------------------------------------------------
// Y[M][N] = bf16( X[M][K] deq(W)^T + Ts[M][rp] Bt ), Bt(j, n) = B[j][n] for j < r else 0.
hipError_t launch_fwd_gemm(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w,
                           const uint16_t* Ts, int64_t rp, const uint16_t* B, int64_t r, uint16_t* Y,
                           hipStream_t s);
// Few tokens (one 256-token panel), few feature tiles: the same GEMM cut into K-slices of
// `stages` 64-deep stages, fp32 partials partial[slice][m][n] (row length npad), no adapter
// term; ceil(K / 64 / stages) slices.  The epilogue of the weight-streaming path finishes Y.
hipError_t launch_fwd_gemm_split(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w, int stages,
                                 float* partial, int64_t npad, hipStream_t s);

// ---- fused forward, few tokens M <= 64 (gemv.hip) ---------------------------------------------
// k_fwd_nf4_gemv writes fp32 partials: partial[split][m][n] (X deq(W)^T over `splits` slices
// of the reduction) and, at float offset tpart, tpartial[aslice][m][j] (X A over `asplits`
// slices of ka rows); launch_gemv_epilogue forms T, Ts = bf16(s T), T_save = bf16(T) when
// T_save is not NULL, and Y = bf16( sum of weight partials + Ts B ).
struct GemvPlan {
  int splits;                 // weight slices of 32 blocks (2048 reduction indices)
  int64_t rgroups;            // 16-row groups of the weight
  int64_t rranges;            // weight workgroups per slice (contiguous ranges of row groups)
  int64_t npad;               // weight partial row length (rgroups * 16)
  int64_t agroups;            // 64-column adapter groups
  int asplits;                // adapter slices of ka rows of A
  int ka;
  int ngr;                    // 16-token groups of the batch (ceil(M / 16))
  int tg;                     // token groups each weight lane feeds (1, 2 or 4 >= ngr)
  size_t tpart;               // float offset of the adapter partials
};
GemvPlan gemv_plan(int64_t M, int64_t K, int64_t N, int64_t rp, bool adapters_only = false);
size_t gemv_partial_floats(const GemvPlan& pl, int64_t M);
// adapters_only: launch only the X A workgroups (their partials feed the epilogue after the
// split large-M forward)
hipError_t launch_gemv(const uint16_t* X, int64_t M, int64_t K, int64_t N, const NF4View& w, const uint16_t* A,
                       int64_t r, const GemvPlan& pl, float* partial, hipStream_t s, bool adapters_only = false);
hipError_t launch_gemv_epilogue(const float* partial, const GemvPlan& pl, int64_t M, int64_t N, const uint16_t* B,
                                int64_t r, float scale, uint16_t* Y, uint16_t* T_save, hipStream_t s);

// ---- backward dX (dx_gemm.hip) --------------------------------------------------------------
// dX[M][K] = bf16( dY[M][N] deq(W) + Gs[M][rp] A^T ), A [K][r].
hipError_t launch_dx_gemm(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const NF4View& w,
                          const uint16_t* Gs, int64_t rp, const uint16_t* A, int64_t r, uint16_t* dX,
                          hipStream_t s);
// few tokens: the reduction in slices of `stages` stages, fp32 partials [slice][M][K]
// (no adapter term), then the epilogue sums the slices in order, adds Gs A^T, rounds once
// g_partials (optional): a split-K product (both operands contiguous along the reduction, at
// least 2 splits, its partial buffer set) whose workgroups run first in the same launch: G's
// partials for the epilogue's fold, without a launch of their own.
hipError_t launch_dx_gemm_split(const uint16_t* dY, int64_t M, int64_t K, int64_t N, const NF4View& w, int stages,
                                float* partial, hipStream_t s, const LoraProblem* g_partials = nullptr);
// G still in split-K partials of the rank-r kernel (partial == NULL: Gs is in memory already):
// the epilogue forms Gs = bf16(scale G) itself and stores it to Gs_out [M][rp] for dA.
struct GFold {
  const float* partial;   // [tile][split][64][64], tile = (m / 64) tiles_j + j / 64
  int splits;
  int64_t tiles_j;
  float scale;
  uint16_t* Gs_out;
};
// With at most 16 tokens (one token group) the same launch can also finish the adapter
// gradients (dA == NULL: it does not): each dX workgroup forms dA = X^T Gs for its 64 rows of
// dA, and ceil(N / 64) more workgroups form dB = s T^T dY for 64 columns of dB each.
struct GradFold {
  const uint16_t* X;    // [M][K]
  const uint16_t* T;    // [M][r], bf16(X A)
  const uint16_t* dY;   // [M][N]
  float* dA;            // [K][r]
  float* dB;            // [r][N]
  int64_t N;
  float scale;
};
hipError_t launch_dx_split_epilogue(const float* partial, int splits, int64_t M, int64_t K, const uint16_t* Gs,
                                    int64_t rp, const uint16_t* A, int64_t r, uint16_t* dX, const GFold& gf,
                                    hipStream_t s, const GradFold* grads = nullptr);

// ---- adapter merge (merge.hip): out [N][K] = bf16(deq(W) + scale (A B)^T), K % 64 == 0 -------
hipError_t launch_merge_adapter(const NF4View& w, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int64_t r,
                                float scale, uint16_t* out, hipStream_t s);

// ---- AdamW step on adapter parameters (adamw.hip) ------------------------------------------
hipError_t launch_adamw(float* param, uint16_t* param_bf16, const float* grad, float* m, float* v, int64_t n,
                        int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                        hipStream_t s);

}  // namespace qlora
