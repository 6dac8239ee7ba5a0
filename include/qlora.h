/*
 * libqlora -- QLoRA linear layer for AMD Instinct MI355X (gfx950).
 *
 * A frozen bf16 weight is stored as 4-bit NormalFloat (NF4) codes with one
 * absmax constant per 64-weight block; the constants are themselves quantized
 * to 8-bit floats in groups of 256 with one fp32 scale per group ("double
 * quantization").  The layer computes, in bf16 with fp32 accumulation,
 *
 *     Y  = X deq(W)^T + s (X A) B
 *     dX = dY deq(W) + s (dY B^T) A^T,   dA = s X^T (dY B^T),   dB = s (X A)^T dY
 *
 * with no gradient for the frozen W.  Sources ("QLoRA: Efficient Finetuning of
 * Quantized LLMs", intuitivepapers.ai): sections "Quantize in blocks, not all
 * at once", "NormalFloat: 4 bits for a bell curve", "Double quantization" and
 * "The QLoRA layer, end to end" (the one-layer code listing).  The review page
 * "QLoRA Review: 4-Bit Finetuning for 65B Models on One GPU", section "The
 * Gradient Flow Trick", states the same layer with s = 1.
 *
 * Conventions for every call
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are dense
 *     row-major.  W is [rows = out][cols = in] (the layout of a torch Linear
 *     weight); A is [in][r]; B is [r][out]; X is [M][in]; Y, dY are [M][out].
 *   - Device pointers unless stated otherwise.  The caller owns every buffer;
 *     the library never allocates or frees device memory and keeps no state
 *     other than read-only constants, so concurrent calls on different streams
 *     are safe when they write disjoint buffers.
 *   - Calls are asynchronous on `stream`.  QLORA_OK means the arguments were
 *     valid and every launch was accepted, not that the kernels finished.
 *   - Arguments are validated on the host before any launch; on error nothing
 *     is launched and the status says why.  The library never prints or aborts.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,        /* a required pointer is NULL                                   */
  QLORA_ERR_SHAPE = 2,       /* a size is out of range or violates a divisibility rule        */
  QLORA_ERR_ALIGN = 3,       /* a pointer is not aligned as required (16 bytes)               */
  QLORA_ERR_UNSUPPORTED = 4, /* a valid but unsupported option (rank, format flag)            */
  QLORA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the matching *_workspace query */
  QLORA_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed                    */
} qlora_status;

/* Quantized weight: caller-owned views of device buffers.  block_size B is the number
 * of contiguous weights (of the flattened row-major tensor) that share one constant:
 * 64 ("Quantize in blocks, not all at once"), or 32, 128 or 256 as format variants
 * ("Double quantization" weighs precision against constant overhead); 0 means 64.
 *   codes  : ncode / 2 bytes, ncode = rows*cols rounded up to a multiple of max(B, 64).
 *            The group of 8 elements 8g..8g+7 sits in bytes 4g..4g+3, and byte i of a
 *            group holds element i in bits 3..0 and element i+4 in bits 7..4 (so every
 *            64 elements take 32 bytes whatever B).  Positions past the end of the
 *            tensor hold the code of the table's exact zero (7 for NF4, 8 for FP4 and
 *            INT4).  (Not "two adjacent elements per byte": with this order one mask
 *            gives four codes in element order and a shift plus mask the other four,
 *            each ready for the byte-permute table lookup of the kernels.)
 *   absmax : double_quant = 1 -> nblk bytes, FP8 E4M3 code of (absmax_b - mu) / c1
 *            (OCP e4m3fn: the quantizer writes magnitudes up to 448; the codes 0x7F
 *            and 0xFF are NaN and give NaN weights if a caller stores them)
 *            double_quant = 0 -> nblk floats, the block absmax itself
 *            (nblk = ceil(rows*cols / B))
 *   c1     : double_quant = 1 -> nsup floats, one scale per 256 blocks
 *            (nsup = ceil(nblk / 256)); unused (may be NULL) otherwise
 *   mu     : double_quant = 1 -> 1 float, the mean of all block absmax values;
 *            unused (may be NULL) otherwise
 * Block scale used by dequant ("doubleDequant", inner step first):
 *   s'_b = fl32(fl32(e4m3(absmax_b) * c1_{b/256}) + mu)   (double_quant = 1)
 *   s'_b = absmax_b                                       (double_quant = 0)
 * Dequantized weight: bf16_RNE(fl32(level[code] * s'_b)).                        */
typedef struct {
  int64_t rows;
  int64_t cols;
  int32_t double_quant;
  int32_t codebook;      /* qlora_codebook: the 16-entry table the codes index (0 = NF4) */
  int32_t block_size;    /* weights per constant: 32, 64, 128 or 256 (0 = 64)          */
  int32_t reserved;      /* 0                                                            */
  uint8_t* codes;
  void* absmax;
  float* c1;
  float* mu;
} qlora_nf4;

/* Human-readable name of a status code (static string). */
const char* qlora_status_str(qlora_status s);

/* Library version string (static): "libqlora <version> (gfx950, src <hash>)", where
 * <hash> identifies the sources the library was built from (16 hex digits of a sha256
 * over the sources, this header and the compile flags).                            */
const char* qlora_version(void);

/* Host only.  The 16 NF4 levels (fp32, ascending; index 7 is the exact zero)
 * and the 15 decision thresholds the encoder uses: code = #{k : x > t_k}, with
 * t_k the largest fp32 not above the midpoint of levels k and k+1, which gives
 * the nearest level with ties to the lower index.  The levels follow the
 * procedure in "NormalFloat: 4 bits for a bell curve": standard-normal
 * quantiles with the tails pulled in by the offset 0.9677083, 8 positive, 7
 * negative and an exact zero, divided by the largest magnitude.  Computed once
 * in float64 by the library's own inverse normal CDF, then rounded to fp32.
 * Either pointer may be NULL.                                                   */
qlora_status qlora_nf4_codebook(float levels[16], float thresholds[15]);

/* The 16-entry tables a quantized weight can use (qlora_nf4.codebook).  Every table
 * is strictly ascending, spans [-1, 1] with an exact zero, and is used the same way
 * (encoder thresholds at the rounded-down midpoints, dequant level[code] * s').
 *   QLORA_CODEBOOK_NF4  -- the NormalFloat levels above (zero at index 7).
 *   QLORA_CODEBOOK_FP4  -- the 15 values of a 4-bit float with 2 exponent and 1
 *                          mantissa bits (OCP E2M1: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 *                          negatives) divided by 6, so the block maximum maps to 1;
 *                          index 0 holds -4/3, outside [-1, 1], never chosen (E2M1's two
 *                          zeros leave one of its 16 codes without a value of its own).
 *   QLORA_CODEBOOK_INT4 -- k / 7 for k = -8..7 (symmetric absmax int4, round(7 x));
 *                          index 0 (-8/7) is never chosen.
 * The pages compare NF4 with FP4 and Int4 data types ("NormalFloat: 4 bits for a
 * bell curve"); they print no FP4 table, so this one is E2M1, stated here.       */
typedef enum { QLORA_CODEBOOK_NF4 = 0, QLORA_CODEBOOK_FP4 = 1, QLORA_CODEBOOK_INT4 = 2 } qlora_codebook;

/* Host only.  Levels and encoder thresholds of any codebook (as qlora_nf4_codebook);
 * UNSUPPORTED for an unknown codebook.  Either pointer may be NULL.               */
qlora_status qlora_codebook_table(int32_t codebook, float levels[16], float thresholds[15]);

/* Host only.  Bytes of each buffer of a quantized [rows][cols] weight with blocks of
 * block_size (0 = 64) ("Double quantization": 4-bit codes, 8-bit constants per block,
 * one fp32 per 256 constants, one fp32 mean).  rows, cols >= 1.  Any output may be
 * NULL.  UNSUPPORTED for a block size other than 0, 32, 64, 128, 256.             */
qlora_status qlora_nf4_sizes(int64_t rows, int64_t cols, int32_t double_quant, int32_t block_size,
                             size_t* codes_bytes, size_t* absmax_bytes, size_t* c1_bytes, size_t* mu_bytes);

/* Host only.  Workspace bytes each call needs (0 means none; pass ws = NULL). */
size_t qlora_quantize_workspace(int64_t rows, int64_t cols, int32_t double_quant, int32_t block_size);
size_t qlora_fwd_workspace(int64_t M, int64_t in_features, int64_t out_features, int32_t r);
size_t qlora_bwd_workspace(int64_t M, int64_t in_features, int64_t out_features, int32_t r);

/* Blockwise NF4 quantization of W [rows][cols] bf16 into `out` (whose rows,
 * cols, double_quant and buffers the caller sets; see qlora_nf4_sizes).
 * Per block of out->block_size: a = max|w| (a below 2^-126 makes the block all zero codes with
 * a = 0); x = fl32(w * fl32(1/a)); code = nearest level of out->codebook, ties to
 * the lower index ("Quantize in blocks, not all at once"; "NormalFloat").  With
 * double_quant: mu = fl32(S / nblk), S the exact sum of all a rounded once to
 * float64; per group of 256 blocks m = max|fl32(a - mu)|, c1 = fl32(m / 448)
 * (c1 below 2^-126 -> c1 = 0 and codes 0), c2 = E4M3_RNE(fl32(fl32(a - mu) *
 * fl32(1/c1))) ("Double quantization").  Results are deterministic.
 * Any rows, cols >= 1 (a partial last block and group are allowed).
 * Requires: W and out->codes 16-byte aligned; W finite.                          */
qlora_status qlora_quantize_nf4(const uint16_t* W, int64_t rows, int64_t cols, const qlora_nf4* out, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* doubleDequant of a whole weight into W_out [rows][cols] bf16 (bit-exact with
 * the definition in the qlora_nf4 comment).  W_out 16-byte aligned.            */
qlora_status qlora_dequant(const qlora_nf4* w, uint16_t* W_out, hipStream_t stream);

/* Forward ("The QLoRA layer, end to end"):
 *   Y [M][out] = bf16( X [M][in] deq(W)^T + scale * T B ),  T = X A  [M][r]
 * The bf16 weight is decoded inside the kernels and never written out.  T is rounded
 * to bf16 before its product with B.  If T_save is not NULL, bf16(T) is written
 * there [M][r] for the backward.  M >= 0; M = 0 is a no-op, and then the token
 * buffers X, Y and T_save may be NULL.
 * Requires: in % 64 == 0 and in % block_size == 0 (blocks lie inside weight rows),
 * out % 8 == 0 (rows of B, dY and Y are moved as 16-byte vectors of 8 bf16),
 * r % 8 == 0, 8 <= r <= 256; all pointers 16-byte aligned; ws of
 * qlora_fwd_workspace(M, in, out, r) bytes.                                     */
qlora_status qlora_linear_fwd(const uint16_t* X, int64_t M, const qlora_nf4* w, const uint16_t* A,
                              const uint16_t* B, int32_t r, float scale, uint16_t* Y, uint16_t* T_save,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward ("The QLoRA layer, end to end"; no gradient for W):
 *   G  = dY B^T                         [M][r]   (rounded to bf16 after scaling by `scale`)
 *   dX = bf16( dY deq(W) + scale G A^T ) [M][in] (skipped if dX is NULL)
 *   dA = scale X^T G                    [in][r]  fp32, overwritten
 *   dB = scale T^T dY                   [r][out] fp32, overwritten
 * T_saved is bf16(X A) from the forward, or NULL to recompute it.  With M = 0,
 * dA and dB are set to zero and dY, X, T_saved, dX may be NULL.  Same shape and alignment rules as the forward;
 * ws of qlora_bwd_workspace(M, in, out, r) bytes.                              */
qlora_status qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* T_saved, int64_t M,
                              const qlora_nf4* w, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                              uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes, hipStream_t stream);

/* The forward of qlora_linear_fwd with no workspace argument and no allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results (bit for bit) and rules as
 * qlora_linear_fwd; the scratch memory is a fixed array of QLORA_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.  Returns
 * QLORA_ERR_WORKSPACE (and launches nothing) when qlora_fwd_workspace(M, in, out, r) exceeds
 * that size.  Calls that overlap in time on one GPU (several streams or host threads) share
 * the array and race: the caller serializes them.  The first call on each device takes the
 * array's device address (hipGetSymbolAddress) with that device current.                */
#define QLORA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
qlora_status qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M, const qlora_nf4* w, const uint16_t* A,
                                      const uint16_t* B, int32_t r, float scale, uint16_t* Y, uint16_t* T_save,
                                      hipStream_t stream);

/* Merge the adapter into the base weight ("QLoRA: quantising the part you are not
 * training", section "What it costs": merging into the quantised base means
 * requantising): W_out [out][in] bf16 with
 *   W_out[n][k] = bf16_RNE( fl32( deq(W)[n][k] + fl32(scale * d) ) ),
 *   d = fp32 fused multiply-add chain over j = 0..r-1 of A[k][j] * B[j][n],
 * deq(W) the bf16 dequantized weight of the qlora_nf4 comment.  Quantize W_out again
 * with qlora_quantize_nf4 to get a merged 4-bit weight.  Same shape and alignment
 * rules as qlora_linear_fwd (in % 64 == 0, in % block_size == 0, out % 8 == 0, r % 8 == 0,
 * 8 <= r <= 256, 16-byte aligned pointers).                                         */
qlora_status qlora_merge_adapter(const qlora_nf4* w, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                                 uint16_t* W_out, hipStream_t stream);

/* One AdamW step on n adapter parameters ("Paged optimizers": only the adapters carry
 * gradients and optimizer state, kept in fp32).  With t = step (>= 1), in fp32 with each
 * product and sum rounded separately, the bias corrections formed on the host in float64:
 *   p <- p * (1 - lr wd)
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - (lr / (1 - beta1^t)) m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * param, m, v are updated in place; if param_bf16 is not NULL, bf16_RNE(p) is written there
 * (the working copy qlora_linear_fwd/bwd read as A or B).  grad is dA or dB from
 * qlora_linear_bwd.  The state may live in any memory the GPU can address (device memory,
 * or host memory the caller has made device-accessible to page the state out).
 * Requires: n >= 0 (0 is a no-op); step >= 1; 0 <= beta1, beta2 < 1; eps > 0; param, grad,
 * m, v non-NULL and 16-byte aligned, param_bf16 8-byte aligned; no overlap.             */
qlora_status qlora_adamw_step(float* param, uint16_t* param_bf16, const float* grad, float* m, float* v, int64_t n,
                              int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                              hipStream_t stream);

/* Paging of optimizer state ("QLoRA: Efficient Finetuning of Quantized LLMs", section
 * "Paged optimizers": the adapters' optimizer state is moved out to CPU memory when GPU
 * memory runs short and brought back before the optimizer step needs it).  The state stays
 * in device memory by default; these calls move `bytes` bytes of it between device memory
 * and pinned host memory with the GPU's copy engines, asynchronously on `stream` (the copy
 * is ordered after earlier work on the stream and before later work, so a page-in followed
 * by qlora_adamw_step on the same stream updates the paged-in state).
 *   qlora_state_page_out: device -> host;  qlora_state_page_in: host -> device.
 * Requires: both pointers non-NULL and 16-byte aligned; bytes a multiple of 4 (0 is a
 * no-op); `host` inside pinned host memory (hipHostMalloc, torch pin_memory) and `device`
 * inside device memory, as the HIP runtime reports them (UNSUPPORTED otherwise: pageable
 * memory would make the copy synchronous); the two ranges must not overlap.  The caller
 * keeps the host buffer alive until the copy has completed.                            */
qlora_status qlora_state_page_out(const void* device, void* host, size_t bytes, hipStream_t stream);
qlora_status qlora_state_page_in(const void* host, void* device, size_t bytes, hipStream_t stream);

/* Optional per-kernel timing, for benchmarking.  While enabled, every kernel
 * launch of this library is bracketed by HIP events on its stream.
 * qlora_profile_read synchronizes those events and returns, per kernel name,
 * the launch count and total milliseconds since the last reset; returns the
 * number of entries written (at most max_entries).  Not thread-safe against
 * concurrent launches from other threads while reading.                        */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} qlora_kernel_time;

qlora_status qlora_profile_enable(int32_t enable);
int32_t qlora_profile_read(qlora_kernel_time* out, int32_t max_entries, int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
