// libqlora host layer: the C ABI declared in include/qlora.h.
//
// Validates every argument on the host, carves the caller's workspace, and
// enqueues the kernels on the caller's stream.  Allocates no device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "qlora.h"

namespace qlora {

// ------------------------------------------------------------------------------------------
// per-kernel timing (optional)
// ------------------------------------------------------------------------------------------
namespace {
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
std::atomic<int> g_prof_enabled{0};
std::mutex g_prof_mu;
std::vector<ProfRecord> g_prof_pending;
struct ProfAgg {
  std::string name;
  int64_t launches = 0;
  double ms = 0.0;
};
std::vector<ProfAgg> g_prof_agg;
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : slot_(-1), s_(s) {
  if (!g_prof_enabled.load(std::memory_order_relaxed)) return;
  ProfRecord rec{name, nullptr, nullptr};
  if (hipEventCreate(&rec.start) != hipSuccess) return;
  if (hipEventCreate(&rec.stop) != hipSuccess) {
    (void)hipEventDestroy(rec.start);
    return;
  }
  (void)hipEventRecord(rec.start, s);
  std::lock_guard<std::mutex> g(g_prof_mu);
  slot_ = (int)g_prof_pending.size();
  g_prof_pending.push_back(rec);
}

ProfScope::~ProfScope() {
  if (slot_ < 0) return;
  hipEvent_t stop;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    stop = g_prof_pending[slot_].stop;
  }
  (void)hipEventRecord(stop, s_);
}

}  // namespace qlora

using namespace qlora;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t rank_pad(int64_t r) { return (r + 63) / 64 * 64; }

// Sequential carving of a workspace into 256-byte aligned pieces.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    off = round_up(off, 256);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// Weights per constant (0 in the descriptor means 64) and its log2; 0 for an unknown size.
int block_of(int32_t b) { return b == 0 ? 64 : b; }
int block_shift(int32_t b) {
  switch (block_of(b)) {
    case 32: return 5;
    case 64: return 6;
    case 128: return 7;
    case 256: return 8;
  }
  return 0;
}
// elements the code buffer holds: whole blocks and whole 64-element chunks
int64_t code_elems(int64_t numel, int block) {
  const int64_t unit = std::max(block, 64);
  return (numel + unit - 1) / unit * unit;
}

NF4View view_of(const qlora_nf4* w) {
  NF4View v;
  v.codes = w->codes;
  v.absmax = w->absmax;
  v.c1 = w->c1;
  v.mu = w->mu;
  v.dq = w->double_quant;
  v.cb = w->codebook;
  v.bshift = block_shift(w->block_size);
  return v;
}

#define QL_HIP(call)                              \
  do {                                            \
    if ((call) != hipSuccess) return QLORA_ERR_HIP; \
  } while (0)

qlora_status check_nf4(const qlora_nf4* w) {
  if (!w || !w->codes || !w->absmax) return QLORA_ERR_NULL;
  if (w->double_quant != 0 && w->double_quant != 1) return QLORA_ERR_UNSUPPORTED;
  if (w->codebook < 0 || w->codebook >= kNumCodebooks) return QLORA_ERR_UNSUPPORTED;
  if (block_shift(w->block_size) == 0) return QLORA_ERR_UNSUPPORTED;
  if (w->double_quant && (!w->c1 || !w->mu)) return QLORA_ERR_NULL;
  if (w->rows < 1 || w->cols < 1 || w->rows >= kMaxDim || w->cols >= kMaxDim) return QLORA_ERR_SHAPE;
  if (!aligned16(w->codes) || !aligned4(w->absmax) || (w->c1 && !aligned4(w->c1)) || (w->mu && !aligned4(w->mu)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

qlora_status check_linear(int64_t M, const qlora_nf4* w, int32_t r) {
  qlora_status st = check_nf4(w);
  if (st != QLORA_OK) return st;
  if (M < 0 || M >= (int64_t(1) << 26)) return QLORA_ERR_SHAPE;
  if (w->cols % 64 != 0 || w->cols % block_of(w->block_size) != 0 || w->rows % 8 != 0) return QLORA_ERR_SHAPE;
  if (w->rows > (int64_t(1) << 22) || w->cols > (int64_t(1) << 22)) return QLORA_ERR_SHAPE;
  if (r < 8 || r > 256 || r % 8 != 0) return QLORA_ERR_UNSUPPORTED;
  // the large-M kernels address each operand with 32-bit byte offsets
  const uint64_t lim = uint64_t(1) << 32;
  const uint64_t in = (uint64_t)w->cols, out = (uint64_t)w->rows;
  if (((uint64_t)M + 512) * std::max(in, out) * 2 >= lim) return QLORA_ERR_SHAPE;
  if ((out + 128) * (in / 64) * 32 >= lim) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

// ---- workspace layouts ----------------------------------------------------------------------
constexpr int kMaxSplits = kMaxLoraSplits;

SmallGemm gemm_T(const uint16_t* X, const uint16_t* A, int64_t M, int64_t in, int64_t r) {
  // T[m][j] = sum_k X[m][k] A[k][j]
  return SmallGemm{X, in, 1, A, r, 1, M, r, in};
}
SmallGemm gemm_G(const uint16_t* dY, const uint16_t* B, int64_t M, int64_t out, int64_t r) {
  // G[m][j] = sum_n dY[m][n] B[j][n]
  return SmallGemm{dY, out, 1, B, 1, out, M, r, out};
}
SmallGemm gemm_dA(const uint16_t* X, const uint16_t* Gs, int64_t M, int64_t in, int64_t r, int64_t rp) {
  // dA[i][j] = sum_m X[m][i] Gs[m][j]
  return SmallGemm{X, 1, in, Gs, rp, 1, in, r, M};
}
SmallGemm gemm_dB(const uint16_t* T, int64_t ldT, const uint16_t* dY, int64_t M, int64_t out, int64_t r) {
  // dB[j][n] = sum_m T[m][j] dY[m][n]
  return SmallGemm{T, 1, ldT, dY, out, 1, r, out, M};
}

bool use_gemv(int64_t M) { return M <= 64; }   // few tokens: the weight-streaming path

// Up to 1024 tokens the large-M GEMM has ceil(M/256) token panels x out/128 feature tiles,
// which can leave most of the GPU idle: cut the reduction into slices of `stages` stages so
// that tiles x slices come to about one workgroup per CU (at least 4 stages a slice).
// Returns the stages per slice, or 0 for the plain path.  The epilogue's cost grows with
// the output (M x out) and the slices: 2 slices measured at best even and up to 23 %
// slower (4096 -> 16384 and 16384 -> 4096 at 128 and 256 tokens, 4096 x 4096 at 1024),
// 4 or more faster by 15-45 %; so the slices must at least triple the workgroups for one
// token panel and at least quadruple them past it.  (Past 1024 tokens the X A workgroups of the
// weight-streaming kernel, one per 16-token group, would re-read A too often; 64 tokens or
// fewer take the weight-streaming path itself.)
constexpr int64_t kSplitMaxTokens = 1024;
int64_t min_slices(int64_t M) { return M > 256 ? 4 : 3; }
int64_t split_stages(int64_t M, int64_t in, int64_t out) {
  if (M <= 64 || M > kSplitMaxTokens) return 0;
  const int64_t tiles = ((M + 255) / 256) * ((out + 127) / 128), nkb = in / 64;
  if (tiles < 1) return 0;   // a size query with an empty dimension
  const int64_t s = std::min((256 + tiles / 2) / tiles, nkb / 4);
  if (s < min_slices(M)) return 0;
  return (nkb + s - 1) / s;
}
int64_t split_count(int64_t in, int64_t stages) { return (in / 64 + stages - 1) / stages; }

// The same for dX (the backward has no weight-streaming path, so from one token on):
// in/128 column tiles per token panel, ceil(out/64) reduction stages over the weight's rows.
int64_t dx_split_stages(int64_t M, int64_t in, int64_t out) {
  if (M > kSplitMaxTokens) return 0;
  const int64_t tiles = ((M + 255) / 256) * ((in + 127) / 128), nred = (out + 63) / 64;
  if (tiles < 1) return 0;   // M = 0 (or a size query with an empty dimension)
  const int64_t s = std::min((256 + tiles / 2) / tiles, nred / 4);
  if (s < min_slices(M)) return 0;
  return (nred + s - 1) / s;
}
int64_t dx_split_count(int64_t out, int64_t stages) { return ((out + 63) / 64 + stages - 1) / stages; }

LoraEpi epi_none() { return LoraEpi{nullptr, 0, 0.0f, nullptr, 0, 0.0f, nullptr, 0.0f}; }

struct FwdWs {
  uint16_t* Ts;
  float* partial;
  LoraProblem t;
  GemvPlan gv;
  size_t bytes;
};

FwdWs fwd_layout(void* base, int64_t M, int64_t in, int64_t out, int32_t r) {
  Carve c(base);
  const int64_t rp = rank_pad(r);
  const int64_t Mm = std::max<int64_t>(M, 1);
  FwdWs ws;
  ws.t = lora_problem(gemm_T(nullptr, nullptr, Mm, in, r), epi_none(), kMaxSplits);
  const int64_t st = split_stages(M, in, out);
  ws.gv = gemv_plan(Mm, in, out, rp, st != 0);
  if (st) {   // the split forward's slices take the place of the weight slices
    ws.gv.splits = (int)split_count(in, st);
    ws.gv.tpart = (size_t)ws.gv.splits * Mm * ws.gv.npad;
  }
  const size_t pf = use_gemv(M) || st ? gemv_partial_floats(ws.gv, Mm) : lora_partial_floats(ws.t);
  ws.Ts = c.take<uint16_t>((size_t)Mm * rp);
  ws.partial = c.take<float>(std::max<size_t>(pf, 1));
  ws.bytes = round_up(c.off, 256);
  return ws;
}

struct BwdWs {
  uint16_t* Gs;
  uint16_t* T;
  float* partial;
  LoraProblem t, g, da, db;
  size_t bytes;
};

BwdWs bwd_layout(void* base, int64_t M, int64_t in, int64_t out, int32_t r) {
  Carve c(base);
  const int64_t rp = rank_pad(r);
  const int64_t Mm = std::max<int64_t>(M, 1);
  BwdWs ws;
  ws.t = lora_problem(gemm_T(nullptr, nullptr, Mm, in, r), epi_none(), kMaxSplits);
  ws.g = lora_problem(gemm_G(nullptr, nullptr, Mm, out, r), epi_none(), kMaxSplits);
  ws.da = lora_problem(gemm_dA(nullptr, nullptr, Mm, in, r, rp), epi_none(), kMaxSplits);
  ws.db = lora_problem(gemm_dB(nullptr, r, nullptr, Mm, out, r), epi_none(), kMaxSplits);
  const int64_t dst = dx_split_stages(M, in, out);
  const size_t pdx = dst ? (size_t)dx_split_count(out, dst) * Mm * in : 0;   // split dX partials
  // the split dX partials follow G's partials, which its epilogue still reads
  const size_t pf = std::max({lora_partial_floats(ws.t), lora_partial_floats(ws.g) + pdx,
                              lora_partial_floats(ws.da) + lora_partial_floats(ws.db)});
  ws.Gs = c.take<uint16_t>((size_t)Mm * rp);
  ws.T = c.take<uint16_t>((size_t)Mm * r);
  ws.partial = c.take<float>(std::max<size_t>(pf, 1));
  ws.bytes = round_up(c.off, 256);
  return ws;
}

struct QuantWs {
  unsigned long long* sums;   // one exact partial sum of the block constants per quantize workgroup
  float* absmax;
  size_t bytes;
};

QuantWs quant_layout(void* base, int64_t numel, int block) {
  Carve c(base);
  QuantWs ws;
  ws.sums = c.take<unsigned long long>((size_t)kQuantSlots * kSumLimbs);
  ws.absmax = c.take<float>((size_t)((numel + block - 1) / block));
  ws.bytes = round_up(c.off, 256);
  return ws;
}

}  // namespace

namespace qlora {
// Argument checks of the forward (everything except the workspace), shared with the entry
// point that brings its own scratch memory.
qlora_status linear_fwd_check(const uint16_t* X, int64_t M, const qlora_nf4* w, const uint16_t* A, const uint16_t* B,
                              int32_t r, const uint16_t* Y, const uint16_t* T_save) {
  const qlora_status st = check_linear(M, w, r);
  if (st != QLORA_OK) return st;
  // with no tokens the token buffers may be NULL (e.g. empty tensors)
  if (!A || !B || (M > 0 && (!X || !Y))) return QLORA_ERR_NULL;
  if ((X && !aligned16(X)) || !aligned16(A) || !aligned16(B) || (Y && !aligned16(Y)) ||
      (T_save && !aligned16(T_save)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}
}  // namespace qlora

extern "C" {

const char* qlora_status_str(qlora_status s) {
  switch (s) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "required pointer is NULL";
    case QLORA_ERR_SHAPE: return "size out of range or violates a divisibility rule";
    case QLORA_ERR_ALIGN: return "pointer not aligned as required";
    case QLORA_ERR_UNSUPPORTED: return "unsupported option";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_HIP: return "HIP runtime call or kernel launch failed";
  }
  return "unknown status";
}

#ifndef QLORA_SOURCE_HASH
#define QLORA_SOURCE_HASH "unknown"
#endif
const char* qlora_version(void) { return "libqlora 0.2 (gfx950, src " QLORA_SOURCE_HASH ")"; }

qlora_status qlora_codebook_table(int32_t codebook, float levels[16], float thresholds[15]) {
  if (codebook < 0 || codebook >= kNumCodebooks) return QLORA_ERR_UNSUPPORTED;
  if (levels) std::memcpy(levels, codebook_levels_host(codebook), 16 * sizeof(float));
  if (thresholds) std::memcpy(thresholds, codebook_thresholds_host(codebook), 15 * sizeof(float));
  return QLORA_OK;
}

qlora_status qlora_nf4_codebook(float levels[16], float thresholds[15]) {
  if (levels) std::memcpy(levels, nf4_levels_host(), 16 * sizeof(float));
  if (thresholds) std::memcpy(thresholds, nf4_thresholds_host(), 15 * sizeof(float));
  return QLORA_OK;
}

qlora_status qlora_nf4_sizes(int64_t rows, int64_t cols, int32_t dq, int32_t block_size, size_t* codes_bytes,
                             size_t* absmax_bytes, size_t* c1_bytes, size_t* mu_bytes) {
  if (rows < 1 || cols < 1 || rows >= kMaxDim || cols >= kMaxDim) return QLORA_ERR_SHAPE;
  if (dq != 0 && dq != 1) return QLORA_ERR_UNSUPPORTED;
  if (block_shift(block_size) == 0) return QLORA_ERR_UNSUPPORTED;
  const int block = block_of(block_size);
  const int64_t numel = rows * cols;
  const int64_t nblk = (numel + block - 1) / block;
  const int64_t nsup = (nblk + 255) / 256;
  if (codes_bytes) *codes_bytes = (size_t)code_elems(numel, block) / 2;
  if (absmax_bytes) *absmax_bytes = (size_t)nblk * (dq ? 1 : 4);
  if (c1_bytes) *c1_bytes = dq ? (size_t)nsup * 4 : 0;
  if (mu_bytes) *mu_bytes = dq ? 4 : 0;
  return QLORA_OK;
}

size_t qlora_quantize_workspace(int64_t rows, int64_t cols, int32_t dq, int32_t block_size) {
  if (!dq || rows < 1 || cols < 1 || rows >= kMaxDim || cols >= kMaxDim || block_shift(block_size) == 0) return 0;
  return quant_layout(nullptr, rows * cols, block_of(block_size)).bytes;
}

size_t qlora_fwd_workspace(int64_t M, int64_t in, int64_t out, int32_t r) {
  if (M < 0 || in < 64 || out < 8 || r < 8 || r > 256) return 0;
  return fwd_layout(nullptr, M, in, out, r).bytes;
}

size_t qlora_bwd_workspace(int64_t M, int64_t in, int64_t out, int32_t r) {
  if (M < 0 || in < 64 || out < 8 || r < 8 || r > 256) return 0;
  return bwd_layout(nullptr, M, in, out, r).bytes;
}

qlora_status qlora_quantize_nf4(const uint16_t* W, int64_t rows, int64_t cols, const qlora_nf4* out, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  if (!W || !out || !out->codes || !out->absmax) return QLORA_ERR_NULL;
  if (rows < 1 || cols < 1 || rows >= kMaxDim || cols >= kMaxDim) return QLORA_ERR_SHAPE;
  if (out->rows != rows || out->cols != cols) return QLORA_ERR_SHAPE;
  const qlora_status st = check_nf4(out);
  if (st != QLORA_OK) return st;
  if (!aligned16(W)) return QLORA_ERR_ALIGN;
  const int64_t numel = rows * cols;
  const int block = block_of(out->block_size);
  const int64_t nblk = (numel + block - 1) / block;
  if (out->double_quant) {
    const QuantWs need = quant_layout(nullptr, numel, block);
    if (!ws || ws_bytes < need.bytes) return QLORA_ERR_WORKSPACE;
    if (!aligned16(ws)) return QLORA_ERR_ALIGN;
    const QuantWs q = quant_layout(ws, numel, block);
    QL_HIP(launch_quantize(W, numel, out->codebook, block, out->codes, q.absmax, q.sums, stream));
    QL_HIP(launch_dq_encode(q.absmax, nblk, q.sums, quantize_grid(numel, block), out->mu,
                            static_cast<uint8_t*>(out->absmax), out->c1, stream));
  } else {
    QL_HIP(launch_quantize(W, numel, out->codebook, block, out->codes, static_cast<float*>(out->absmax), nullptr,
                           stream));
  }
  return QLORA_OK;
}

qlora_status qlora_dequant(const qlora_nf4* w, uint16_t* W_out, hipStream_t stream) {
  const qlora_status st = check_nf4(w);
  if (st != QLORA_OK) return st;
  if (!W_out) return QLORA_ERR_NULL;
  if (!aligned16(W_out)) return QLORA_ERR_ALIGN;
  QL_HIP(launch_dequant(view_of(w), w->rows * w->cols, W_out, stream));
  return QLORA_OK;
}

qlora_status qlora_linear_fwd(const uint16_t* X, int64_t M, const qlora_nf4* w, const uint16_t* A,
                              const uint16_t* B, int32_t r, float scale, uint16_t* Y, uint16_t* T_save, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  const qlora_status st = qlora::linear_fwd_check(X, M, w, A, B, r, Y, T_save);
  if (st != QLORA_OK) return st;
  const int64_t in = w->cols, out = w->rows, rp = rank_pad(r);
  const FwdWs need = fwd_layout(nullptr, M, in, out, r);
  if (!ws || ws_bytes < need.bytes) return QLORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (M == 0) return QLORA_OK;
  const FwdWs L = fwd_layout(ws, M, in, out, r);
  const NF4View v = view_of(w);

  if (use_gemv(M)) {
    // few tokens: one pass over the packed weight that also forms the partials of X A, then
    // an epilogue that finishes T, Ts and Y
    QL_HIP(launch_gemv(X, M, in, out, v, A, r, L.gv, L.partial, stream));
    QL_HIP(launch_gemv_epilogue(L.partial, L.gv, M, out, B, r, scale, Y, T_save, stream));
    return QLORA_OK;
  }
  if (const int64_t st = split_stages(M, in, out)) {
    // one token panel, few feature tiles: X A partials, the GEMM in K-slices (fp32 partials),
    // and the weight-streaming path's epilogue for the sums, T, Ts B and Y
    QL_HIP(launch_gemv(X, M, in, out, v, A, r, L.gv, L.partial, stream, true));
    QL_HIP(launch_fwd_gemm_split(X, M, in, out, v, (int)st, L.partial, L.gv.npad, stream));
    QL_HIP(launch_gemv_epilogue(L.partial, L.gv, M, out, B, r, scale, Y, T_save, stream));
    return QLORA_OK;
  }
  // T = X A (bf16 to T_save) and Ts = bf16(s T) padded to rp columns, then the fused product
  LoraProblem pt = lora_problem(gemm_T(X, A, M, in, r), LoraEpi{T_save, r, 1.0f, L.Ts, rp, scale, nullptr, 0.0f},
                                kMaxSplits);
  pt.partial = L.partial;
  QL_HIP(launch_lora(pt, nullptr, "k_lora_xa", stream));
  if (pt.splits > 1) QL_HIP(launch_lora_reduce(pt, nullptr, "k_lora_xa_reduce", stream));
  QL_HIP(launch_fwd_gemm(X, M, in, out, v, L.Ts, rp, B, r, Y, stream));
  return QLORA_OK;
}

qlora_status qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* T_saved, int64_t M,
                              const qlora_nf4* w, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                              uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes, hipStream_t stream) {
  qlora_status st = check_linear(M, w, r);
  if (st != QLORA_OK) return st;
  if (!A || !B || !dA || !dB || (M > 0 && (!dY || !X))) return QLORA_ERR_NULL;
  if ((dY && !aligned16(dY)) || (X && !aligned16(X)) || !aligned16(A) || !aligned16(B) ||
      (T_saved && !aligned16(T_saved)) || (dX && !aligned16(dX)) || !aligned4(dA) || !aligned4(dB))
    return QLORA_ERR_ALIGN;
  const int64_t in = w->cols, out = w->rows, rp = rank_pad(r);
  const BwdWs need = bwd_layout(nullptr, M, in, out, r);
  if (!ws || ws_bytes < need.bytes) return QLORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  if (M == 0) {
    QL_HIP(launch_fill_u32(reinterpret_cast<uint32_t*>(dA), in * r, 0u, stream));
    QL_HIP(launch_fill_u32(reinterpret_cast<uint32_t*>(dB), (int64_t)r * out, 0u, stream));
    return QLORA_OK;
  }
  const BwdWs L = bwd_layout(ws, M, in, out, r);
  const NF4View v = view_of(w);

  const uint16_t* T = T_saved;
  if (!T) {
    LoraProblem pt = lora_problem(gemm_T(X, A, M, in, r), LoraEpi{L.T, r, 1.0f, nullptr, 0, 0.0f, nullptr, 0.0f},
                                  kMaxSplits);
    pt.partial = L.partial;
    QL_HIP(launch_lora(pt, nullptr, "k_lora_xa", stream));
    if (pt.splits > 1) QL_HIP(launch_lora_reduce(pt, nullptr, "k_lora_xa_reduce", stream));
    T = L.T;
  }
  // Gs = bf16(s dY B^T), padded to rp columns
  LoraProblem pg = lora_problem(gemm_G(dY, B, M, out, r), LoraEpi{nullptr, 0, 0.0f, L.Gs, rp, scale, nullptr, 0.0f},
                                kMaxSplits);
  pg.partial = L.partial;
  const int64_t dst = dX ? dx_split_stages(M, in, out) : 0;
  // with the split dX and at most 64 tokens, its epilogue sums G's partials itself (and stores
  // Gs for dA); with more tokens every one of its in/64 column blocks would repeat that sum for
  // its token group, which costs more than the reduce launch (measured at 256 and 512 tokens).
  // G's split-K workgroups then run inside the split dX launch (nothing there depends on G).
  const bool fold_g = dst && pg.splits > 1 && M <= 64;
  if (!fold_g) QL_HIP(launch_lora(pg, nullptr, "k_lora_dyb", stream));
  if (pg.splits > 1 && !fold_g) QL_HIP(launch_lora_reduce(pg, nullptr, "k_lora_dyb_reduce", stream));
  if (dX) {
    if (dst) {
      // few tokens, few column tiles: the reduction in slices (fp32 partials, after G's),
      // then the slices' sum plus Gs A^T in one epilogue
      float* const dxpart = L.partial + lora_partial_floats(pg);
      const GFold gf{fold_g ? L.partial : nullptr, pg.splits, pg.tiles_j, scale, L.Gs};
      QL_HIP(launch_dx_gemm_split(dY, M, in, out, v, (int)dst, dxpart, stream, fold_g ? &pg : nullptr));
      if (M <= 16) {
        // one token group: the epilogue also forms dA (from its Gs) and dB (extra workgroups),
        // so the backward ends here
        const GradFold gr{X, T, dY, dA, dB, out, scale};
        QL_HIP(launch_dx_split_epilogue(dxpart, (int)dx_split_count(out, dst), M, in, L.Gs, rp, A, r, dX, gf, stream,
                                        &gr));
        return QLORA_OK;
      }
      QL_HIP(launch_dx_split_epilogue(dxpart, (int)dx_split_count(out, dst), M, in, L.Gs, rp, A, r, dX, gf, stream));
    } else {
      QL_HIP(launch_dx_gemm(dY, M, in, out, v, L.Gs, rp, A, r, dX, stream));
    }
  }
  // dA = X^T Gs and dB = s T^T dY, one launch for both products and one for both reductions
  LoraProblem pa = lora_problem(gemm_dA(X, L.Gs, M, in, r, rp),
                                LoraEpi{nullptr, 0, 0.0f, nullptr, 0, 0.0f, dA, 1.0f}, kMaxSplits);
  LoraProblem pb = lora_problem(gemm_dB(T, r, dY, M, out, r),
                                LoraEpi{nullptr, 0, 0.0f, nullptr, 0, 0.0f, dB, scale}, kMaxSplits);
  pa.partial = L.partial;
  pb.partial = L.partial + lora_partial_floats(pa);
  QL_HIP(launch_lora(pa, &pb, "k_lora_da_db", stream));
  if (pa.splits > 1 || pb.splits > 1) {
    // a product computed in one split wrote its outputs directly; reduce only the others
    if (pa.splits > 1 && pb.splits > 1)
      QL_HIP(launch_lora_reduce(pa, &pb, "k_lora_da_db_reduce", stream));
    else
      QL_HIP(launch_lora_reduce(pa.splits > 1 ? pa : pb, nullptr, "k_lora_da_db_reduce", stream));
  }
  return QLORA_OK;
}

qlora_status qlora_profile_enable(int32_t enable) {
  g_prof_enabled.store(enable ? 1 : 0);
  return QLORA_OK;
}

int32_t qlora_profile_read(qlora_kernel_time* outp, int32_t max_entries, int32_t reset) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& rec : g_prof_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(rec.stop) == hipSuccess && hipEventElapsedTime(&ms, rec.start, rec.stop) == hipSuccess) {
      auto it = std::find_if(g_prof_agg.begin(), g_prof_agg.end(),
                             [&](const ProfAgg& a) { return a.name == rec.name; });
      if (it == g_prof_agg.end()) {
        g_prof_agg.push_back(ProfAgg{rec.name, 0, 0.0});
        it = g_prof_agg.end() - 1;
      }
      it->launches += 1;
      it->ms += ms;
    }
    (void)hipEventDestroy(rec.start);
    (void)hipEventDestroy(rec.stop);
  }
  g_prof_pending.clear();
  int32_t n = 0;
  for (const auto& a : g_prof_agg) {
    if (n >= max_entries || !outp) break;
    std::memset(&outp[n], 0, sizeof(qlora_kernel_time));
    std::strncpy(outp[n].name, a.name.c_str(), sizeof(outp[n].name) - 1);
    outp[n].launches = a.launches;
    outp[n].total_ms = a.ms;
    ++n;
  }
  if (reset) g_prof_agg.clear();
  return n;
}

qlora_status qlora_merge_adapter(const qlora_nf4* w, const uint16_t* A, const uint16_t* B, int32_t r, float scale,
                                 uint16_t* W_out, hipStream_t stream) {
  const qlora_status st = check_linear(0, w, r);
  if (st != QLORA_OK) return st;
  if (!A || !B || !W_out) return QLORA_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(W_out)) return QLORA_ERR_ALIGN;
  QL_HIP(launch_merge_adapter(view_of(w), w->rows, w->cols, A, B, r, scale, W_out, stream));
  return QLORA_OK;
}

}  // extern "C"

namespace {
// hipMemoryTypeHost for pinned host memory, hipMemoryTypeDevice for device memory; -1 when the
// runtime does not know the pointer (pageable host memory)
int memory_type(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error the query leaves for unknown pointers
    return -1;
  }
  return (int)a.type;
}

qlora_status page_copy(const void* src, void* dst, size_t bytes, bool to_host, hipStream_t stream) {
  if (!src || !dst) return QLORA_ERR_NULL;
  if (bytes % 4 != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return QLORA_ERR_ALIGN;
  if (bytes == 0) return QLORA_OK;
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return QLORA_ERR_SHAPE;
  const void* host = to_host ? dst : src;
  const void* dev = to_host ? src : dst;
  if (memory_type(host) != (int)hipMemoryTypeHost || memory_type(dev) != (int)hipMemoryTypeDevice)
    return QLORA_ERR_UNSUPPORTED;
  ProfScope ps(to_host ? "page_out_copy" : "page_in_copy", stream);
  QL_HIP(hipMemcpyAsync(dst, src, bytes, to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice, stream));
  return QLORA_OK;
}
}  // namespace

extern "C" {

qlora_status qlora_state_page_out(const void* device, void* host, size_t bytes, hipStream_t stream) {
  return page_copy(device, host, bytes, true, stream);
}

qlora_status qlora_state_page_in(const void* host, void* device, size_t bytes, hipStream_t stream) {
  return page_copy(host, device, bytes, false, stream);
}

qlora_status qlora_adamw_step(float* param, uint16_t* param_bf16, const float* grad, float* m, float* v, int64_t n,
                              int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                              hipStream_t stream) {
  if (n < 0 || step < 1) return QLORA_ERR_SHAPE;
  if (!(beta1 >= 0.0f && beta1 < 1.0f && beta2 >= 0.0f && beta2 < 1.0f && eps > 0.0f)) return QLORA_ERR_UNSUPPORTED;
  if (n == 0) return QLORA_OK;
  if (!param || !grad || !m || !v) return QLORA_ERR_NULL;
  if (!aligned16(param) || !aligned16(grad) || !aligned16(m) || !aligned16(v) ||
      (param_bf16 && (reinterpret_cast<uintptr_t>(param_bf16) & 7u)))
    return QLORA_ERR_ALIGN;
  QL_HIP(launch_adamw(param, param_bf16, grad, m, v, n, step, lr, beta1, beta2, eps, weight_decay, stream));
  return QLORA_OK;
}

}  // extern "C"
