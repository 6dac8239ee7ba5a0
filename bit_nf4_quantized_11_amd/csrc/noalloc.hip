// qlora_linear_fwd_noalloc: the forward with its scratch memory in a fixed device array of
// the library instead of a caller workspace, for callers that cannot allocate.
//
// The array is a file-scope __device__ object: every GPU the library runs on holds its own
// copy (QLORA_NOALLOC_SCRATCH_BYTES) from the moment the code object is loaded until the
// process ends.  Host code never passes the array's name to a kernel (on the host that name
// is a stand-in, not a device address): on the first call on a device, with that device
// current, its device address is taken with hipGetSymbolAddress and kept per device; every
// later call on that device uses the kept address.
//
// The forward needs no scratch that starts at zero: every partial sum and intermediate it
// reads was written earlier in the same call, so the array's previous contents never matter.
// Calls that overlap in time on one GPU (different streams, or several host threads) share
// the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "qlora.h"

namespace {

static_assert(QLORA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's copy of the scratch array (the current device's), or NULL
// if the runtime cannot give it.
void* scratch_of_current_device(int dev) {
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" qlora_status qlora_linear_fwd_noalloc(const uint16_t* X, int64_t M, const qlora_nf4* w, const uint16_t* A,
                                                 const uint16_t* B, int32_t r, float scale, uint16_t* Y,
                                                 uint16_t* T_save, hipStream_t stream) {
  const qlora_status st = qlora::linear_fwd_check(X, M, w, A, B, r, Y, T_save);
  if (st != QLORA_OK) return st;
  const size_t need = qlora_fwd_workspace(M, w->cols, w->rows, r);
  if (need > (size_t)QLORA_NOALLOC_SCRATCH_BYTES) return QLORA_ERR_WORKSPACE;
  if (M == 0) return QLORA_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  void* ws = scratch_of_current_device(dev);
  if (!ws) return QLORA_ERR_HIP;
  return qlora_linear_fwd(X, M, w, A, B, r, scale, Y, T_save, ws, (size_t)QLORA_NOALLOC_SCRATCH_BYTES, stream);
}
