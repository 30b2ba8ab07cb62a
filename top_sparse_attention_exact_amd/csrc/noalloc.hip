// atopk_bucketed_noalloc: atopk_bucketed with the library's own scratch array
// as the workspace, for callers that cannot allocate device memory.
//
// The workspace is `scratch`, a file-scope device array of kScratchBytes.
// Each GPU the library runs on holds its own copy from the first time the
// library's code is loaded on it until the process ends.  Host code reaches
// a device's copy only through the address hipGetSymbolAddress returns with
// that device current, cached per device on the first call made there; the
// array's name on the host side is not a device address and is never passed
// to a kernel.  Calls on one GPU share its array: two calls in flight at once
// on one GPU (on different streams, or from different threads without
// ordering between them) race on it.  The bucketed kernels write every part
// of their workspace before reading it, so nothing needs clearing between
// calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "atopk.h"

namespace {

constexpr size_t kScratchBytes = ATOPK_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's copy of `scratch` (nullptr if the runtime refuses).
void* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int atopk_bucketed_noalloc(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                           int64_t kb, int final_exact, void* out_vals, int32_t* out_idx, void* stream) {
  size_t need = 0;
  int st = atopk_bucketed_workspace(dtype, m, n, ldx, k, b, kb, final_exact, &need);
  if (st != ATOPK_OK) return st;
  if (need > kScratchBytes) return ATOPK_ERR_WORKSPACE;
  if (m == 0) return atopk_bucketed(x, dtype, m, n, ldx, k, b, kb, final_exact, out_vals, out_idx, nullptr, 0, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATOPK_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATOPK_ERR_UNSUPPORTED;
  void* ws = scratch_on(dev);
  if (ws == nullptr) return ATOPK_ERR_HIP;
  return atopk_bucketed(x, dtype, m, n, ldx, k, b, kb, final_exact, out_vals, out_idx, ws, kScratchBytes, stream);
}

}  // extern "C"
