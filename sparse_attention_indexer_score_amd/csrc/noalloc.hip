// idx_fused_topk_noalloc: the fused top-k with a workspace that the library owns, for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The workspace is the file-scope device array `scratch` (IDX_NOALLOC_SCRATCH_BYTES), one
// copy per GPU, held until the process ends.  Its device address is resolved once per
// device with hipGetSymbolAddress (with that device current) and kept; in host code the
// array's name is only a stand-in and is never passed to a kernel.  Every call on a GPU
// shares that GPU's array: calls that overlap on one GPU (two streams, two threads) race.
// Nothing in it needs clearing between calls: the threshold kernel resets the counters,
// the fallback queue and the statistics at the start of every call, and every other region
// is written before it is read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/idx.h"

namespace {

__device__ __align__(256) uint8_t scratch[IDX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once resolved
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (resolved on the first call on that device).
int device_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return IDX_ENODEV;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return IDX_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return IDX_OK;
}

}  // namespace

extern "C" int idx_fused_topk_noalloc(const idx_problem* p, int32_t k, int32_t* out_idx, void* stream) {
  const size_t need = idx_fused_workspace(p, k);
  // Invalid arguments: the checks of idx_fused_topk give the error (before any device work).
  if (need == 0) return idx_fused_topk(p, k, out_idx, nullptr, 0, nullptr, stream);
  if (need > (size_t)IDX_NOALLOC_SCRATCH_BYTES) return IDX_ESCRATCH;
  void* ws = nullptr;
  const int rc = device_scratch(&ws);
  if (rc != IDX_OK) return rc;
  return idx_fused_topk(p, k, out_idx, ws, (size_t)IDX_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}
