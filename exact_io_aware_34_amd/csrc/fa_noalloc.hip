// fa_decode_noalloc: fa_decode with its key-range partials in a device array
// owned by the library, for callers that cannot allocate device memory.
//
// The array `scratch` is a file-scope __device__ array: every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  In host code the name `scratch` is only a host-side stand-in, so the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is passed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/fa.h"

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's `scratch`, looked up on first use.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_HIP;
  if (dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return FA_ERR_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return FA_OK;
}

}  // namespace

extern "C" int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                                 int causal, int n_splits, int dtype, void* stream) {
  // Bad arguments give a zero size here and fa_decode's own error below.
  const size_t need = fa_decode_workspace_size(B, H, Nq, Nk, d, n_splits);
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_for_current_device(&ws);
    if (rc != FA_OK) return rc;
  }
  // Every partial the merge reads is written by the scan of the same call,
  // so nothing in the array needs clearing.
  return fa_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, n_splits, dtype, ws, need,
                   stream);
}
