// moe_permute_noalloc: moe_permute for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation).  The permute's scratch (the error header, the
// per-chunk expert histogram and the chunk flags) lives in a file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy of the array, at its own address, until the process
// ends; its address is looked up once per device and every later call uses
// that address (the array's name in host code is only a host-side handle).
#include <mutex>

#include "../../include/moe_mi355x.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDev = 64;
std::mutex g_mu;
void *g_scratch[kMaxDev];  // device address of `scratch`, per device

// Device address of this device's `scratch`, or null on failure.
void *scratch_ptr(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess)
      return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int moe_permute_noalloc(const int32_t *topk_idx,
                                   const float *topk_w, const void *x,
                                   int64_t T, int64_t k, int64_t H, int dtype,
                                   int64_t E, int64_t e_begin,
                                   int64_t n_local, void *x_perm,
                                   float *s_perm, int32_t *row_src,
                                   int32_t *inv, int32_t *counts,
                                   int32_t *offsets, hipStream_t stream) {
  // Same validation as moe_permute (it runs again inside that call); the
  // size check against the scratch comes first so that an oversized call
  // never touches the device.
  if (T >= 0 && k >= 1 && n_local >= 1 && T * k < ((int64_t)1 << 31) &&
      n_local <= 4096 &&
      moe_permute_workspace_bytes(T, k, n_local) > kScratchBytes)
    return MOE_E_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
    return MOE_E_HIP;
  void *ws = scratch_ptr(dev);
  if (ws == nullptr) return MOE_E_HIP;
  return moe_permute(topk_idx, topk_w, x, T, k, H, dtype, E, e_begin,
                     n_local, x_perm, s_perm, row_src, inv, counts, offsets,
                     ws, kScratchBytes, stream);
}
