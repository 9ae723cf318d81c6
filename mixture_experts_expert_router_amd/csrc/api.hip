// C-ABI entry points: argument validation, workspace sizing and dispatch to
// the gfx950 kernels.  Declarations, contracts and the passages of the pages
// each operation follows are in include/moe_mi355x.h.
#include <atomic>

#include "../../include/moe_mi355x.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

// Compute units of the current device (cached per device).
int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return 256;
  int n = g_num_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess || n <= 0)
    n = 256;
  n = (n + 7) / 8 * 8;
  g_num_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

constexpr int64_t kMaxRows = (int64_t)1 << 31;

size_t tile_ws_bytes(int64_t n_local) {
  return moe::gemm_workspace_bytes(n_local);
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_E_ARG: return "invalid argument";
    case MOE_E_SHAPE: return "invalid or inconsistent sizes";
    case MOE_E_ALIGN: return "pointer not 16-byte aligned";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_UNSUPPORTED: return "unsupported combination";
    case MOE_E_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int moe_version(void) { return 100; }

int moe_route_topk(const void *x, const void *w_router, const float *bias,
                   float *logits, int64_t T, int64_t H, int64_t E, int64_t k,
                   int dtype, int32_t *topk_idx, float *topk_w,
                   hipStream_t stream) {
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return MOE_E_ARG;
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E)
    return MOE_E_SHAPE;
  if (T * E >= kMaxRows) return MOE_E_SHAPE;
  const bool gemm = x != nullptr || w_router != nullptr;
  if (gemm && (x == nullptr || w_router == nullptr)) return MOE_E_ARG;
  if (!gemm && bias != nullptr) return MOE_E_ARG;
  if (logits == nullptr || topk_idx == nullptr || topk_w == nullptr)
    return T == 0 ? MOE_OK : MOE_E_ARG;
  if (T == 0) return MOE_OK;
  if (gemm) {
    if (H < 1) return MOE_E_SHAPE;
    if (dtype == MOE_DT_BF16) {
      if (H % 64 != 0) return MOE_E_SHAPE;
      if (!aligned16(x) || !aligned16(w_router)) return MOE_E_ALIGN;
      hipError_t err = moe::launch_router_gemm_bf16(
          (const uint16_t *)x, (const uint16_t *)w_router, bias, logits, T,
          (int)H, (int)E, num_cus(), stream);
      if (err != hipSuccess) return MOE_E_HIP;
    } else {
      hipError_t err = moe::launch_router_gemm_f32(
          (const float *)x, (const float *)w_router, bias, logits, T, H, E,
          stream);
      if (err != hipSuccess) return MOE_E_HIP;
    }
  }
  return status_of(moe::launch_topk(logits, T, (int)E, (int)k, topk_idx,
                                    topk_w, stream));
}

size_t moe_permute_workspace_bytes(int64_t T, int64_t k, int64_t n_local) {
  if (T < 0 || k < 1 || n_local < 1) return 0;
  return moe::permute_workspace_bytes(T, k, n_local);
}

int moe_permute(const int32_t *topk_idx, const float *topk_w, const void *x,
                int64_t T, int64_t k, int64_t H, int dtype, int64_t e_begin,
                int64_t n_local, void *x_perm, float *s_perm,
                int32_t *row_src, int32_t *inv, int32_t *counts,
                int32_t *offsets, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return MOE_E_ARG;
  if (T < 0 || k < 1 || k > 32 || n_local < 1 || n_local > 4096 ||
      e_begin < 0 || e_begin > INT32_MAX - n_local)
    return MOE_E_SHAPE;
  if (T * k >= kMaxRows) return MOE_E_SHAPE;
  if (counts == nullptr || offsets == nullptr) return MOE_E_ARG;
  if (T > 0 && (topk_idx == nullptr || row_src == nullptr || inv == nullptr))
    return MOE_E_ARG;
  int64_t row_bytes = 0;
  if (x != nullptr) {
    if (x_perm == nullptr) return MOE_E_ARG;
    const int64_t esz = dtype == MOE_DT_BF16 ? 2 : 4;
    if (H < 1 || (H * esz) % 16 != 0) return MOE_E_SHAPE;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_E_ALIGN;
    row_bytes = H * esz;
  }
  const size_t need = moe::permute_workspace_bytes(T, k, n_local);
  if (workspace == nullptr || workspace_bytes < need) return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  if (T == 0) {
    // nothing routed: zero counts and offsets on the device
    if (hipMemsetAsync(counts, 0, (size_t)n_local * 4, stream) != hipSuccess ||
        hipMemsetAsync(offsets, 0, (size_t)(n_local + 1) * 4, stream) !=
            hipSuccess)
      return MOE_E_HIP;
    return MOE_OK;
  }
  return status_of(moe::launch_permute(
      topk_idx, topk_w, x, T, k, row_bytes, e_begin, n_local, x_perm, s_perm,
      row_src, inv, counts, offsets, workspace, num_cus(), stream));
}

size_t moe_grouped_ffn_workspace_bytes(int64_t R_cap, int64_t n_local,
                                       int64_t H, int64_t I, int dtype) {
  (void)R_cap; (void)H; (void)I; (void)dtype;
  if (n_local < 1) return 0;
  return tile_ws_bytes(n_local);
}

namespace {

int check_ffn(const int32_t *offsets, int64_t n_local, int64_t R_cap,
              int64_t H, int64_t I, int dtype, void *workspace,
              size_t workspace_bytes) {
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return MOE_E_ARG;
  if (n_local < 1 || n_local > 4096 || R_cap < 0 || R_cap >= kMaxRows ||
      H < 1 || I < 1)
    return MOE_E_SHAPE;
  if (dtype == MOE_DT_BF16) {
    if (H % 64 != 0 || I % 64 != 0) return MOE_E_SHAPE;
    if (H * I >= kMaxRows * 2) return MOE_E_SHAPE;
  } else if (H % 4 != 0 || I % 4 != 0) {
    return MOE_E_SHAPE;
  }
  if (offsets == nullptr) return MOE_E_ARG;
  if (workspace == nullptr || workspace_bytes < tile_ws_bytes(n_local))
    return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  return MOE_OK;
}

}  // namespace

int moe_grouped_gate_up(const void *x_perm, const int32_t *offsets,
                        const float *s_perm, int64_t n_local, int64_t R_cap,
                        int64_t H, int64_t I, const void *w_gate,
                        const void *w_up, int dtype, void *a, void *workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int st = check_ffn(offsets, n_local, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (R_cap == 0) return MOE_OK;
  if (!x_perm || !w_gate || !w_up || !a) return MOE_E_ARG;
  if (!aligned16(x_perm) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(a))
    return MOE_E_ALIGN;
  hipError_t err;
  if (dtype == MOE_DT_BF16)
    err = moe::launch_gate_up_bf16(
        (const uint16_t *)x_perm, offsets, s_perm, (int)n_local, R_cap,
        (int)H, (int)I, (const uint16_t *)w_gate, (const uint16_t *)w_up,
        (uint16_t *)a, (int32_t *)workspace, num_cus(), stream);
  else
    err = moe::launch_gate_up_f32((const float *)x_perm, offsets, s_perm,
                                  (int)n_local, R_cap, H, I,
                                  (const float *)w_gate, (const float *)w_up,
                                  (float *)a, stream);
  return status_of(err);
}

int moe_grouped_down(const void *a, const int32_t *offsets, int64_t n_local,
                     int64_t R_cap, int64_t H, int64_t I, const void *w_down,
                     int dtype, void *y, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  int st = check_ffn(offsets, n_local, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (R_cap == 0) return MOE_OK;
  if (!a || !w_down || !y) return MOE_E_ARG;
  if (!aligned16(a) || !aligned16(w_down) || !aligned16(y))
    return MOE_E_ALIGN;
  hipError_t err;
  if (dtype == MOE_DT_BF16)
    err = moe::launch_down_bf16((const uint16_t *)a, offsets, (int)n_local,
                                R_cap, (int)H, (int)I,
                                (const uint16_t *)w_down, (uint16_t *)y,
                                (int32_t *)workspace, num_cus(), stream);
  else
    err = moe::launch_down_f32((const float *)a, offsets, (int)n_local, R_cap,
                               H, I, (const float *)w_down, (float *)y,
                               stream);
  return status_of(err);
}

int moe_grouped_ffn(const void *x_perm, const int32_t *offsets,
                    const float *s_perm, int64_t n_local, int64_t R_cap,
                    int64_t H, int64_t I, const void *w_gate,
                    const void *w_up, const void *w_down, int dtype, void *a,
                    void *y, void *workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  int st = check_ffn(offsets, n_local, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (R_cap == 0) return MOE_OK;
  if (!w_down || !y) return MOE_E_ARG;
  if (!aligned16(w_down) || !aligned16(y)) return MOE_E_ALIGN;
  st = moe_grouped_gate_up(x_perm, offsets, s_perm, n_local, R_cap, H, I,
                           w_gate, w_up, dtype, a, workspace, workspace_bytes,
                           stream);
  if (st != MOE_OK) return st;
  return moe_grouped_down(a, offsets, n_local, R_cap, H, I, w_down, dtype, y,
                          workspace, workspace_bytes, stream);
}

int moe_unpermute_combine(const void *y, const int32_t *inv,
                          const float *topk_w, int64_t T, int64_t k,
                          int64_t H, int dtype, void *out,
                          hipStream_t stream) {
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return MOE_E_ARG;
  if (T < 0 || k < 1 || k > 32 || H < 1) return MOE_E_SHAPE;
  if (H % (dtype == MOE_DT_BF16 ? 8 : 4) != 0) return MOE_E_SHAPE;
  if (T * k >= kMaxRows) return MOE_E_SHAPE;
  if (T == 0) return MOE_OK;
  if (!y || !inv || !out) return MOE_E_ARG;
  if (!aligned16(y) || !aligned16(out)) return MOE_E_ALIGN;
  return status_of(moe::launch_combine(y, inv, topk_w, T, (int)k, H, dtype,
                                       out, num_cus(), stream));
}

int moe_debug_sync(hipStream_t stream) {
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_E_HIP;
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // extern "C"
