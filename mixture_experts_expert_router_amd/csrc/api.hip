// C-ABI entry points: argument validation, workspace sizing and dispatch to
// the gfx950 kernels.  Declarations, contracts and the passages of the pages
// each operation follows are in include/moe_mi355x.h.
#include <algorithm>
#include <atomic>
#include <initializer_list>

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

bool all_aligned16(std::initializer_list<const void *> ps) {
  for (const void *q : ps)
    if (!aligned16(q)) return false;
  return true;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

constexpr int64_t kMaxRows = (int64_t)1 << 31;

// One workspace size serves every FFN entry point (grouped, per-expert
// loop, fused).
size_t tile_ws_bytes(int64_t n_local, int64_t R_cap, int64_t H, int64_t I) {
  return std::max(moe::gemm_workspace_bytes(n_local, R_cap, H, I),
                  moe::ffn_fused_workspace_bytes(n_local, R_cap, H, I));
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
    case MOE_E_SCRATCH:
      return "needs more scratch than the no-allocation variant holds";
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
                int64_t T, int64_t k, int64_t H, int dtype, int64_t E,
                int64_t e_begin, int64_t n_local, void *x_perm, float *s_perm,
                int32_t *row_src, int32_t *inv, int32_t *counts,
                int32_t *offsets, void *workspace, size_t workspace_bytes,
                hipStream_t stream) {
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return MOE_E_ARG;
  if (T < 0 || k < 1 || k > 32 || n_local < 1 || n_local > 4096 ||
      E < 1 || E > INT32_MAX || e_begin < 0 || e_begin > E - n_local)
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
    return status_of(
        moe::launch_permute_empty(counts, offsets, n_local, workspace, stream));
  }
  return status_of(moe::launch_permute(
      topk_idx, topk_w, x, T, k, row_bytes, E, e_begin, n_local, x_perm, s_perm,
      row_src, inv, counts, offsets, workspace, num_cus(), stream));
}

size_t moe_grouped_ffn_workspace_bytes(int64_t R_cap, int64_t n_local,
                                       int64_t H, int64_t I, int dtype) {
  (void)dtype;
  if (n_local < 1 || R_cap < 0 || H < 1 || I < 1) return 0;
  return tile_ws_bytes(n_local, R_cap, H, I);
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
  if (workspace == nullptr ||
      workspace_bytes < tile_ws_bytes(n_local, R_cap, H, I))
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
  else {
    err = moe::launch_check_offsets(offsets, (int)n_local, R_cap,
                                    (int32_t *)workspace, stream);
    if (err == hipSuccess)
      err = moe::launch_gate_up_f32((const float *)x_perm, offsets, s_perm,
                                    (int)n_local, R_cap, H, I,
                                    (const float *)w_gate, (const float *)w_up,
                                    (float *)a, stream);
  }
  return status_of(err);
}

int moe_grouped_gate_up_gather(const void *x, const int32_t *row_src,
                               int64_t T, int64_t k, const int32_t *offsets,
                               const float *s_perm, int64_t n_local,
                               int64_t R_cap, int64_t H, int64_t I,
                               const void *w_gate, const void *w_up, int dtype,
                               void *a, void *workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  int st = check_ffn(offsets, n_local, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (dtype != MOE_DT_BF16) return MOE_E_UNSUPPORTED;
  if (T < 1 || k < 1 || k > 32 || T * k >= kMaxRows || R_cap > T * k)
    return MOE_E_SHAPE;
  if (R_cap == 0) return MOE_OK;
  if (!x || !row_src || !w_gate || !w_up || !a) return MOE_E_ARG;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(a))
    return MOE_E_ALIGN;
  return status_of(moe::launch_gate_up_bf16(
      (const uint16_t *)x, offsets, s_perm, (int)n_local, R_cap, (int)H,
      (int)I, (const uint16_t *)w_gate, (const uint16_t *)w_up, (uint16_t *)a,
      (int32_t *)workspace, num_cus(), stream, row_src, (int)k, T));
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
  else {
    err = moe::launch_check_offsets(offsets, (int)n_local, R_cap,
                                    (int32_t *)workspace, stream);
    if (err == hipSuccess)
      err = moe::launch_down_f32((const float *)a, offsets, (int)n_local,
                                 R_cap, H, I, (const float *)w_down, (float *)y,
                                 stream);
  }
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
  if (dtype == MOE_DT_BF16) {
    // one plan kernel for both GEMMs
    if (!x_perm || !w_gate || !w_up || !a) return MOE_E_ARG;
    if (!all_aligned16({x_perm, w_gate, w_up, a})) return MOE_E_ALIGN;
    return status_of(moe::launch_ffn_grouped_bf16(
        (const uint16_t *)x_perm, nullptr, 1, 1, offsets, s_perm,
        (int)n_local, R_cap, (int)H, (int)I, (const uint16_t *)w_gate,
        (const uint16_t *)w_up, (const uint16_t *)w_down, (uint16_t *)a,
        (uint16_t *)y, (int32_t *)workspace, num_cus(), stream));
  }
  st = moe_grouped_gate_up(x_perm, offsets, s_perm, n_local, R_cap, H, I,
                           w_gate, w_up, dtype, a, workspace, workspace_bytes,
                           stream);
  if (st != MOE_OK) return st;
  return moe_grouped_down(a, offsets, n_local, R_cap, H, I, w_down, dtype, y,
                          workspace, workspace_bytes, stream);
}

int moe_grouped_ffn_gather(const void *x, const int32_t *row_src, int64_t T,
                           int64_t k, const int32_t *offsets,
                           const float *s_perm, int64_t n_local,
                           int64_t R_cap, int64_t H, int64_t I,
                           const void *w_gate, const void *w_up,
                           const void *w_down, int dtype, void *a, void *y,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  int st = check_ffn(offsets, n_local, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (dtype != MOE_DT_BF16) return MOE_E_UNSUPPORTED;
  if (T < 1 || k < 1 || k > 32 || T * k >= kMaxRows || R_cap > T * k)
    return MOE_E_SHAPE;
  if (R_cap == 0) return MOE_OK;
  if (!x || !row_src || !w_gate || !w_up || !w_down || !a || !y)
    return MOE_E_ARG;
  if (!all_aligned16({x, w_gate, w_up, w_down, a, y})) return MOE_E_ALIGN;
  return status_of(moe::launch_ffn_grouped_bf16(
      (const uint16_t *)x, row_src, (int)k, T, offsets, s_perm, (int)n_local,
      R_cap, (int)H, (int)I, (const uint16_t *)w_gate, (const uint16_t *)w_up,
      (const uint16_t *)w_down, (uint16_t *)a, (uint16_t *)y,
      (int32_t *)workspace, num_cus(), stream));
}

int moe_grouped_ffn_fused(const void *x, const int32_t *row_src, int64_t T,
                          int64_t k, const int32_t *offsets,
                          const float *s_perm, int64_t n_local, int64_t R_cap,
                          int64_t H, int64_t I, const void *w_gate,
                          const void *w_up, const void *w_down, int dtype,
                          void *a, void *y, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  int st = check_ffn(offsets, n_local, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (dtype != MOE_DT_BF16) return MOE_E_UNSUPPORTED;
  if (row_src) {
    if (T < 1 || k < 1 || k > 32 || T * k >= kMaxRows || R_cap > T * k)
      return MOE_E_SHAPE;
  }
  if (R_cap == 0) return MOE_OK;
  if (!x || !w_gate || !w_up || !w_down || !a || !y) return MOE_E_ARG;
  if (!all_aligned16({x, w_gate, w_up, w_down, a, y})) return MOE_E_ALIGN;
  return status_of(moe::launch_ffn_fused_bf16(
      (const uint16_t *)x, row_src, (int)k, T, offsets, s_perm, (int)n_local,
      R_cap, (int)H, (int)I, (const uint16_t *)w_gate, (const uint16_t *)w_up,
      (const uint16_t *)w_down, (uint16_t *)a, (uint16_t *)y,
      (int32_t *)workspace, num_cus(), stream));
}

int moe_grouped_ffn_loop(const void *x_perm, const int32_t *offsets,
                         const int32_t *host_counts, const float *s_perm,
                         int64_t n_local, int64_t R_cap, int64_t H, int64_t I,
                         const void *w_gate, const void *w_up,
                         const void *w_down, int dtype, void *a, void *y,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  int st = check_ffn(offsets, n_local, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (dtype != MOE_DT_BF16) return MOE_E_UNSUPPORTED;
  if (host_counts == nullptr) return MOE_E_ARG;
  int64_t total = 0;
  for (int64_t e = 0; e < n_local; ++e) {
    if (host_counts[e] < 0) return MOE_E_SHAPE;
    total += host_counts[e];
  }
  if (total > R_cap) return MOE_E_SHAPE;
  if (R_cap == 0 || total == 0) return MOE_OK;
  if (!x_perm || !w_gate || !w_up || !w_down || !a || !y) return MOE_E_ARG;
  if (!all_aligned16({x_perm, w_gate, w_up, w_down, a, y})) return MOE_E_ALIGN;
  return status_of(moe::launch_ffn_loop_bf16(
      (const uint16_t *)x_perm, offsets, host_counts, s_perm, (int)n_local,
      R_cap, (int)H, (int)I, (const uint16_t *)w_gate, (const uint16_t *)w_up,
      (const uint16_t *)w_down, (uint16_t *)a, (uint16_t *)y,
      (int32_t *)workspace, num_cus(), stream));
}

int moe_eplb_plan(const int32_t *counts, int64_t E, int64_t n_slots,
                  int64_t n_ranks, int32_t *rep, int32_t *rep_first,
                  int32_t *rep_slot, int32_t *slot_expert, int32_t *slot_copy,
                  hipStream_t stream) {
  if (E < 1 || E > 1024 || n_slots < E || n_slots > 4096 || n_ranks < 1 ||
      n_ranks > 1024 || n_slots % n_ranks != 0)
    return MOE_E_SHAPE;
  if (!counts || !rep || !rep_first || !rep_slot || !slot_expert || !slot_copy)
    return MOE_E_ARG;
  return status_of(moe::launch_eplb_plan(counts, (int)E, (int)n_slots,
                                         (int)n_ranks, rep, rep_first, rep_slot,
                                         slot_expert, slot_copy, stream));
}

size_t moe_permute_replicated_workspace_bytes(int64_t T, int64_t k, int64_t E,
                                              int64_t n_slots) {
  if (T < 0 || k < 1 || E < 1 || n_slots < 1) return 0;
  return moe::permute_replicated_workspace_bytes(T, k, E, n_slots);
}

int moe_permute_replicated(const int32_t *topk_idx, const float *topk_w,
                           const void *x, int64_t T, int64_t k, int64_t H,
                           int dtype, int64_t E, int64_t S,
                           const int32_t *rep_first, const int32_t *rep_slot,
                           const int32_t *slot_expert,
                           const int32_t *slot_copy, int64_t s_begin,
                           int64_t n_slots, void *x_perm, float *s_perm,
                           int32_t *row_src, int32_t *inv, int32_t *counts,
                           int32_t *offsets, void *workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (dtype != MOE_DT_F32 && dtype != MOE_DT_BF16) return MOE_E_ARG;
  if (T < 1 || k < 1 || k > 32 || E < 1 || E > 4096 || S < E || S > 4096 ||
      n_slots < 1 || s_begin < 0 || s_begin > S - n_slots)
    return MOE_E_SHAPE;
  if (T * k >= kMaxRows) return MOE_E_SHAPE;
  if (!topk_idx || !rep_first || !rep_slot || !slot_expert || !slot_copy ||
      !row_src || !inv || !counts || !offsets)
    return MOE_E_ARG;
  int64_t row_bytes = 0;
  if (x != nullptr) {
    if (x_perm == nullptr) return MOE_E_ARG;
    const int64_t esz = dtype == MOE_DT_BF16 ? 2 : 4;
    if (H < 1 || (H * esz) % 16 != 0) return MOE_E_SHAPE;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_E_ALIGN;
    row_bytes = H * esz;
  }
  if (topk_w && !s_perm) return MOE_E_ARG;
  const size_t need = moe::permute_replicated_workspace_bytes(T, k, E, n_slots);
  if (workspace == nullptr || workspace_bytes < need) return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  return status_of(moe::launch_permute_replicated(
      topk_idx, topk_w, x, T, k, row_bytes, E, rep_first, rep_slot,
      slot_expert, slot_copy, s_begin, n_slots, x_perm, s_perm, row_src, inv,
      counts, offsets, workspace, num_cus(), stream));
}

int moe_grouped_ffn_slots(const void *x_perm, const int32_t *offsets,
                          const float *s_perm, int64_t n_slots,
                          const int32_t *slot_expert, int64_t n_experts,
                          int64_t R_cap, int64_t H, int64_t I,
                          const void *w_gate, const void *w_up,
                          const void *w_down, int dtype, void *a, void *y,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  int st = check_ffn(offsets, n_slots, R_cap, H, I, dtype, workspace,
                     workspace_bytes);
  if (st != MOE_OK) return st;
  if (dtype != MOE_DT_BF16) return MOE_E_UNSUPPORTED;
  if (n_experts < 1 || n_experts > (1 << 20)) return MOE_E_SHAPE;
  if (R_cap == 0) return MOE_OK;
  if (!slot_expert || !x_perm || !w_gate || !w_up || !w_down || !a || !y)
    return MOE_E_ARG;
  if (!all_aligned16({x_perm, w_gate, w_up, w_down, a, y})) return MOE_E_ALIGN;
  hipError_t err = moe::launch_gate_up_bf16(
      (const uint16_t *)x_perm, offsets, s_perm, (int)n_slots, R_cap, (int)H,
      (int)I, (const uint16_t *)w_gate, (const uint16_t *)w_up, (uint16_t *)a,
      (int32_t *)workspace, num_cus(), stream, nullptr, 1, 1, slot_expert,
      (int)n_experts);
  if (err != hipSuccess) return MOE_E_HIP;
  return status_of(moe::launch_down_bf16(
      (const uint16_t *)a, offsets, (int)n_slots, R_cap, (int)H, (int)I,
      (const uint16_t *)w_down, (uint16_t *)y, (int32_t *)workspace, num_cus(),
      stream, slot_expert, (int)n_experts));
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

int moe_read_device_error(const void *workspace, hipStream_t stream,
                          int32_t *host_code) {
  if (workspace == nullptr || host_code == nullptr) return MOE_E_ARG;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof v, hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MOE_E_HIP;
  *host_code = v;
  return MOE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- MXFP8
namespace {

// Bump allocator over a caller workspace (256-byte aligned pieces).
struct Carve {
  char *base;
  size_t used = 0;
  explicit Carve(void *b) : base((char *)b) {}
  template <typename T>
  T *take(size_t count) {
    T *p = base ? (T *)(base + used) : nullptr;
    used += (count * sizeof(T) + 255) / 256 * 256;
    return p;
  }
};

bool mx_shape_ok(int64_t n_local, int64_t R_cap, int64_t H, int64_t I) {
  return n_local >= 1 && n_local <= 4096 && R_cap >= 0 && R_cap < kMaxRows &&
         H >= 512 && I >= 512 && H % 512 == 0 && I % 512 == 0 &&
         (int64_t)n_local * I < kMaxRows && (int64_t)n_local * H < kMaxRows;
}

// Row capacity of transposed (column-quantised) expert segments padded
// to 512 rows each (also enough for padding to 256).
int64_t mx_kpad_cap(int64_t R_cap, int64_t n_local) {
  return (R_cap + 511 * n_local + 511) / 512 * 512;
}

// Workspace layouts.  Sizes depend only on the arguments, so the same
// carving gives the byte count (base == null) and the pointers.
// Every workspace begins with the error header (device error word first).
int32_t *carve_err(Carve &c) {
  return c.take<int32_t>(moe::kErrHeaderBytes / 4);
}

struct LinWs {                     // grouped linear: tile plan + MX(x)
  int32_t *err, *tiles;
  uint8_t *xq, *xs;
};
LinWs carve_lin(Carve &c, int64_t R_cap, int64_t n_local, int64_t K) {
  LinWs w;
  w.err = carve_err(c);
  w.tiles = c.take<int32_t>(n_local + 1);
  w.xq = c.take<uint8_t>((size_t)R_cap * K);
  w.xs = c.take<uint8_t>((size_t)R_cap * (K / 32));
  return w;
}

struct DownBwdWs {                 // backward of the down projection
  int32_t *err, *tiles, *kpad;
  uint8_t *dyq, *dys;
  float *ds_part;
  uint8_t *dyT, *dyTs, *aT, *aTs;
  int64_t kcap;
};
DownBwdWs carve_down_bwd(Carve &c, int64_t R_cap, int64_t n_local, int64_t H,
                         int64_t I) {
  DownBwdWs w;
  w.kcap = mx_kpad_cap(R_cap, n_local);
  w.err = carve_err(c);
  w.tiles = c.take<int32_t>(n_local + 1);
  w.kpad = c.take<int32_t>(n_local + 1);
  w.dyq = c.take<uint8_t>((size_t)R_cap * H);
  w.dys = c.take<uint8_t>((size_t)R_cap * (H / 32));
  w.ds_part = c.take<float>((size_t)R_cap * moe::mx_ds_parts(I));
  w.dyT = c.take<uint8_t>((size_t)H * w.kcap);
  w.dyTs = c.take<uint8_t>((size_t)H * (w.kcap / 32));
  w.aT = c.take<uint8_t>((size_t)I * w.kcap);
  w.aTs = c.take<uint8_t>((size_t)I * (w.kcap / 32));
  return w;
}

struct GateUpBwdWs {               // backward of the gate/up projection
  int32_t *err, *tiles, *kpad;
  uint8_t *dguq, *dgus;
  uint8_t *xT, *xTs, *dgT, *dgTs, *duT, *duTs;
  int64_t kcap;
};
// own_dgu == false: the MX copies of [dg | du] come from DguCodes instead.
GateUpBwdWs carve_gate_up_bwd(Carve &c, int64_t R_cap, int64_t n_local,
                              int64_t H, int64_t I, bool own_dgu = true) {
  GateUpBwdWs w{};
  w.kcap = mx_kpad_cap(R_cap, n_local);
  w.err = carve_err(c);
  w.tiles = c.take<int32_t>(n_local + 1);
  w.kpad = c.take<int32_t>(n_local + 1);
  if (own_dgu) {
    w.dguq = c.take<uint8_t>((size_t)R_cap * 2 * I);
    w.dgus = c.take<uint8_t>((size_t)R_cap * (2 * I / 32));
  }
  w.xT = c.take<uint8_t>((size_t)H * w.kcap);
  w.xTs = c.take<uint8_t>((size_t)H * (w.kcap / 32));
  if (own_dgu) {
    w.dgT = c.take<uint8_t>((size_t)I * w.kcap);
    w.dgTs = c.take<uint8_t>((size_t)I * (w.kcap / 32));
    w.duT = c.take<uint8_t>((size_t)I * w.kcap);
    w.duTs = c.take<uint8_t>((size_t)I * (w.kcap / 32));
  }
  return w;
}

// The fused backward's MX copies of [dg | du], written by the SwiGLU-backward
// epilogue: row-wise along 2I (for dX) and column-wise per expert segment,
// segments padded to 256 rows at tpad (for dW_g, dW_u).
struct DguCodes {
  int32_t *tpad;
  uint8_t *q, *qs;                 // [R_cap, 2I], [R_cap, 2I/32]
  uint8_t *gT, *gTs, *uT, *uTs;    // [I, kcap], [I, kcap/32]
  int64_t kcap;
};
DguCodes carve_dgu_codes(Carve &c, int64_t R_cap, int64_t n_local, int64_t I) {
  DguCodes d;
  d.kcap = mx_kpad_cap(R_cap, n_local);
  d.tpad = c.take<int32_t>(n_local + 1);
  d.q = c.take<uint8_t>((size_t)R_cap * 2 * I);
  d.qs = c.take<uint8_t>((size_t)R_cap * (2 * I / 32));
  d.gT = c.take<uint8_t>((size_t)I * d.kcap);
  d.gTs = c.take<uint8_t>((size_t)I * (d.kcap / 32));
  d.uT = c.take<uint8_t>((size_t)I * d.kcap);
  d.uTs = c.take<uint8_t>((size_t)I * (d.kcap / 32));
  return d;
}

size_t fwd_bytes(int64_t R_cap, int64_t n_local, int64_t I) {
  Carve c(nullptr);
  carve_lin(c, R_cap, n_local, I);
  return c.used;
}
size_t lin_bytes(int64_t R_cap, int64_t n_local, int64_t K) {
  Carve c(nullptr);
  carve_lin(c, R_cap, n_local, K);
  return c.used;
}
size_t down_bwd_bytes(int64_t R_cap, int64_t n_local, int64_t H, int64_t I) {
  Carve c(nullptr);
  carve_down_bwd(c, R_cap, n_local, H, I);
  return c.used;
}
size_t gate_up_bwd_bytes(int64_t R_cap, int64_t n_local, int64_t H,
                         int64_t I) {
  Carve c(nullptr);
  carve_gate_up_bwd(c, R_cap, n_local, H, I);
  return c.used;
}
// Fused backward: dgu (bf16 and MX), then one region that both halves use
// in turn.
size_t bwd_bytes(int64_t R_cap, int64_t n_local, int64_t H, int64_t I) {
  Carve c(nullptr);
  carve_err(c);
  carve_dgu_codes(c, R_cap, n_local, I);
  Carve g(nullptr);
  carve_gate_up_bwd(g, R_cap, n_local, H, I, /*own_dgu=*/false);
  return c.used + std::max(down_bwd_bytes(R_cap, n_local, H, I), g.used);
}

// y = MX(x) . MX(W_e)^T per row segment; the quantisation of x stops at the
// device row count offsets[G].
// quantised: ws.xq / ws.xs already hold MX(x) (written by the producing
// GEMM's epilogue), and x itself is not read.
hipError_t run_linear(const void *x, const int32_t *offsets, int64_t n_local,
                      int64_t R_cap, int64_t K, int64_t N, const uint8_t *w,
                      const uint8_t *wsc, void *y, const LinWs &ws, int cus,
                      hipStream_t stream, bool quantised = false) {
  if (!quantised) {
    hipError_t err = moe::launch_mx_quant_rows(
        (const uint16_t *)x, R_cap, K, K, ws.xq, K, ws.xs, K / 32,
        offsets + n_local, stream);
    if (err != hipSuccess) return err;
  }
  moe::MxGemmDesc e{};
  e.A = ws.xq; e.As = ws.xs; e.lda = K; e.ldas = K / 32;
  e.B0 = w; e.B0s = wsc; e.ldb = K; e.ldbs = K / 32;
  e.b_stride = N * K; e.bs_stride = N * K / 32;
  e.offsets = offsets; e.tile_ws = ws.tiles; e.err = ws.err; e.G = (int)n_local;
  e.N = (int)N; e.K = (int)K; e.R_cap = R_cap;
  e.C = y; e.ldc = N;
  return moe::launch_mx_rowseg(e, moe::MXE_BF16, cus, stream);
}

// The backward of the down projection.  dgu (bf16 [dg | du], may be null)
// is written for the unfused stage API; with `codes` the epilogue writes
// [dg | du] as MX codes instead (row-wise, and column-wise per segment).
// Either way a = s SiLU(g) u is recomputed in fp32 from the saved fp32 g, u
// in the same epilogue, which writes its column-wise codes for dW_d.
hipError_t run_down_bwd(const void *dy, const float *gu,
                        const int32_t *offsets, const float *s_perm,
                        int64_t n_local, int64_t R_cap, int64_t H, int64_t I,
                        const uint8_t *wdt, const uint8_t *wdts, void *dgu,
                        float *ds, void *dw_down, const DownBwdWs &w,
                        int32_t *errw, int cus, hipStream_t stream, int gf,
                        const DguCodes *codes = nullptr) {
  const int G = (int)n_local;
  const int64_t kc = w.kcap;
  // padded segment starts of every column-wise copy (256 rows: one tile)
  int32_t *tpad = codes ? codes->tpad : w.kpad;
  hipError_t err;
#define MX_TRY(x) do { err = (x); if (err != hipSuccess) return err; } while (0)
  // dY along H (row-wise)
  MX_TRY(moe::launch_mx_quant_rows((const uint16_t *)dy, R_cap, H, H, w.dyq, H,
                                   w.dys, H / 32, offsets + G, stream, gf));
  MX_TRY(moe::launch_mx_pad_offsets(offsets, G, R_cap, 256, tpad, stream));
  // da = dY W_d (K = H); SwiGLU backward in the epilogue -> dg, du, ds, and
  // the column-wise codes of a
  {
    moe::MxGemmDesc d{};
    d.A = w.dyq; d.As = w.dys; d.lda = H; d.ldas = H / 32;
    d.B0 = wdt; d.B0s = wdts; d.ldb = n_local * H; d.ldbs = n_local * H / 32;
    d.b_stride = H; d.bs_stride = H / 32;
    d.offsets = offsets; d.tile_ws = w.tiles; d.err = errw; d.G = G;
    d.N = (int)I; d.K = (int)H; d.R_cap = R_cap;
    d.row_scale = s_perm; d.gu = (float *)gu; d.ldgu = 2 * I;
    d.dgu = (uint16_t *)dgu; d.ds_part = w.ds_part; d.ds = ds;
    d.t2 = w.aT; d.t2s = w.aTs; d.ldt = kc; d.ldts = kc / 32; d.tpad = tpad;
    d.fa = gf;
    if (codes) {
      // [dg | du] quantised by the epilogue: along 2I for the dX GEMM, and
      // down each expert segment (padded to 256 rows) for dW_g, dW_u
      d.q = codes->q; d.qs = codes->qs; d.ldq = 2 * I; d.ldqs = 2 * I / 32;
      d.t0 = codes->gT; d.t0s = codes->gTs; d.t1 = codes->uT; d.t1s = codes->uTs;
    }
    MX_TRY(moe::launch_mx_rowseg(d, moe::MXE_SWIGLU_BWD, cus, stream));
  }
  // dW_d[e] [H, I] = dY_e^T a_e: blocks of 32 rows inside each expert's
  // segment, segments zero-padded to 256 rows like the codes of a
  MX_TRY(moe::launch_mx_quant_cols((const uint16_t *)dy, R_cap, H, H, offsets,
                                   G, 256, tpad, w.dyT, kc, w.dyTs, kc / 32,
                                   cus, stream, gf));
  moe::MxGemmDesc d{};
  d.kseg = tpad; d.G = G; d.fa = gf;
  d.lda = kc; d.ldas = kc / 32; d.ldb = kc; d.ldbs = kc / 32;
  d.A = w.dyT; d.As = w.dyTs; d.B0 = w.aT; d.B0s = w.aTs;
  d.M = (int)H; d.N = (int)I; d.C = dw_down; d.ldc = I; d.c_stride = H * I;
  return moe::launch_mx_kseg(d, cus, stream);
}

hipError_t run_gate_up_bwd(const void *dgu, const void *x_perm,
                           const int32_t *offsets, int64_t n_local,
                           int64_t R_cap, int64_t H, int64_t I,
                           const uint8_t *wgt, const uint8_t *wgts,
                           const uint8_t *wut, const uint8_t *wuts, void *dx,
                           void *dw_gate, void *dw_up, const GateUpBwdWs &w,
                           int32_t *errw, int cus, hipStream_t stream, int gf,
                           const DguCodes *codes = nullptr) {
  const int G = (int)n_local;
  hipError_t err;
  // [dg | du] along I (row-wise; blocks never straddle the two halves),
  // unless the producing epilogue already wrote it
  const uint8_t *dguq = codes ? codes->q : w.dguq;
  const uint8_t *dgus = codes ? codes->qs : w.dgus;
  if (!codes)
    MX_TRY(moe::launch_mx_quant_rows((const uint16_t *)dgu, R_cap, 2 * I, 2 * I,
                                     w.dguq, 2 * I, w.dgus, 2 * I / 32,
                                     offsets + G, stream, gf));
  // dX = dg W_g + du W_u: one GEMM with K = 2I, B switching at K = I
  {
    moe::MxGemmDesc d{};
    d.A = dguq; d.As = dgus; d.lda = 2 * I; d.ldas = 2 * I / 32;
    d.B0 = wgt; d.B0s = wgts; d.B1 = wut; d.B1s = wuts;
    d.ldb = n_local * I; d.ldbs = n_local * I / 32;
    d.b_stride = I; d.bs_stride = I / 32;
    d.offsets = offsets; d.tile_ws = w.tiles; d.err = errw; d.G = G;
    d.N = (int)H; d.K = (int)(2 * I); d.R_cap = R_cap; d.ksplit = (int)I;
    d.C = dx; d.ldc = H; d.fa = gf;
    MX_TRY(moe::launch_mx_rowseg(d, moe::MXE_BF16, cus, stream));
  }
  // Column-wise copies for the weight gradients: segments padded to 512
  // rows, or to 256 rows to match the epilogue's dg, du copies.
  const int64_t kc = w.kcap;
  const int align = codes ? 256 : 512;
  int32_t *kpad = codes ? codes->tpad : w.kpad;
  MX_TRY(moe::launch_mx_quant_cols((const uint16_t *)x_perm, R_cap, H, H,
                                   offsets, G, align, kpad, w.xT, kc, w.xTs,
                                   kc / 32, cus, stream));
  const uint8_t *dgT = codes ? codes->gT : w.dgT, *dgTs = codes ? codes->gTs : w.dgTs;
  const uint8_t *duT = codes ? codes->uT : w.duT, *duTs = codes ? codes->uTs : w.duTs;
  if (!codes) {
    const uint16_t *dg = (const uint16_t *)dgu;
    MX_TRY(moe::launch_mx_quant_cols(dg, R_cap, I, 2 * I, offsets, G, 512,
                                     w.kpad, w.dgT, kc, w.dgTs, kc / 32, cus,
                                     stream, gf));
    MX_TRY(moe::launch_mx_quant_cols(dg + I, R_cap, I, 2 * I, offsets, G, 512,
                                     w.kpad, w.duT, kc, w.duTs, kc / 32, cus,
                                     stream, gf));
  }
#undef MX_TRY
  // dW_g[e] [I, H] = dg_e^T x_e ; dW_u likewise with du
  moe::MxGemmDesc d{};
  d.kseg = kpad; d.G = G; d.fa = gf;
  d.lda = kc; d.ldas = kc / 32; d.ldb = kc; d.ldbs = kc / 32;
  d.A = dgT; d.As = dgTs; d.B0 = w.xT; d.B0s = w.xTs;
  d.M = (int)I; d.N = (int)H; d.C = dw_gate; d.ldc = H; d.c_stride = I * H;
  err = moe::launch_mx_kseg(d, cus, stream);
  if (err != hipSuccess) return err;
  d.A = duT; d.As = duTs; d.C = dw_up;
  return moe::launch_mx_kseg(d, cus, stream);
}

bool grad_format_ok(int f) { return f == MOE_MX_E4M3 || f == MOE_MX_E5M2; }

bool all_aligned(std::initializer_list<const void *> ps) {
  for (const void *q : ps)
    if (!aligned16(q)) return false;
  return true;
}

}  // namespace

extern "C" {

int moe_mxfp8_quantize(const void *in, int64_t rows, int64_t cols,
                       int64_t ld_in, int axis, int format,
                       const int32_t *seg_offsets, int64_t n_seg,
                       int64_t align, uint8_t *codes, int64_t ld_codes,
                       uint8_t *scales, int64_t ld_scales,
                       int32_t *pad_offsets, hipStream_t stream) {
  if (axis != 0 && axis != 1) return MOE_E_ARG;
  if (format != MOE_MX_E4M3 && format != MOE_MX_E5M2) return MOE_E_ARG;
  if (rows < 0 || cols < 1 || cols % 32 != 0 || ld_in < cols) return MOE_E_SHAPE;
  if (rows >= kMaxRows || cols >= kMaxRows) return MOE_E_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!in || !codes || !scales) return MOE_E_ARG;
  if (!aligned16(codes)) return MOE_E_ALIGN;
  if (axis == 0) {
    if (ld_in % 8 != 0 || ld_codes < cols || ld_codes % 16 != 0 ||
        ld_scales < cols / 32)
      return MOE_E_SHAPE;
    if (!aligned16(in)) return MOE_E_ALIGN;
    return status_of(moe::launch_mx_quant_rows(
        (const uint16_t *)in, rows, cols, ld_in, codes, ld_codes, scales,
        ld_scales, nullptr, stream, format));
  }
  if (align != 32 && align != 512) return MOE_E_SHAPE;
  if (ld_codes % 16 != 0 || ld_in % 8 != 0) return MOE_E_SHAPE;
  if (!aligned16(in)) return MOE_E_ALIGN;
  if (seg_offsets) {
    if (n_seg < 1 || n_seg > 1 << 20 || pad_offsets == nullptr) return MOE_E_ARG;
    if (ld_codes < rows + (align - 1) * n_seg) return MOE_E_SHAPE;
  } else {
    if (ld_codes < (rows + align - 1) / align * align) return MOE_E_SHAPE;
  }
  if (ld_scales < ld_codes / 32) return MOE_E_SHAPE;
  return status_of(moe::launch_mx_quant_cols(
      (const uint16_t *)in, rows, cols, ld_in, seg_offsets, (int)n_seg,
      (int)align, pad_offsets, codes, ld_codes, scales, ld_scales, num_cus(),
      stream, format));
}

size_t moe_grouped_mlp_mxfp8_fwd_workspace_bytes(int64_t R_cap,
                                                 int64_t n_local, int64_t H,
                                                 int64_t I) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return 0;
  return fwd_bytes(R_cap, n_local, I);
}

int moe_grouped_mlp_mxfp8_fwd(const uint8_t *xq, const uint8_t *xs,
                              const int32_t *offsets, const float *s_perm,
                              int64_t n_local, int64_t R_cap, int64_t H,
                              int64_t I, const uint8_t *wg, const uint8_t *wgs,
                              const uint8_t *wu, const uint8_t *wus,
                              const uint8_t *wd, const uint8_t *wds, void *a,
                              float *gu, void *y, void *workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return MOE_E_SHAPE;
  if (R_cap == 0) return MOE_OK;
  if (!xq || !xs || !offsets || !wg || !wgs || !wu || !wus || !a)
    return MOE_E_ARG;
  if (y && (!wd || !wds)) return MOE_E_ARG;
  if (!all_aligned({xq, xs, wg, wgs, wu, wus, wd, wds, a, y, gu}))
    return MOE_E_ALIGN;
  if (!workspace || workspace_bytes < fwd_bytes(R_cap, n_local, I))
    return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  Carve c(workspace);
  const LinWs w = carve_lin(c, R_cap, n_local, I);
  const int cus = num_cus();
  moe::MxGemmDesc d{};
  // gate/up: x (along H) x W_g, W_u (along H); SwiGLU x scale epilogue
  d.A = xq; d.As = xs; d.lda = H; d.ldas = H / 32;
  d.B0 = wg; d.B0s = wgs; d.B1 = wu; d.B1s = wus;
  d.ldb = H; d.ldbs = H / 32; d.b_stride = I * H; d.bs_stride = I * H / 32;
  d.offsets = offsets; d.tile_ws = w.tiles; d.err = w.err; d.G = (int)n_local;
  d.N = (int)I; d.K = (int)H; d.R_cap = R_cap;
  d.C = a; d.ldc = I; d.row_scale = s_perm;
  d.gu = gu; d.ldgu = 2 * I;
  // the epilogue also quantises a along I (from fp32), for the down projection
  d.q = w.xq; d.qs = w.xs; d.ldq = I; d.ldqs = I / 32;
  hipError_t err = moe::launch_mx_rowseg(d, moe::MXE_SWIGLU, cus, stream);
  if (err != hipSuccess) return MOE_E_HIP;
  if (!y) return MOE_OK;
  // down: MX(a) (along I) x W_d (along I)
  return status_of(run_linear(a, offsets, n_local, R_cap, I, H, wd, wds, y, w,
                              cus, stream, /*quantised=*/true));
}

int moe_grouped_mlp_mxfp8_fwd_down(const int32_t *offsets, int64_t n_local,
                                   int64_t R_cap, int64_t H, int64_t I,
                                   const uint8_t *wd, const uint8_t *wds,
                                   void *y, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return MOE_E_SHAPE;
  if (R_cap == 0) return MOE_OK;
  if (!offsets || !wd || !wds || !y) return MOE_E_ARG;
  if (!all_aligned({wd, wds, y})) return MOE_E_ALIGN;
  if (!workspace || workspace_bytes < fwd_bytes(R_cap, n_local, I))
    return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  Carve c(workspace);
  const LinWs w = carve_lin(c, R_cap, n_local, I);
  return status_of(run_linear(nullptr, offsets, n_local, R_cap, I, H, wd, wds,
                              y, w, num_cus(), stream, /*quantised=*/true));
}

size_t moe_grouped_linear_mxfp8_workspace_bytes(int64_t R_cap,
                                                int64_t n_local, int64_t K) {
  if (!mx_shape_ok(n_local, R_cap, K, 512)) return 0;
  return lin_bytes(R_cap, n_local, K);
}

int moe_grouped_linear_mxfp8(const void *x, const int32_t *offsets,
                             int64_t n_local, int64_t R_cap, int64_t K,
                             int64_t N, const uint8_t *w,
                             const uint8_t *w_scales, void *y, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!mx_shape_ok(n_local, R_cap, K, 512)) return MOE_E_SHAPE;
  if (N < 1 || (int64_t)n_local * N >= kMaxRows) return MOE_E_SHAPE;
  if (R_cap == 0) return MOE_OK;
  if (!x || !offsets || !w || !w_scales || !y) return MOE_E_ARG;
  if (!all_aligned({x, w, w_scales, y})) return MOE_E_ALIGN;
  if (!workspace || workspace_bytes < lin_bytes(R_cap, n_local, K))
    return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  Carve c(workspace);
  const LinWs ws = carve_lin(c, R_cap, n_local, K);
  return status_of(run_linear(x, offsets, n_local, R_cap, K, N, w, w_scales,
                              y, ws, num_cus(), stream));
}

size_t moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes(int64_t R_cap,
                                                      int64_t n_local,
                                                      int64_t H, int64_t I) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return 0;
  return down_bwd_bytes(R_cap, n_local, H, I);
}

int moe_grouped_mlp_mxfp8_bwd_down(
    const void *dy, const float *gu, const int32_t *offsets,
    const float *s_perm, int64_t n_local, int64_t R_cap, int64_t H, int64_t I,
    const uint8_t *wdt, const uint8_t *wdts, void *dgu, float *ds,
    void *dw_down, int grad_format, void *workspace, size_t workspace_bytes,
    hipStream_t stream) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return MOE_E_SHAPE;
  if (!grad_format_ok(grad_format)) return MOE_E_ARG;
  if (R_cap == 0) return MOE_OK;
  if (!dy || !gu || !offsets || !wdt || !wdts || !dgu || !ds || !dw_down)
    return MOE_E_ARG;
  if (!all_aligned({dy, gu, wdt, wdts, dgu, ds, dw_down}))
    return MOE_E_ALIGN;
  if (!workspace || workspace_bytes < down_bwd_bytes(R_cap, n_local, H, I))
    return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  Carve c(workspace);
  const DownBwdWs w = carve_down_bwd(c, R_cap, n_local, H, I);
  return status_of(run_down_bwd(dy, gu, offsets, s_perm, n_local, R_cap, H,
                                I, wdt, wdts, dgu, ds, dw_down, w, w.err,
                                num_cus(), stream, grad_format));
}

size_t moe_grouped_mlp_mxfp8_bwd_gate_up_workspace_bytes(int64_t R_cap,
                                                         int64_t n_local,
                                                         int64_t H,
                                                         int64_t I) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return 0;
  return gate_up_bwd_bytes(R_cap, n_local, H, I);
}

int moe_grouped_mlp_mxfp8_bwd_gate_up(
    const void *dgu, const void *x_perm, const int32_t *offsets,
    int64_t n_local, int64_t R_cap, int64_t H, int64_t I, const uint8_t *wgt,
    const uint8_t *wgts, const uint8_t *wut, const uint8_t *wuts, void *dx,
    void *dw_gate, void *dw_up, int grad_format, void *workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return MOE_E_SHAPE;
  if (!grad_format_ok(grad_format)) return MOE_E_ARG;
  if (R_cap == 0) return MOE_OK;
  if (!dgu || !x_perm || !offsets || !wgt || !wgts || !wut || !wuts || !dx ||
      !dw_gate || !dw_up)
    return MOE_E_ARG;
  if (!all_aligned({dgu, x_perm, wgt, wgts, wut, wuts, dx, dw_gate, dw_up}))
    return MOE_E_ALIGN;
  if (!workspace || workspace_bytes < gate_up_bwd_bytes(R_cap, n_local, H, I))
    return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  Carve c(workspace);
  const GateUpBwdWs w = carve_gate_up_bwd(c, R_cap, n_local, H, I);
  return status_of(run_gate_up_bwd(dgu, x_perm, offsets, n_local, R_cap, H, I,
                                   wgt, wgts, wut, wuts, dx, dw_gate, dw_up, w,
                                   w.err, num_cus(), stream, grad_format));
}

size_t moe_grouped_mlp_mxfp8_bwd_workspace_bytes(int64_t R_cap,
                                                 int64_t n_local, int64_t H,
                                                 int64_t I) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return 0;
  return bwd_bytes(R_cap, n_local, H, I);
}

int moe_grouped_mlp_mxfp8_bwd(
    const void *dy, const void *x_perm, const float *gu,
    const int32_t *offsets, const float *s_perm, int64_t n_local,
    int64_t R_cap, int64_t H, int64_t I, const uint8_t *wdt,
    const uint8_t *wdts, const uint8_t *wgt, const uint8_t *wgts,
    const uint8_t *wut, const uint8_t *wuts, void *dx, float *ds,
    void *dw_gate, void *dw_up, void *dw_down, int grad_format,
    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!mx_shape_ok(n_local, R_cap, H, I)) return MOE_E_SHAPE;
  if (!grad_format_ok(grad_format)) return MOE_E_ARG;
  if (R_cap == 0) return MOE_OK;
  if (!dy || !x_perm || !gu || !offsets || !wdt || !wdts || !wgt ||
      !wgts || !wut || !wuts || !dx || !ds || !dw_gate || !dw_up || !dw_down)
    return MOE_E_ARG;
  if (!all_aligned({dy, x_perm, gu, wdt, wdts, wgt, wgts, wut, wuts, dx, ds,
                    dw_gate, dw_up, dw_down}))
    return MOE_E_ALIGN;
  if (!workspace || workspace_bytes < bwd_bytes(R_cap, n_local, H, I))
    return MOE_E_WORKSPACE;
  if (!aligned16(workspace)) return MOE_E_ALIGN;
  Carve c(workspace);
  int32_t *err = carve_err(c);
  // [dg | du] never exists in bf16 here: the SwiGLU-backward epilogue writes
  // its MX copies (row-wise and per segment column-wise) directly.
  const DguCodes codes = carve_dgu_codes(c, R_cap, n_local, I);
  Carve shared = c;   // both halves carve the same region, one after the other
  const int cus = num_cus();
  const DownBwdWs wd = carve_down_bwd(c, R_cap, n_local, H, I);
  hipError_t herr = run_down_bwd(dy, gu, offsets, s_perm, n_local, R_cap,
                                 H, I, wdt, wdts, nullptr, ds, dw_down, wd, err,
                                 cus, stream, grad_format, &codes);
  if (herr != hipSuccess) return MOE_E_HIP;
  const GateUpBwdWs wg =
      carve_gate_up_bwd(shared, R_cap, n_local, H, I, /*own_dgu=*/false);
  return status_of(run_gate_up_bwd(nullptr, x_perm, offsets, n_local, R_cap,
                                   H, I, wgt, wgts, wut, wuts, dx, dw_gate,
                                   dw_up, wg, err, cus, stream, grad_format,
                                   &codes));
}


int moe_mxfp8_workspace_view(int call, int tensor, int64_t R_cap,
                             int64_t n_local, int64_t H, int64_t I,
                             moe_mx_view *view) {
  if (view == nullptr) return MOE_E_ARG;
  if (!mx_shape_ok(n_local, R_cap, H, I)) return MOE_E_SHAPE;
  // Carve from a nominal base to read offsets off the same layout the
  // calls use.
  char *const base = (char *)(uintptr_t)4096;
  Carve c(base);
  auto off = [&](const void *p) { return (int64_t)((const char *)p - base); };
  moe_mx_view v{};
  v.pad = -1;
  if (call == MOE_MXCALL_FWD && tensor == MOE_MXT_A_ROWS) {
    const LinWs w = carve_lin(c, R_cap, n_local, I);
    v.codes = off(w.xq); v.scales = off(w.xs);
    v.ld_codes = I; v.ld_scales = I / 32; v.rows = R_cap; v.cols = I;
  } else if (call == MOE_MXCALL_BWD_DOWN && tensor == MOE_MXT_A_COLS) {
    const DownBwdWs w = carve_down_bwd(c, R_cap, n_local, H, I);
    v.codes = off(w.aT); v.scales = off(w.aTs); v.pad = off(w.kpad);
    v.ld_codes = w.kcap; v.ld_scales = w.kcap / 32; v.rows = I; v.cols = w.kcap;
  } else if (call == MOE_MXCALL_BWD &&
             (tensor == MOE_MXT_DGU_ROWS || tensor == MOE_MXT_DG_COLS ||
              tensor == MOE_MXT_DU_COLS)) {
    carve_err(c);
    const DguCodes d = carve_dgu_codes(c, R_cap, n_local, I);
    if (tensor == MOE_MXT_DGU_ROWS) {
      v.codes = off(d.q); v.scales = off(d.qs);
      v.ld_codes = 2 * I; v.ld_scales = 2 * I / 32; v.rows = R_cap; v.cols = 2 * I;
    } else {
      const bool g = tensor == MOE_MXT_DG_COLS;
      v.codes = off(g ? d.gT : d.uT); v.scales = off(g ? d.gTs : d.uTs);
      v.pad = off(d.tpad);
      v.ld_codes = d.kcap; v.ld_scales = d.kcap / 32; v.rows = I; v.cols = d.kcap;
    }
  } else {
    return MOE_E_UNSUPPORTED;
  }
  *view = v;
  return MOE_OK;
}

}  // extern "C"
