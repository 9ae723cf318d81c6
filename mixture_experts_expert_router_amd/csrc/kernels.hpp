// Launchers of the gfx950 kernels (host side).  Every launcher enqueues on
// the given stream and returns the launch status; arguments are validated by
// the C-ABI entry points before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum GemmEpilogue { EPI_SWIGLU = 0, EPI_BF16 = 1, EPI_F32_BIAS = 2 };

hipError_t launch_router_gemm_f32(const float *x, const float *w,
                                  const float *bias, float *logits, int64_t T,
                                  int64_t H, int64_t E, hipStream_t s);
hipError_t launch_router_gemm_bf16(const uint16_t *x, const uint16_t *w,
                                   const float *bias, float *logits, int64_t T,
                                   int H, int E, int num_cus, hipStream_t s);
hipError_t launch_topk(const float *logits, int64_t T, int E, int k,
                       int32_t *idx, float *w, hipStream_t s);

size_t permute_workspace_bytes(int64_t T, int64_t k, int64_t n_local);
hipError_t launch_permute(const int32_t *idx, const float *w, const void *x,
                          int64_t T, int64_t k, int64_t row_bytes,
                          int64_t e_begin, int64_t n_local, void *x_perm,
                          float *s_perm, int32_t *row_src, int32_t *inv,
                          int32_t *counts, int32_t *offsets, void *ws,
                          int num_cus, hipStream_t s);

// Workspace of one grouped GEMM launch: two tile prefixes of n_local + 1.
size_t gemm_workspace_bytes(int64_t n_local);

hipError_t launch_gate_up_bf16(const uint16_t *x_perm, const int32_t *offsets,
                               const float *s_perm, int n_local, int64_t R_cap,
                               int H, int I, const uint16_t *w_gate,
                               const uint16_t *w_up, uint16_t *a,
                               int32_t *tile_ws, int num_cus, hipStream_t s);
hipError_t launch_down_bf16(const uint16_t *a, const int32_t *offsets,
                            int n_local, int64_t R_cap, int H, int I,
                            const uint16_t *w_down, uint16_t *y,
                            int32_t *tile_ws, int num_cus, hipStream_t s);

hipError_t launch_gate_up_f32(const float *x_perm, const int32_t *offsets,
                              const float *s_perm, int n_local, int64_t R_cap,
                              int64_t H, int64_t I, const float *w_gate,
                              const float *w_up, float *a, hipStream_t s);
hipError_t launch_down_f32(const float *a, const int32_t *offsets,
                           int n_local, int64_t R_cap, int64_t H, int64_t I,
                           const float *w_down, float *y, hipStream_t s);

hipError_t launch_combine(const void *y, const int32_t *inv,
                          const float *topk_w, int64_t T, int k, int64_t H,
                          int dtype, void *out, int num_cus, hipStream_t s);

}  // namespace moe
