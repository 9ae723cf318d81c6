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
hipError_t launch_permute_empty(int32_t *counts, int32_t *offsets,
                                int64_t n_local, hipStream_t s);
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
                               int32_t *tile_ws, int num_cus, hipStream_t s,
                               const int32_t *row_src = nullptr,
                               int k = 1, int64_t T = 1);
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

// ---- MXFP8 ----
hipError_t launch_mx_quant_rows(const uint16_t *in, int64_t rows, int64_t cols,
                                int64_t ld_in, uint8_t *codes,
                                int64_t ld_codes, uint8_t *scales,
                                int64_t ld_scales, const int32_t *rows_dev,
                                hipStream_t s);
// pad[s+1] = pad[s] + ceil((seg[s+1] - seg[s]) / align) * align, pad[0] = 0.
hipError_t launch_mx_pad_offsets(const int32_t *seg, int nseg, int align,
                                 int32_t *pad, hipStream_t s);
hipError_t launch_mx_quant_cols(const uint16_t *in, int64_t rows,
                                int64_t cols, int64_t ld_in,
                                const int32_t *seg, int nseg, int align,
                                int32_t *pad, uint8_t *codes,
                                int64_t ld_codes, uint8_t *scales,
                                int64_t ld_scales, int num_cus,
                                hipStream_t s);

// One MXFP8 grouped GEMM (see mx_gemm.hip for the modes and epilogues).
struct MxGemmDesc {
  const uint8_t *A, *As;           // codes / scales, K-contiguous
  int64_t lda, ldas;
  const uint8_t *B0, *B0s, *B1, *B1s;
  int64_t ldb, ldbs, b_stride, bs_stride;
  const int32_t *offsets;          // row-segment mode: [G + 1]
  const int32_t *kseg;             // K-segment mode: [G + 1]
  int32_t *tile_ws;                // row-segment mode: [G + 1] scratch
  int G, M, N, K;
  int64_t R_cap;
  void *C;
  int64_t ldc, c_stride;
  const float *row_scale;
  uint16_t *gu;
  int64_t ldgu;
  uint16_t *dgu;
  float *ds_part;
  float *ds;
  int ksplit;
  // SwiGLU: MX codes / scales of a along I; SwiGLU backward: of [dg | du]
  // along 2I (row-wise, blocks of 32 columns).  Null: not written.
  uint8_t *q, *qs;
  int64_t ldq, ldqs;
  // SwiGLU backward: column-wise MX codes / scales of dg (t0) and du (t1),
  // [N, ldt] / [N, ldts], segments padded to 256 rows at tpad (null: none).
  uint8_t *t0, *t0s, *t1, *t1s;
  int64_t ldt, ldts;
  const int32_t *tpad;
};
enum { MXE_BF16 = 0, MXE_SWIGLU = 1, MXE_SWIGLU_BWD = 2 };
hipError_t launch_mx_rowseg(const MxGemmDesc &d, int epi, int num_cus,
                            hipStream_t s);
hipError_t launch_mx_kseg(const MxGemmDesc &d, int num_cus, hipStream_t s);
// Partial ds values per row that the SwiGLU-backward epilogue writes.
size_t mx_ds_parts(int64_t N);

}  // namespace moe
