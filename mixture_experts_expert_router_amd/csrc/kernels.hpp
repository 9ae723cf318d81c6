// Launchers of the gfx950 kernels (host side).  Every launcher enqueues on
// the given stream and returns the launch status; arguments are validated by
// the C-ABI entry points before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Every workspace begins with a header of kErrHeaderBytes whose first int32
// is the device error word (bit values as MOE_DEVERR_* in moe_mi355x.h).
constexpr size_t kErrHeaderBytes = 256;
constexpr int32_t kDevErrExpertIndex = 1;  // a top-k index outside [0, E)
constexpr int32_t kDevErrRows = 2;         // offsets past R_cap or decreasing
constexpr int32_t kDevErrWait = 4;         // a fused down unit stopped waiting

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
                                int64_t n_local, void *ws, hipStream_t s);
hipError_t launch_permute(const int32_t *idx, const float *w, const void *x,
                          int64_t T, int64_t k, int64_t row_bytes, int64_t E,
                          int64_t e_begin, int64_t n_local, void *x_perm,
                          float *s_perm, int32_t *row_src, int32_t *inv,
                          int32_t *counts, int32_t *offsets, void *ws,
                          int num_cus, hipStream_t s);

// x_perm[r] = x[row_src[r] / k] for r < *R_ptr (16-byte vectors).
hipError_t launch_permute_gather(const void *x, int64_t row_bytes, int64_t k,
                                 const int32_t *row_src, const int32_t *R_ptr,
                                 void *x_perm, int64_t F, int num_cus,
                                 hipStream_t s);

// ---- expert-parallel load balancing ----
hipError_t launch_eplb_plan(const int32_t *counts, int E, int S, int G,
                            int32_t *rep, int32_t *rep_first,
                            int32_t *rep_slot, int32_t *slot_expert,
                            int32_t *slot_copy, hipStream_t s);
size_t permute_replicated_workspace_bytes(int64_t T, int64_t k, int64_t E,
                                          int64_t n_slots);
hipError_t launch_permute_replicated(
    const int32_t *idx, const float *w, const void *x, int64_t T, int64_t k,
    int64_t row_bytes, int64_t E, const int32_t *rep_first,
    const int32_t *rep_slot, const int32_t *slot_expert,
    const int32_t *slot_copy, int64_t s_begin, int64_t n_slots, void *x_perm,
    float *s_perm, int32_t *row_src, int32_t *inv, int32_t *counts,
    int32_t *offsets, void *ws, int num_cus, hipStream_t s);

// Workspace of the grouped GEMM launches of an FFN: the error header, two
// tile prefixes of n_local + 1 and the split word, then the split-K arrival
// counters and fp32 partial slots (as many as rows up to R_cap can use, at
// most 512 of 128 KiB).
size_t gemm_workspace_bytes(int64_t n_local, int64_t R_cap, int64_t H,
                            int64_t I);

// group_w (device [n_local] or null): group g uses the weights of stacked
// expert group_w[g] (of n_w); null: expert g.
hipError_t launch_gate_up_bf16(const uint16_t *x_perm, const int32_t *offsets,
                               const float *s_perm, int n_local, int64_t R_cap,
                               int H, int I, const uint16_t *w_gate,
                               const uint16_t *w_up, uint16_t *a,
                               int32_t *tile_ws, int num_cus, hipStream_t s,
                               const int32_t *row_src = nullptr,
                               int k = 1, int64_t T = 1,
                               const int32_t *group_w = nullptr, int n_w = 0);
hipError_t launch_down_bf16(const uint16_t *a, const int32_t *offsets,
                            int n_local, int64_t R_cap, int H, int I,
                            const uint16_t *w_down, uint16_t *y,
                            int32_t *tile_ws, int num_cus, hipStream_t s,
                            const int32_t *group_w = nullptr, int n_w = 0);

// The grouped FFN issued expert by expert (gate/up, then down, per expert
// with host_counts[e] > 0), each launch one group of the same kernels.
hipError_t launch_ffn_loop_bf16(const uint16_t *x_perm, const int32_t *offsets,
                               const int32_t *host_counts, const float *s_perm,
                               int n_local, int64_t R_cap, int H, int I,
                               const uint16_t *w_gate, const uint16_t *w_up,
                               const uint16_t *w_down, uint16_t *a,
                               uint16_t *y, int32_t *tile_ws, int num_cus,
                               hipStream_t s);
// The FFN (gate/up, ScaledSwiGLU, down) in one persistent launch after a
// plan kernel, on the grouped GEMM's tiles; x is gathered through row_src
// (x [T, H]) or, with row_src null, read as x_perm [R_cap, H].
size_t ffn_fused_workspace_bytes(int64_t n_local, int64_t R_cap, int64_t H,
                                 int64_t I);
hipError_t launch_ffn_fused_bf16(const uint16_t *x, const int32_t *row_src,
                                 int k, int64_t T, const int32_t *offsets,
                                 const float *s_perm, int n_local,
                                 int64_t R_cap, int H, int I,
                                 const uint16_t *w_gate, const uint16_t *w_up,
                                 const uint16_t *w_down, uint16_t *a,
                                 uint16_t *y, int32_t *ws, int num_cus,
                                 hipStream_t s);
// The grouped FFN: one plan kernel for both GEMMs, then the gate/up and the
// down launches of the grouped GEMM (the same kernels, tiles and results as
// launch_gate_up_bf16 followed by launch_down_bf16); x as for the one-launch
// FFN; the workspace as the one-launch FFN's.
hipError_t launch_ffn_grouped_bf16(const uint16_t *x, const int32_t *row_src,
                                   int k, int64_t T, const int32_t *offsets,
                                   const float *s_perm, int n_local,
                                   int64_t R_cap, int H, int I,
                                   const uint16_t *w_gate,
                                   const uint16_t *w_up,
                                   const uint16_t *w_down, uint16_t *a,
                                   uint16_t *y, int32_t *ws, int num_cus,
                                   hipStream_t s);
hipError_t launch_gate_up_f32(const float *x_perm, const int32_t *offsets,
                              const float *s_perm, int n_local, int64_t R_cap,
                              int64_t H, int64_t I, const float *w_gate,
                              const float *w_up, float *a, hipStream_t s);
// Writes the error word of a grouped call that has no plan kernel (fp32).
hipError_t launch_check_offsets(const int32_t *offsets, int n_local,
                                int64_t R_cap, int32_t *err, hipStream_t s);
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
                                hipStream_t s, int fmt = 0);
// pad[s+1] = pad[s] + ceil(len_s / align) * align, pad[0] = 0, where len_s
// is the length of segment s cut at `rows` (see seg_rows).
hipError_t launch_mx_pad_offsets(const int32_t *seg, int nseg, int64_t rows,
                                 int align, int32_t *pad, hipStream_t s);
hipError_t launch_mx_quant_cols(const uint16_t *in, int64_t rows,
                                int64_t cols, int64_t ld_in,
                                const int32_t *seg, int nseg, int align,
                                int32_t *pad, uint8_t *codes,
                                int64_t ld_codes, uint8_t *scales,
                                int64_t ld_scales, int num_cus,
                                hipStream_t s, int fmt = 0);

// One MXFP8 grouped GEMM (see mx_gemm.hip for the modes and epilogues).
struct MxGemmDesc {
  const uint8_t *A, *As;           // codes / scales, K-contiguous
  int64_t lda, ldas;
  const uint8_t *B0, *B0s, *B1, *B1s;
  int64_t ldb, ldbs, b_stride, bs_stride;
  const int32_t *offsets;          // row-segment mode: [G + 1]
  const int32_t *kseg;             // K-segment mode: [G + 1]
  int32_t *tile_ws;                // row-segment mode: [G + 1] scratch
  int32_t *err;                    // row-segment mode: error word or null
  int G, M, N, K;
  int64_t R_cap;
  void *C;
  int64_t ldc, c_stride;
  const float *row_scale;
  float *gu;                       // fp32 [g | u] (SwiGLU out, backward in)
  int64_t ldgu;
  uint16_t *dgu;                   // bf16 [dg | du] out (or null)
  float *ds_part;
  float *ds;
  int ksplit;
  // SwiGLU: MX codes / scales of a along I; SwiGLU backward: of [dg | du]
  // along 2I (row-wise, blocks of 32 columns), encoded from fp32.  Null: not
  // written.
  uint8_t *q, *qs;
  int64_t ldq, ldqs;
  // SwiGLU backward: column-wise MX codes / scales of dg (t0), du (t1) and
  // a (t2), [N, ldt] / [N, ldts], segments padded to 256 rows at tpad,
  // encoded from fp32 (null: not written).
  uint8_t *t0, *t0s, *t1, *t1s, *t2, *t2s;
  int64_t ldt, ldts;
  const int32_t *tpad;
  // Element format of A (0 = E4M3, 1 = E5M2 for gradient operands); with the
  // SwiGLU-backward epilogue also the format of the dg, du codes (q, t0,
  // t1), while t2 (a) stays E4M3.  B is always E4M3.
  int fa;
};
enum { MXE_BF16 = 0, MXE_SWIGLU = 1, MXE_SWIGLU_BWD = 2 };
hipError_t launch_mx_rowseg(const MxGemmDesc &d, int epi, int num_cus,
                            hipStream_t s);
hipError_t launch_mx_kseg(const MxGemmDesc &d, int num_cus, hipStream_t s);
// Partial ds values per row that the SwiGLU-backward epilogue writes.
size_t mx_ds_parts(int64_t N);

}  // namespace moe
