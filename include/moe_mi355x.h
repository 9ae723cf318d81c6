/*
 * moe_mi355x.h - C ABI of the MoE expert-layer library for MI355X (gfx950).
 *
 * One GPU's share of a Mixture-of-Experts expert layer:
 *   route (router GEMM, softmax, top-k, renormalise)
 *   -> permute (per-expert counts, offsets, stable dispatch of token rows)
 *   -> grouped gate/up GEMM with the SwiGLU x routing-scale epilogue
 *   -> grouped down GEMM
 *   -> unpermute / combine (weighted sum back to token order)
 * plus an MXFP8 variant of the grouped MLP (E4M3 values, one E8M0 scale per
 * 32 values along the reduction axis).
 *
 * Passages of the pages that define the operations (cited by page title and
 * section):
 *   "Wide-EPとは?" explainer (scholia-notes), sections
 *     前提:MoE(Mixture of Experts)とは - a router chooses a few experts per
 *       token; only those compute; their results are summed.
 *     MoEの課題 - which expert is chosen when is not known beforehand.
 *     効果2:演算強度が上がる - grouping many tokens per expert (GroupGEMM)
 *       reuses each weight byte read from HBM.
 *     前提条件:GPU間の高速通信 - tokens go to their expert (dispatch) and the
 *       results come back (combine).
 *   BioNeMo MoE article (quantumzeitgeist), sections
 *     GroupedLinear Optimizes Expert Computation in MoE Models - expert
 *       matrices stay separate but are submitted as one operation; the
 *       ScaledSwiGLU step folds the routing probabilities ("scales") into the
 *       expert FFN; the fused MLP avoids materialising intermediates.
 *     MXFP8 Precision Reduces Memory Footprint for Biological Models - 8-bit
 *       values, a scale per block of 32 consecutive values; quantisation,
 *       SwiGLU and routing-weight scaling fused into one kernel.
 *   NVL72 Wide-EP news item (mexc.fm), "Kernel Optimization and Load
 *     Balancing" - expert routing moves data whose sizes are not static.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns
 *     every buffer and the stream.  The library never allocates or frees
 *     device memory and never synchronises the stream (except
 *     moe_debug_sync, which exists for tests).
 *   - Work is enqueued on `stream` (NULL = the default stream).
 *   - Return value: MOE_OK, or an MOE_E_* code.  Arguments are validated on
 *     the host before anything is enqueued; on a validation error nothing is
 *     enqueued.  A failed launch returns MOE_E_HIP.  No exception crosses the
 *     ABI and the library never aborts.
 *   - Per-expert row counts exist only on the device (they are data); every
 *     consumer reads them from `offsets`, so no host round trip happens.
 *   - Matrices are row-major.  Weights are stored K-contiguous like
 *     nn.Linear: W_router [E, H], W_gate and W_up [n_local, I, H],
 *     W_down [n_local, H, I].
 *   - dtype MOE_DT_BF16: activations, weights and outputs bf16 (raw 16-bit),
 *     fp32 accumulation, outputs rounded to nearest even.  MOE_DT_F32: all
 *     fp32.  Routing weights, logits and scales are always fp32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_E_ARG = 1,          /* NULL where a buffer is required, bad enum    */
  MOE_E_SHAPE = 2,        /* sizes out of range or inconsistent           */
  MOE_E_ALIGN = 3,        /* pointer not 16-byte aligned                  */
  MOE_E_WORKSPACE = 4,    /* workspace missing or too small               */
  MOE_E_UNSUPPORTED = 5,  /* valid but not implemented combination        */
  MOE_E_HIP = 6           /* a HIP launch or runtime call failed          */
};

enum moe_dtype { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 };

/* Human-readable name of a status code (static string, host). */
const char *moe_status_string(int status);

/* Library version as 10000*major + 100*minor + patch (host). */
int moe_version(void);

/*
 * moe_route_topk - router scores, softmax over all E experts, the k most
 * probable experts per token, their probabilities renormalised to sum to 1.
 * (Wide-EP explainer, 前提:MoEとは: the router picks k of E per token.)
 *
 * Two modes:
 *   x != NULL and w_router != NULL:  logits[t, e] = sum_h x[t,h] w_router[e,h]
 *       (+ bias[e] when bias != NULL), written to `logits` (fp32), then top-k.
 *   x == NULL and w_router == NULL:  `logits` is an input; only top-k runs
 *       (bias must be NULL).
 * x [T, H], w_router [E, H] of `dtype`; bias [E] fp32; logits [T, E] fp32.
 * Outputs: topk_idx [T, k] int32 (descending probability; equal logits go to
 * the lower expert index first) and topk_w [T, k] fp32.
 * The top-k decision is taken on the fp32 logits.  The weights are
 * exp(l_j - l_max) / sum over the kept experts of exp(l - l_max).
 * Limits: 1 <= k <= min(E, 32), 1 <= E <= 1024, T >= 0 (T == 0 enqueues
 * nothing), H >= 1; in GEMM mode with bf16, H % 64 == 0.
 */
int moe_route_topk(const void *x, const void *w_router, const float *bias,
                   float *logits, int64_t T, int64_t H, int64_t E, int64_t k,
                   int dtype, int32_t *topk_idx, float *topk_w,
                   hipStream_t stream);

/*
 * moe_permute - local dispatch: lay the (token, slot) pairs routed to this
 * GPU's experts [e_begin, e_begin + n_local) out expert by expert.
 * (Wide-EP explainer, 前提条件:GPU間の高速通信 - dispatch; MoEの課題 and the
 * NVL72 news item - counts are data, not static sizes.)
 *
 * Flat slot f = t*k + j.  Inside an expert, slots keep ascending f (a stable
 * counting sort), so the result is unique and deterministic.
 * Inputs:  topk_idx [T, k] int32; topk_w [T, k] fp32 or NULL;
 *          x [T, H] of dtype or NULL (then x_perm is not written).
 * Outputs: counts [n_local], offsets [n_local + 1] (exclusive scan,
 *          offsets[n_local] = R, the rows this GPU computes),
 *          row_src [T*k] (rows < R: the flat slot placed there),
 *          inv [T, k] (row of slot f, or -1 when its expert is not local),
 *          x_perm [T*k, H] (rows < R: x_perm[r] = x[row_src[r] / k]),
 *          s_perm [T*k] fp32 (rows < R: topk_w of that slot; skipped when
 *          topk_w is NULL or s_perm is NULL).
 * Rows >= R of the capacity-sized outputs are left untouched.
 * Indices outside [e_begin, e_begin + n_local) are non-local: dropped.
 * workspace: moe_permute_workspace_bytes(T, k, n_local) bytes, 16-aligned.
 * Limits: 1 <= k <= 32, T*k < 2^31, 1 <= n_local <= 4096, H % 8 == 0 when
 * x is given (bf16) or H % 4 == 0 (fp32).
 */
size_t moe_permute_workspace_bytes(int64_t T, int64_t k, int64_t n_local);
int moe_permute(const int32_t *topk_idx, const float *topk_w, const void *x,
                int64_t T, int64_t k, int64_t H, int dtype, int64_t e_begin,
                int64_t n_local, void *x_perm, float *s_perm,
                int32_t *row_src, int32_t *inv, int32_t *counts,
                int32_t *offsets, void *workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * moe_grouped_gate_up - for every local expert e and its rows
 * [offsets[e], offsets[e+1]) of x_perm, in one launch for all experts
 * (BioNeMo article, GroupedLinear section):
 *   g = x_perm . W_gate[e]^T,  u = x_perm . W_up[e]^T   (fp32 accumulation)
 *   a = s_perm[r] * SiLU(g) * u   (ScaledSwiGLU; s_perm NULL -> scale 1)
 * g and u never leave the chip; only `a` [R_cap, I] (dtype) is written, rows
 * < R.  SiLU(z) = z * sigmoid(z).
 * workspace: moe_grouped_ffn_workspace_bytes(...) bytes, 16-aligned.
 * Limits (bf16): H % 64 == 0, I % 64 == 0, 1 <= n_local <= 4096,
 * R_cap < 2^31.  (fp32): H % 4 == 0, I % 4 == 0.
 */
size_t moe_grouped_ffn_workspace_bytes(int64_t R_cap, int64_t n_local,
                                       int64_t H, int64_t I, int dtype);
int moe_grouped_gate_up(const void *x_perm, const int32_t *offsets,
                        const float *s_perm, int64_t n_local, int64_t R_cap,
                        int64_t H, int64_t I, const void *w_gate,
                        const void *w_up, int dtype, void *a, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_gate_up_gather - moe_grouped_gate_up with the expert rows
 * read straight from the token rows: permuted row r is x[row_src[r] / k]
 * (row_src as written by moe_permute, which may then skip x_perm by passing
 * x = NULL).  Saves writing and re-reading the permuted copy of x.
 * x [T, H] bf16; row_src [R_cap] int32 (rows < offsets[n_local] are read;
 * an index past the last token is clamped to it).  Other arguments as for
 * moe_grouped_gate_up; results are identical to it on x_perm.
 * dtype: MOE_DT_BF16 only (MOE_E_UNSUPPORTED otherwise); R_cap <= T * k.
 */
int moe_grouped_gate_up_gather(const void *x, const int32_t *row_src,
                               int64_t T, int64_t k, const int32_t *offsets,
                               const float *s_perm, int64_t n_local,
                               int64_t R_cap, int64_t H, int64_t I,
                               const void *w_gate, const void *w_up, int dtype,
                               void *a, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_down - y[r] = a[r] . W_down[e]^T for every local expert's rows
 * (fp32 accumulation, dtype output), rows < R of y [R_cap, H].
 * Same limits and workspace as moe_grouped_gate_up.
 */
int moe_grouped_down(const void *a, const int32_t *offsets, int64_t n_local,
                     int64_t R_cap, int64_t H, int64_t I, const void *w_down,
                     int dtype, void *y, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn - moe_grouped_gate_up followed by moe_grouped_down; `a`
 * [R_cap, I] (dtype) is the one intermediate handed between them.
 */
int moe_grouped_ffn(const void *x_perm, const int32_t *offsets,
                    const float *s_perm, int64_t n_local, int64_t R_cap,
                    int64_t H, int64_t I, const void *w_gate,
                    const void *w_up, const void *w_down, int dtype, void *a,
                    void *y, void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * moe_unpermute_combine - bring expert outputs back to token order and add
 * them up (Wide-EP explainer, 前提:MoEとは and 前提条件:GPU間の高速通信):
 *   out[t] = sum over j ascending with inv[t,j] >= 0 of c_tj * y[inv[t,j]]
 * with c_tj = topk_w[t,j] when topk_w != NULL, else 1 (use NULL when the
 * routing scale already went into the gate/up epilogue).  fp32 accumulation,
 * one rounding to dtype at the end; tokens with no local slot get a zero
 * row.  No atomics: the result is bitwise reproducible.
 * y [>= max(inv)+1, H], inv [T, k] int32, out [T, H] (dtype).
 * Limits: 1 <= k <= 32, H % 8 == 0 (bf16) or H % 4 == 0 (fp32).
 */
int moe_unpermute_combine(const void *y, const int32_t *inv,
                          const float *topk_w, int64_t T, int64_t k,
                          int64_t H, int dtype, void *out, hipStream_t stream);

/*
 * ---- MXFP8 (BioNeMo MoE article, "MXFP8 Precision Reduces Memory Footprint
 * for Biological Models": 8-bit values with one scale per block of 32
 * consecutive values; "GroupedLinear Optimizes Expert Computation in MoE
 * Models": the GroupedLinear -> ScaledSwiGLU -> GroupedLinear chain as one
 * fused forward and one fused backward).
 * Element format FP8 E4M3 (OCP "FN": bias 7, max 448, 0x7F/0xFF NaN), scale
 * E8M0 (2^(byte - 127)).  Conversion rule (the pages give none; OCP MX v1.0):
 * X = floor(log2(max|v|)) - 8 per block, scale byte X + 127 (clamped to
 * [0, 254]), code = v * 2^-X rounded to nearest E4M3, ties to even,
 * saturating at +-448, sign kept for values rounding to zero; an all-zero
 * block has scale byte 0.
 */

/*
 * moe_mxfp8_quantize - MX-quantise a bf16 matrix in[rows, cols] (row pitch
 * ld_in elements, ld_in % 8 == 0, `in` 16-byte aligned), cols % 32 == 0.
 * axis 0: blocks of 32 along each row.  codes [rows, ld_codes] bytes
 *   (ld_codes % 16 == 0), scales [rows, ld_scales] (>= cols/32).
 * axis 1: blocks of 32 down each column, output transposed for a GEMM whose
 *   reduction runs over rows: codes [cols, ld_codes], scales [cols,
 *   ld_scales].  Rows may be split into segments seg_offsets[0..n_seg]
 *   (device, non-decreasing; NULL = one segment [0, rows)); each segment is
 *   zero-padded to a multiple of `align` (32 or 512) and starts at column
 *   pad_offsets[s] of the output (written to pad_offsets [n_seg + 1], device,
 *   when seg_offsets is given).  ld_codes must hold the padded total
 *   (>= rows + (align - 1) * n_seg), ld_scales >= ld_codes / 32.
 * Codes and scales of a given input match the rule above bit for bit.
 */
int moe_mxfp8_quantize(const void *in, int64_t rows, int64_t cols,
                       int64_t ld_in, int axis, const int32_t *seg_offsets,
                       int64_t n_seg, int64_t align, uint8_t *codes,
                       int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                       int32_t *pad_offsets, hipStream_t stream);

/*
 * moe_grouped_mlp_mxfp8_fwd - MXFP8 grouped MLP forward on permuted rows:
 *   g, u = MX(x) . MX(W_gate)^T, MX(x) . MX(W_up)^T     (blocks along H)
 *   a    = s * SiLU(g) * u                               (bf16, written)
 *   y    = MX(a) . MX(W_down)^T                          (blocks along I)
 * Inputs: xq/xs = x_perm quantised along H (axis 0: [R_cap, H] codes,
 * [R_cap, H/32] scales); W_gate/W_up codes [n_local*I, H] + scales
 * [n_local*I, H/32] and W_down codes [n_local*H, I] + scales [n_local*H,
 * I/32] (axis 0 of the stacked weights); offsets, s_perm as in
 * moe_grouped_gate_up (s_perm may be NULL).
 * Outputs (bf16): a [R_cap, I]; gu [R_cap, 2I] = [g | u] per row (may be
 * NULL; the backward needs it); y [R_cap, H].  Rows < R are written.
 * The SwiGLU epilogue also writes MX(a) (blocks along I, from the bf16 a it
 * stores) into the workspace, and the down projection reads those codes
 * (the fused quantisation of the MXFP8 section).
 * y == NULL stops after a (wd, wds are then not read); the down projection
 * is then moe_grouped_mlp_mxfp8_fwd_down with the same workspace, or
 * moe_grouped_linear_mxfp8 on a (same result).
 * workspace: moe_grouped_mlp_mxfp8_fwd_workspace_bytes() bytes.
 * Limits: H % 512 == 0, I % 512 == 0, 1 <= n_local <= 4096.
 */
size_t moe_grouped_mlp_mxfp8_fwd_workspace_bytes(int64_t R_cap,
                                                 int64_t n_local, int64_t H,
                                                 int64_t I);
int moe_grouped_mlp_mxfp8_fwd(const uint8_t *xq, const uint8_t *xs,
                              const int32_t *offsets, const float *s_perm,
                              int64_t n_local, int64_t R_cap, int64_t H,
                              int64_t I, const uint8_t *wg, const uint8_t *wgs,
                              const uint8_t *wu, const uint8_t *wus,
                              const uint8_t *wd, const uint8_t *wds, void *a,
                              void *gu, void *y, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_mlp_mxfp8_fwd_down - the down projection of
 * moe_grouped_mlp_mxfp8_fwd, y = MX(a) . MX(W_down)^T, reading the MX(a)
 * that a preceding moe_grouped_mlp_mxfp8_fwd call with y == NULL left in
 * `workspace` (same stream or ordered after it; same offsets, n_local,
 * R_cap, H, I).  Result identical to the one-call forward.
 * wd, wds, y as in moe_grouped_mlp_mxfp8_fwd; the same workspace size.
 */
int moe_grouped_mlp_mxfp8_fwd_down(const int32_t *offsets, int64_t n_local,
                                   int64_t R_cap, int64_t H, int64_t I,
                                   const uint8_t *wd, const uint8_t *wds,
                                   void *y, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_linear_mxfp8 - one MXFP8 GroupedLinear on permuted rows (the
 * GroupedLinear of "GroupedLinear Optimizes Expert Computation in MoE
 * Models", operands as in the MXFP8 section of the BioNeMo MoE article):
 *   y[r, :] = MX(x[r, :]) . MX(W_e)^T   for rows r of expert e's segment
 * x [R_cap, K] bf16 is quantised along K inside the call (rows past
 * offsets[n_local] are not read); W codes [n_local*N, K] + scales
 * [n_local*N, K/32] (axis 0 of the stacked [n_local, N, K] weights);
 * y [R_cap, N] bf16, rows < R written.  The forward's down projection is
 * this call with x = a, K = I, N = H.
 * workspace: moe_grouped_linear_mxfp8_workspace_bytes() bytes.
 * Limits: K % 512 == 0, N >= 1, 1 <= n_local <= 4096.
 */
size_t moe_grouped_linear_mxfp8_workspace_bytes(int64_t R_cap,
                                                int64_t n_local, int64_t K);
int moe_grouped_linear_mxfp8(const void *x, const int32_t *offsets,
                             int64_t n_local, int64_t R_cap, int64_t K,
                             int64_t N, const uint8_t *w,
                             const uint8_t *w_scales, void *y, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_mlp_mxfp8_bwd - backward of the forward above by the chain
 * rule, every GEMM operand MX-quantised along that GEMM's reduction axis:
 *   da = MX(dY) . MX_H(W_down)                 (K = H)
 *   dg = da*s*u*SiLU'(g), du = da*s*SiLU(g), ds = sum_i da*SiLU(g)*u
 *   dX = MX(dg) . MX_I(W_gate) + MX(du) . MX_I(W_up)   (K = I)
 *   dW_down[e] = MX_R(dY_e)^T . MX_R(a_e), dW_gate[e] = MX_R(dg_e)^T .
 *   MX_R(x_e), dW_up[e] = MX_R(du_e)^T . MX_R(x_e)   (K = rows of expert e)
 * Inputs (bf16): dy [R_cap, H], x_perm [R_cap, H], a [R_cap, I], gu [R_cap,
 * 2I] from the forward; offsets, s_perm; the weights quantised along the
 * other axis (axis 1 of the stacked weights): wdt/wdts = W_down as [n_local*H,
 * I] -> codes [I, n_local*H], scales [I, n_local*H/32]; wgt/wgts, wut/wuts =
 * W_gate, W_up as [n_local*I, H] -> codes [H, n_local*I], scales [H,
 * n_local*I/32].
 * Outputs: dx [R_cap, H] bf16, ds [R_cap] fp32 (sum in a fixed order),
 * dw_gate, dw_up [n_local, I, H] bf16, dw_down [n_local, H, I] bf16 (an
 * expert without rows gets zero gradients).
 * The call computes what moe_grouped_mlp_mxfp8_bwd_down followed by
 * moe_grouped_mlp_mxfp8_bwd_gate_up compute, with identical bits, but [dg |
 * du] never exists in bf16: the epilogue that produces it writes its MX codes
 * (along 2I, and down each expert's rows) into the workspace directly.
 * workspace: moe_grouped_mlp_mxfp8_bwd_workspace_bytes() bytes.
 * Limits as for the forward.
 */
size_t moe_grouped_mlp_mxfp8_bwd_workspace_bytes(int64_t R_cap,
                                                 int64_t n_local, int64_t H,
                                                 int64_t I);
int moe_grouped_mlp_mxfp8_bwd(
    const void *dy, const void *x_perm, const void *a, const void *gu,
    const int32_t *offsets, const float *s_perm, int64_t n_local,
    int64_t R_cap, int64_t H, int64_t I, const uint8_t *wdt,
    const uint8_t *wdts, const uint8_t *wgt, const uint8_t *wgts,
    const uint8_t *wut, const uint8_t *wuts, void *dx, float *ds,
    void *dw_gate, void *dw_up, void *dw_down, void *workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_mlp_mxfp8_bwd_down - first half of the backward: the down
 * projection's data and weight gradients and the ScaledSwiGLU backward.
 *   da = MX(dY) . MX_H(W_down);  dg, du, ds as above;
 *   dW_down[e] = MX_R(dY_e)^T . MX_R(a_e)
 * Inputs: dy [R_cap, H], a [R_cap, I], gu [R_cap, 2I] (bf16), offsets,
 * s_perm (may be NULL: s = 1), wdt/wdts as for moe_grouped_mlp_mxfp8_bwd.
 * Outputs: dgu [R_cap, 2I] bf16 = [dg | du] per row, ds [R_cap] fp32,
 * dw_down [n_local, H, I] bf16.
 * workspace: moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes() bytes.
 */
size_t moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes(int64_t R_cap,
                                                      int64_t n_local,
                                                      int64_t H, int64_t I);
int moe_grouped_mlp_mxfp8_bwd_down(
    const void *dy, const void *a, const void *gu, const int32_t *offsets,
    const float *s_perm, int64_t n_local, int64_t R_cap, int64_t H, int64_t I,
    const uint8_t *wdt, const uint8_t *wdts, void *dgu, float *ds,
    void *dw_down, void *workspace, size_t workspace_bytes,
    hipStream_t stream);

/*
 * moe_grouped_mlp_mxfp8_bwd_gate_up - second half of the backward: the
 * gate/up projection's data and weight gradients from [dg | du].
 *   dX = MX(dg) . MX_I(W_gate) + MX(du) . MX_I(W_up);
 *   dW_gate[e] = MX_R(dg_e)^T . MX_R(x_e), dW_up[e] = MX_R(du_e)^T . MX_R(x_e)
 * Inputs: dgu [R_cap, 2I] bf16, x_perm [R_cap, H] bf16, offsets, wgt/wgts,
 * wut/wuts as for moe_grouped_mlp_mxfp8_bwd.  Outputs: dx [R_cap, H],
 * dw_gate, dw_up [n_local, I, H] (bf16).
 * workspace: moe_grouped_mlp_mxfp8_bwd_gate_up_workspace_bytes() bytes.
 */
size_t moe_grouped_mlp_mxfp8_bwd_gate_up_workspace_bytes(int64_t R_cap,
                                                         int64_t n_local,
                                                         int64_t H,
                                                         int64_t I);
int moe_grouped_mlp_mxfp8_bwd_gate_up(
    const void *dgu, const void *x_perm, const int32_t *offsets,
    int64_t n_local, int64_t R_cap, int64_t H, int64_t I, const uint8_t *wgt,
    const uint8_t *wgts, const uint8_t *wut, const uint8_t *wuts, void *dx,
    void *dw_gate, void *dw_up, void *workspace, size_t workspace_bytes,
    hipStream_t stream);

/* Waits for `stream` and reports a pending HIP error as MOE_E_HIP (tests). */
int moe_debug_sync(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
