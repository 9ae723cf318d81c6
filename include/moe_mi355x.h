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
  MOE_E_HIP = 6,          /* a HIP launch or runtime call failed          */
  MOE_E_SCRATCH = 7       /* needs more than the no-allocation variant's
                             scratch (MOE_NOALLOC_SCRATCH_BYTES)          */
};

enum moe_dtype { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 };

/*
 * Device error word.  Every workspace the library takes begins with a
 * 256-byte header whose first int32 the call's kernels set: 0 when nothing
 * went wrong, otherwise an OR of the bits below.  Read it with
 * moe_read_device_error after the call.  (NVL72 news item, "Kernel
 * Optimization and Load Balancing": routing moves data whose sizes are not
 * static, so bad sizes and indices surface on the device, not the host.)
 */
enum moe_device_error {
  MOE_DEVERR_EXPERT_INDEX = 1,  /* moe_permute: a topk_idx outside [0, E);
                                   its slot was dropped (inv = -1)      */
  MOE_DEVERR_ROWS = 2,          /* grouped GEMMs: offsets decrease or run
                                   past R_cap; rows at or past R_cap were
                                   not computed                          */
  MOE_DEVERR_WAIT = 4           /* moe_grouped_ffn_fused: a down tile
                                   stopped waiting for its expert's a
                                   (a bound of 0.2 s; not expected)      */
};

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
 * Non-finite logits: -0 equals +0; NaN ranks below every number (-inf
 * included), so every token gets k distinct indices in [0, E).  With l_max
 * finite, NaN and -inf logits weigh 0; with l_max = +inf the +inf logits
 * share the weight equally; with l_max = -inf or NaN the k kept experts
 * share it equally.
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
 * Inputs:  topk_idx [T, k] int32 with values in [0, E); topk_w [T, k] fp32
 *          or NULL; x [T, H] of dtype or NULL (then x_perm is not written).
 *          E is the number of experts of the layer; this GPU's experts
 *          [e_begin, e_begin + n_local) must lie inside [0, E).
 * Outputs: counts [n_local], offsets [n_local + 1] (exclusive scan,
 *          offsets[n_local] = R, the rows this GPU computes),
 *          row_src [T*k] (rows < R: the flat slot placed there),
 *          inv [T, k] (row of slot f, or -1 when its expert is not local),
 *          x_perm [T*k, H] (rows < R: x_perm[r] = x[row_src[r] / k]),
 *          s_perm [T*k] fp32 (rows < R: topk_w of that slot; skipped when
 *          topk_w is NULL or s_perm is NULL).
 * Rows >= R of the capacity-sized outputs are left untouched.
 * Indices outside [e_begin, e_begin + n_local) are non-local: dropped.  An
 * index outside [0, E) is dropped too and sets MOE_DEVERR_EXPERT_INDEX in
 * the workspace's error word (which the call otherwise clears): nothing is
 * ever written out of bounds.
 * workspace: moe_permute_workspace_bytes(T, k, n_local) bytes, 16-aligned.
 * Limits: 1 <= k <= 32, T*k < 2^31, 1 <= n_local <= 4096,
 * 0 <= e_begin <= E - n_local, E < 2^31, H % 8 == 0 when x is given (bf16)
 * or H % 4 == 0 (fp32).
 */
size_t moe_permute_workspace_bytes(int64_t T, int64_t k, int64_t n_local);
int moe_permute(const int32_t *topk_idx, const float *topk_w, const void *x,
                int64_t T, int64_t k, int64_t H, int dtype, int64_t E,
                int64_t e_begin, int64_t n_local, void *x_perm, float *s_perm,
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
 * offsets [n_local + 1] (device) must satisfy 0 <= offsets[e] <=
 * offsets[e+1] <= R_cap.  Segments that break this are cut to fit: expert e
 * then computes rows [b, max(b, min(offsets[e+1], R_cap))) with b =
 * min(max(offsets[e], 0), R_cap), so rows at or past R_cap are never read or
 * written (rows two cut segments share hold unspecified values), and
 * MOE_DEVERR_ROWS is set in the workspace's error word, which the call
 * otherwise clears.
 * bf16: experts with more than 64 rows run on 128-row tiles; when those are
 * too few to fill the chip (a few experts of a few hundred rows) the call
 * splits K into 2-4 ranges per tile and adds the fp32 partials (in a fixed
 * order: repeated calls give identical bits; a different split, as the per
 * expert loop may choose, rounds differently).
 * The order in which tiles run never changes a tile's result; launches with
 * many tiles per compute unit hand them out through per-XCD claim counters
 * held in the workspace, so calls that share a workspace must not overlap.
 * workspace: moe_grouped_ffn_workspace_bytes(...) bytes, 16-aligned: the
 * tile plan and claim counters plus, for R_cap > 64, the split-K partial
 * sums (up to 512 slots of 128 KiB: 64 MiB, fewer when R_cap, H and I allow
 * fewer tiles).
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
 * [R_cap, I] (dtype) is the one intermediate handed between them.  For bf16
 * one plan kernel sizes both GEMMs' tile lists from the offsets (instead of
 * one per call); the two grouped launches, their K splits and their output
 * bits are those of the two calls.
 */
int moe_grouped_ffn(const void *x_perm, const int32_t *offsets,
                    const float *s_perm, int64_t n_local, int64_t R_cap,
                    int64_t H, int64_t I, const void *w_gate,
                    const void *w_up, const void *w_down, int dtype, void *a,
                    void *y, void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * moe_grouped_ffn_gather - moe_grouped_ffn with the gate/up GEMM reading
 * the token rows x [T, H] through row_src (permuted row r is
 * x[row_src[r] / k]), as moe_grouped_gate_up_gather does: the permuted copy
 * x_perm is never written.  Wide-EP explainer, 前提条件 (dispatch sends each
 * token row to the experts it chose); the gather is folded into the GEMM's
 * loads.  Outputs a, y, the error word, workspace and limits as
 * moe_grouped_ffn, with T, k and R_cap <= T * k as for
 * moe_grouped_gate_up_gather.  bf16 only (MOE_E_UNSUPPORTED otherwise).
 * Same bits as moe_grouped_gate_up_gather followed by moe_grouped_down.
 */
int moe_grouped_ffn_gather(const void *x, const int32_t *row_src, int64_t T,
                           int64_t k, const int32_t *offsets,
                           const float *s_perm, int64_t n_local,
                           int64_t R_cap, int64_t H, int64_t I,
                           const void *w_gate, const void *w_up,
                           const void *w_down, int dtype, void *a, void *y,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * moe_grouped_ffn_fused - the computation of moe_grouped_ffn (bf16) in one
 * persistent launch after a one-block plan kernel.  BioNeMo MoE article,
 * "GroupedLinear Optimizes Expert Computation in MoE Models": all experts
 * in one operation and the fused MLP without materialised intermediates.
 * The launch runs the grouped GEMMs' tiles (64 or 128 rows x 256 weight
 * rows, the same K splits): its workgroups claim every gate/up tile, then
 * every down tile, by XCD shares of each phase; a down tile starts once
 * all gate/up tiles of its expert's rows have written their part of a, so
 * one launch replaces the two grouped launches, and the gate/up tail
 * overlaps the down start.  Measured against moe_grouped_ffn (one plan
 * kernel for both GEMMs, rotated K loops): 2% slower on an EP8 share of 7-34
 * rows per expert (0.497 against 0.487 ms), 9% slower on an EP64 share of
 * 116-229 rows (one round of gate/up tiles: nothing to overlap, and the
 * early down tiles wait it out), so moe_grouped_ffn is the default path.
 * x: with row_src non-NULL the token rows [T, H] (permuted row r is
 * x[row_src[r] / k], as moe_grouped_gate_up_gather; R_cap <= T * k); with
 * row_src NULL, x_perm [R_cap, H] (T and k unused).
 * a [R_cap, I] and y [R_cap, H] (bf16): outputs, rows < R, the same bits as
 * moe_grouped_ffn when both choose the same K splits (they use the same
 * rule; the fused call splits only within the workspace both GEMMs share).
 * Deterministic: repeated calls give identical bits.
 * Offsets, s_perm and the cut at R_cap as moe_grouped_gate_up; the error
 * word gets MOE_DEVERR_ROWS as there, and MOE_DEVERR_WAIT if a down tile
 * gave up waiting (its rows of y are then unspecified).
 * workspace: moe_grouped_ffn_workspace_bytes(...) bytes, 16-aligned.
 * Limits: dtype MOE_DT_BF16 (MOE_E_UNSUPPORTED otherwise), others as
 * moe_grouped_ffn.
 */
int moe_grouped_ffn_fused(const void *x, const int32_t *row_src, int64_t T,
                          int64_t k, const int32_t *offsets,
                          const float *s_perm, int64_t n_local, int64_t R_cap,
                          int64_t H, int64_t I, const void *w_gate,
                          const void *w_up, const void *w_down, int dtype,
                          void *a, void *y, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn_loop - the computation of moe_grouped_ffn (bf16 only;
 * identical bits unless the two calls split K differently) issued the way the pages' baseline does it: expert by
 * expert, each expert's gate/up and down as launches of their own (BioNeMo
 * MoE article, "GroupedLinear Optimizes Expert Computation in MoE Models":
 * iterating over the experts with a separate launch for each is what the
 * grouped operation replaces).  It exists to measure that difference.  A
 * per-expert loop needs the row counts on the host: host_counts [n_local]
 * (host memory) must equal the device counts (offsets[e+1] - offsets[e]);
 * experts with no rows get no launch.  Other arguments, workspace and
 * limits as for moe_grouped_ffn.  MOE_E_SHAPE if sum(host_counts) > R_cap.
 */
int moe_grouped_ffn_loop(const void *x_perm, const int32_t *offsets,
                         const int32_t *host_counts, const float *s_perm,
                         int64_t n_local, int64_t R_cap, int64_t H, int64_t I,
                         const void *w_gate, const void *w_up,
                         const void *w_down, int dtype, void *a, void *y,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * ---- Expert-parallel load balancing ("Wide-EPとは?" explainer, section
 * 負荷の偏り:EPLB: expert loads are skewed, and a GPU holding the hot
 * experts becomes the bottleneck while the others idle; between forward
 * passes the balancer looks at each expert's load, rearranges the placement
 * and gives the heaviest experts copies on several GPUs.  The pages give no
 * algorithm; the rule taken is stated below.)
 *
 * moe_eplb_plan - a placement of E experts on n_slots physical slots (one
 * expert copy each) over n_ranks ranks of n_slots / n_ranks slots, from
 * observed per-expert loads counts [E] (device; e.g. the counts of an
 * earlier moe_permute over all experts; negative counts read as 0):
 *   1. every expert gets one copy; each of the n_slots - E spare slots goes
 *      to the expert with the largest load per copy, counts[e] / copies
 *      (ties: lower expert);
 *   2. copy i of r copies of an expert with n rows is expected to take
 *      floor((i+1) n / r) - floor(i n / r) rows;
 *   3. copies are placed in order of decreasing expected rows (ties: lower
 *      expert, then lower copy), each on the rank with the smallest expected
 *      load so far among those with a free slot that do not yet hold that
 *      expert (if every rank with a free slot holds it: among those with a
 *      free slot; ties: lower rank);
 *   4. rank g owns slots [g S/G, (g+1) S/G), in increasing (expert, copy)
 *      order.
 * Outputs (device, int32): rep [E] copies per expert, rep_first [E + 1]
 * prefix of rep, rep_slot [n_slots] the slot of copy i of expert e at
 * rep_first[e] + i, slot_expert / slot_copy [n_slots] the expert and copy
 * index each slot holds.  Integer arithmetic only: deterministic.  One
 * workgroup.
 * Limits: 1 <= E <= 1024, E <= n_slots <= 4096, 1 <= n_ranks <= 1024,
 * n_slots % n_ranks == 0.
 */
int moe_eplb_plan(const int32_t *counts, int64_t E, int64_t n_slots,
                  int64_t n_ranks, int32_t *rep, int32_t *rep_first,
                  int32_t *rep_slot, int32_t *slot_expert, int32_t *slot_copy,
                  hipStream_t stream);

/*
 * moe_permute_replicated - moe_permute onto this rank's slots [s_begin,
 * s_begin + n_slots) of a plan, for the current routing topk_idx [T, k]:
 * with n_e the current number of entries routed to expert e, copy i of its r
 * copies takes the entries at positions [floor(i n_e / r), floor((i+1) n_e /
 * r)) among e's entries in ascending flat order f = t*k + j (a hot expert's
 * rows are split evenly among its copies); inside a slot entries keep
 * ascending f.  Outputs as moe_permute with the local slots in place of the
 * local experts: counts [n_slots], offsets [n_slots + 1], row_src, inv
 * (-1 for entries of other ranks' slots), x_perm, s_perm (topk_w of each row;
 * required when topk_w is given).  Indices outside [0, E) are dropped and set
 * MOE_DEVERR_EXPERT_INDEX in the workspace's error word.
 * rep_first, rep_slot, slot_expert, slot_copy: a plan of moe_eplb_plan for
 * E experts on S slots; 0 <= s_begin <= S - n_slots.
 * workspace: moe_permute_replicated_workspace_bytes(T, k, E, n_slots).
 * Limits: T >= 1, 1 <= k <= 32, T*k < 2^31, E <= S <= 4096, H as for
 * moe_permute.
 */
size_t moe_permute_replicated_workspace_bytes(int64_t T, int64_t k, int64_t E,
                                              int64_t n_slots);
int moe_permute_replicated(const int32_t *topk_idx, const float *topk_w,
                           const void *x, int64_t T, int64_t k, int64_t H,
                           int dtype, int64_t E, int64_t S,
                           const int32_t *rep_first, const int32_t *rep_slot,
                           const int32_t *slot_expert,
                           const int32_t *slot_copy, int64_t s_begin,
                           int64_t n_slots, void *x_perm, float *s_perm,
                           int32_t *row_src, int32_t *inv, int32_t *counts,
                           int32_t *offsets, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_ffn_slots - moe_grouped_ffn over slots whose weights are
 * looked up per slot: slot g (rows [offsets[g], offsets[g+1])) uses the
 * stacked weights of expert slot_expert[g] (device int32 [n_slots], values
 * in [0, n_experts); out-of-range values are clamped and set
 * MOE_DEVERR_EXPERT_INDEX).  The copies of one expert on a rank share its
 * weights.  bf16 only.  Workspace: moe_grouped_ffn_workspace_bytes(R_cap,
 * n_slots, H, I, dtype).  Other arguments as for moe_grouped_ffn.
 */
int moe_grouped_ffn_slots(const void *x_perm, const int32_t *offsets,
                          const float *s_perm, int64_t n_slots,
                          const int32_t *slot_expert, int64_t n_experts,
                          int64_t R_cap, int64_t H, int64_t I,
                          const void *w_gate, const void *w_up,
                          const void *w_down, int dtype, void *a, void *y,
                          void *workspace, size_t workspace_bytes,
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
 * MX element formats.  Every MXFP8 operand is E4M3 (the OCP FP8 "FN"
 * format, largest finite 448, shared exponent floor(log2 amax) - 8) except
 * that the backward entry points can take their gradient operands (dY, dg,
 * du) in E5M2 (OCP FP8 E5M2, largest finite 57344, shared exponent
 * floor(log2 amax) - 15), whose wider range suits gradients.  The pages fix
 * neither; E4M3 everywhere is the default reading.
 */
enum moe_mx_format { MOE_MX_E4M3 = 0, MOE_MX_E5M2 = 1 };

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
 * format: element format (moe_mx_format; MOE_E_ARG otherwise).
 * Codes and scales of a given input match the rule above bit for bit.
 */
int moe_mxfp8_quantize(const void *in, int64_t rows, int64_t cols,
                       int64_t ld_in, int axis, int format,
                       const int32_t *seg_offsets, int64_t n_seg,
                       int64_t align, uint8_t *codes, int64_t ld_codes,
                       uint8_t *scales, int64_t ld_scales,
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
 * Outputs: a [R_cap, I] bf16; gu [R_cap, 2I] fp32 = [g | u] per row (may
 * be NULL; the backward needs it: the saved pre-activations stay in fp32, so
 * the backward differentiates at the values the forward computed); y
 * [R_cap, H] bf16.  Rows < R are written.
 * The SwiGLU epilogue also writes MX(a) (blocks along I) into the workspace,
 * encoded from the fp32 a before any rounding (quantisation, SwiGLU and the
 * routing scale in one kernel: the MXFP8 section), and the down projection
 * reads those codes; the bf16 `a` output is the same fp32 a rounded.
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
                              float *gu, void *y, void *workspace,
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
 * Inputs: dy [R_cap, H] and x_perm [R_cap, H] (bf16), gu [R_cap, 2I] (fp32,
 * from the forward); offsets, s_perm; the weights quantised along the
 * other axis (axis 1 of the stacked weights): wdt/wdts = W_down as [n_local*H,
 * I] -> codes [I, n_local*H], scales [I, n_local*H/32]; wgt/wgts, wut/wuts =
 * W_gate, W_up as [n_local*I, H] -> codes [H, n_local*I], scales [H,
 * n_local*I/32].
 * Outputs: dx [R_cap, H] bf16, ds [R_cap] fp32 (sum in a fixed order),
 * dw_gate, dw_up [n_local, I, H] bf16, dw_down [n_local, H, I] bf16 (an
 * expert without rows gets zero gradients).
 * a = s SiLU(g) u, dg and du are computed in fp32 in the epilogue of the da
 * GEMM, which writes their MX codes (a: down each expert's rows, for dW_d;
 * dg, du: along 2I for dX and down each expert's rows for dW_g, dW_u)
 * encoded from those fp32 values: no tensor of the chain is rounded to bf16
 * before it is quantised.
 * grad_format: element format of the gradient operands dY, dg and du in
 * every GEMM above (moe_mx_format); weights, x and a stay E4M3.
 * workspace: moe_grouped_mlp_mxfp8_bwd_workspace_bytes() bytes.
 * Limits as for the forward; MOE_E_ARG for an unknown grad_format.
 */
size_t moe_grouped_mlp_mxfp8_bwd_workspace_bytes(int64_t R_cap,
                                                 int64_t n_local, int64_t H,
                                                 int64_t I);
int moe_grouped_mlp_mxfp8_bwd(
    const void *dy, const void *x_perm, const float *gu,
    const int32_t *offsets, const float *s_perm, int64_t n_local,
    int64_t R_cap, int64_t H, int64_t I, const uint8_t *wdt,
    const uint8_t *wdts, const uint8_t *wgt, const uint8_t *wgts,
    const uint8_t *wut, const uint8_t *wuts, void *dx, float *ds,
    void *dw_gate, void *dw_up, void *dw_down, int grad_format,
    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_grouped_mlp_mxfp8_bwd_down - first half of the backward: the down
 * projection's data and weight gradients and the ScaledSwiGLU backward.
 *   da = MX(dY) . MX_H(W_down);  dg, du, ds as above;
 *   dW_down[e] = MX_R(dY_e)^T . MX_R(a_e)
 * Inputs: dy [R_cap, H] bf16, gu [R_cap, 2I] fp32, offsets, s_perm (may be
 * NULL: s = 1), wdt/wdts as for moe_grouped_mlp_mxfp8_bwd.
 * Outputs: dgu [R_cap, 2I] bf16 = [dg | du] per row (the fp32 values
 * rounded: this stage API hands [dg | du] on in bf16, and
 * moe_grouped_mlp_mxfp8_bwd_gate_up quantises that bf16 tensor), ds [R_cap]
 * fp32, dw_down [n_local, H, I] bf16.  dW_d uses a recomputed in fp32 from
 * gu, as in moe_grouped_mlp_mxfp8_bwd.  grad_format: element format of dY
 * (as for moe_grouped_mlp_mxfp8_bwd).
 * workspace: moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes() bytes.
 */
size_t moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes(int64_t R_cap,
                                                      int64_t n_local,
                                                      int64_t H, int64_t I);
int moe_grouped_mlp_mxfp8_bwd_down(
    const void *dy, const float *gu, const int32_t *offsets,
    const float *s_perm, int64_t n_local, int64_t R_cap, int64_t H, int64_t I,
    const uint8_t *wdt, const uint8_t *wdts, void *dgu, float *ds,
    void *dw_down, int grad_format, void *workspace, size_t workspace_bytes,
    hipStream_t stream);

/*
 * moe_grouped_mlp_mxfp8_bwd_gate_up - second half of the backward: the
 * gate/up projection's data and weight gradients from [dg | du].
 *   dX = MX(dg) . MX_I(W_gate) + MX(du) . MX_I(W_up);
 *   dW_gate[e] = MX_R(dg_e)^T . MX_R(x_e), dW_up[e] = MX_R(du_e)^T . MX_R(x_e)
 * Inputs: dgu [R_cap, 2I] bf16, x_perm [R_cap, H] bf16, offsets, wgt/wgts,
 * wut/wuts as for moe_grouped_mlp_mxfp8_bwd.  Outputs: dx [R_cap, H],
 * dw_gate, dw_up [n_local, I, H] (bf16).  grad_format: element format of
 * dg and du (as for moe_grouped_mlp_mxfp8_bwd).
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
    void *dw_gate, void *dw_up, int grad_format, void *workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * moe_permute_noalloc - moe_permute without a workspace argument, for
 * callers that cannot allocate device memory: code under stream capture,
 * tight serving loops, harnesses that forbid allocation.  Arguments,
 * outputs, results and limits are those of moe_permute (identical bits).
 * The scratch moe_permute would take from the workspace lives instead in a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES per GPU, held until the
 * process ends; the call itself allocates and frees nothing.  A call whose
 * moe_permute_workspace_bytes(T, k, n_local) exceeds that size returns
 * MOE_E_SCRATCH and enqueues nothing (4 MiB holds, for example, T*k up to
 * 2^20 slots over 256 local experts).  Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams without
 * ordering between them) race and must not be issued.  Nothing in the array
 * has to start at zero: each call rewrites every entry it reads.  The
 * device error word of this variant stays in the array and is not exposed.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int moe_permute_noalloc(const int32_t *topk_idx, const float *topk_w,
                        const void *x, int64_t T, int64_t k, int64_t H,
                        int dtype, int64_t E, int64_t e_begin,
                        int64_t n_local, void *x_perm, float *s_perm,
                        int32_t *row_src, int32_t *inv, int32_t *counts,
                        int32_t *offsets, hipStream_t stream);

/*
 * moe_mxfp8_workspace_view - where the MX codes that a call's GEMMs
 * consumed stay in its workspace after the call, for callers that keep the
 * quantised tensors (reuse, inspection, tests): byte offsets into the
 * workspace and pitches, for the same (R_cap, n_local, H, I) the call took.
 * A view stays valid until the workspace is passed to another call.
 *   call MOE_MXCALL_FWD,      tensor MOE_MXT_A_ROWS: MX(a), blocks along I
 *     (codes [R_cap, I], scales [R_cap, I/32]; rows < R written).
 *   call MOE_MXCALL_BWD_DOWN, tensor MOE_MXT_A_COLS: a = s SiLU(g) u
 *     quantised down each expert's rows (for dW_down): codes [I, cols],
 *     scales [I, cols/32], expert e's rows at columns pad[e] ..
 *     pad[e] + n_e, zero-padded to pad[e+1] (pad: int32 [n_local + 1] at
 *     byte offset `pad`).
 *   call MOE_MXCALL_BWD, tensor MOE_MXT_DGU_ROWS: [dg | du] along 2I
 *     (codes [R_cap, 2I], scales [R_cap, 2I/32]); MOE_MXT_DG_COLS /
 *     MOE_MXT_DU_COLS: dg / du down each expert's rows, laid out as for
 *     MOE_MXT_A_COLS.
 * Other combinations return MOE_E_UNSUPPORTED.  Host only; enqueues nothing.
 */
enum { MOE_MXCALL_FWD = 0, MOE_MXCALL_BWD_DOWN = 1, MOE_MXCALL_BWD = 2 };
enum {
  MOE_MXT_A_ROWS = 0,
  MOE_MXT_A_COLS = 1,
  MOE_MXT_DGU_ROWS = 2,
  MOE_MXT_DG_COLS = 3,
  MOE_MXT_DU_COLS = 4
};
typedef struct moe_mx_view {
  int64_t codes, scales;        /* byte offsets of codes and scales        */
  int64_t ld_codes, ld_scales;  /* row pitches in bytes                    */
  int64_t rows, cols;           /* codes [rows, cols]                      */
  int64_t pad;                  /* byte offset of int32 pad offsets, or -1 */
} moe_mx_view;
int moe_mxfp8_workspace_view(int call, int tensor, int64_t R_cap,
                             int64_t n_local, int64_t H, int64_t I,
                             moe_mx_view *view);

/* Waits for `stream` and reports a pending HIP error as MOE_E_HIP (tests). */
int moe_debug_sync(hipStream_t stream);

/*
 * moe_read_device_error - copy the device error word of `workspace` (a
 * workspace previously passed to a call on `stream`) to *host_code, after
 * waiting for the stream: 0, or an OR of MOE_DEVERR_* bits describing what
 * the last call that used this workspace found on the device.  This call
 * synchronises the stream; it is meant for tests and debugging, not for the
 * hot path.  host_code is a host pointer.  Returns MOE_E_ARG for NULL
 * arguments, MOE_E_HIP when the copy or the wait fails.
 */
int moe_read_device_error(const void *workspace, hipStream_t stream,
                          int32_t *host_code);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
