// Grouped bf16 GEMM on gfx950 MFMA for the expert FFN (and, with one group,
// the router GEMM).
//
// BioNeMo MoE article, "GroupedLinear Optimizes Expert Computation in MoE
// Models": every expert keeps its own weight matrices, yet all experts are
// submitted as one operation; ScaledSwiGLU folds the routing probability into
// the expert FFN and the fused MLP avoids materialising intermediates.  The
// Wide-EP explainer (効果2:演算強度が上がる) gives why: gathering all of an
// expert's tokens into one GEMM reuses each weight byte read from HBM.
//
// Design (a plan kernel, then one launch for all experts):
//   * C[r, n] = sum_k A[r, k] * B_e[n, k] for the rows r of expert e's
//     segment [offsets[e], offsets[e+1]); A and B are K-contiguous bf16.
//   * Work unit = tile of BM rows x BN B-rows of one expert.  A plan kernel
//     turns the device-side offsets into tile prefixes for two classes of
//     experts: those with at most kSmallRows rows (decode-like shares, run
//     with 64-row tiles) and the rest (128-row tiles).  One launch runs both
//     classes' tiles; the host never needs the per-expert counts.  (The FFN
//     can also run as a single launch for both GEMMs: grouped_ffn_kernel at
//     the end of this file.)
//   * Split-K for the 128-row class: when it has too few tiles to fill the
//     chip (a few experts of a few hundred rows: the weight-streaming EP64
//     share), the plan kernel also picks S (2..kSplitMax) and each tile
//     becomes S units over contiguous K ranges.  Every unit stores its fp32
//     accumulators to a slot of the workspace with coherent stores and
//     counts itself in on the tile's counter; the unit that arrives last adds
//     the S partials in fixed K-range order (its own from registers, so the
//     result does not depend on arrival order) and runs the epilogue.  No
//     unit waits for another.
//   * Persistent workgroups, one per compute unit (fewer when there are
//     fewer units of work), read the unit count from the device: XCD x
//     (workgroup id mod 8) takes a contiguous range of units and its
//     workgroups walk it in rounds of consecutive units.  Inside an expert
//     tiles run in bands of 8 m-tiles with the m-tile fastest (banded_mn),
//     so the workgroups of one round share the weight strip and the
//     expert's rows in their L2.
//   * 256 threads = 4 wavefronts in a WM x WN grid; each wavefront owns a
//     (BM/WM) x (BN/WN) sub-tile of 32x32 blocks, v_mfma_f32_32x32x16_bf16
//     with fp32 accumulators.
//   * K advances BK (32 or 64) at a time through a STAGES-deep ring of LDS
//     buffers filled by direct global->LDS loads (global_load_lds_dwordx4, no
//     register staging).  The loads are issued from inline assembly, so the
//     compiler does not serialise them against LDS reads; the kernel waits
//     for them itself: `s_waitcnt vmcnt(n)` for its own loads of the stage
//     about to be used, then a workgroup barrier.  Each lane's global address
//     is chosen so that 16-byte chunks land XOR-swizzled in LDS (conflict-free
//     fragment reads) while every 8 lanes still read one contiguous row piece.
//   * 32-row sub-tiles past the end of an expert's segment are skipped
//     (uniform per wavefront).
//   * A whole tile starts its K loop at a step rotated by its n-tile index
//     (tile_rot), so that concurrent tiles read different columns of their
//     weight rows.
//   * Gather on load (gate/up): A rows may be read straight from the token
//     rows x[row_src[r] / k] instead of a permuted copy.
//   * Epilogues: SWIGLU (B rows alternate 32 gate and the 32 matching up
//     rows, so each lane holds g and u of the same outputs; writes
//     a = s * SiLU(g) * u in bf16), BF16 (plain store) and F32_BIAS (router
//     logits + bias).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

// Workgroups resident and walking the units, one per compute unit (1), or
// one workgroup per unit (0).
#ifndef MOE_GEMM_PERSISTENT
#define MOE_GEMM_PERSISTENT 1
#endif
// Split-K units issue each stage's loads ahead of its MFMAs (1) or spread
// over them as whole tiles do (0).
#ifndef MOE_SPLIT_FRONT
#define MOE_SPLIT_FRONT 1
#endif

namespace moe {

struct GemmArgs {
  const uint16_t *A;        // [rows, K]
  const uint16_t *B0;       // [G, N0, K]: gate / down / router weights
  const uint16_t *B1;       // [G, N0, K]: up weights (SWIGLU only)
  int64_t b_stride;         // elements between experts of B0 / B1
  void *C;                  // output
  int64_t ldc;              // output row stride in elements
  const float *row_scale;   // SWIGLU: per-row routing scale, may be null
  const float *bias;        // F32_BIAS: [N] or null
  const int32_t *offsets;   // [G + 1] row offsets, or null: one group
  const int32_t *tile_prefix;  // [G + 1] tile prefix of this launch's class
  const int32_t *a_rows;    // gather-on-load: A row of permuted row r is
  int a_div, a_rows_max;    //   min(a_rows[r] / a_div, a_rows_max); or null
  int single_rows;          // rows of the single group (offsets == null)
  int r_cap;                // row capacity: segments are cut at it
  const int32_t *group_w;   // weights of group g: stacked expert group_w[g]
  int n_w;                  //   (of n_w, clamped), or g when null
  int G;                    // groups
  int N;                    // output columns (a-columns for SWIGLU)
  int K;
  int NT;                   // n-tiles per m-tile
  const int32_t *split;     // device word: S K-splits per tile, or null: 1
  int32_t *ctr;             // split-K: per-tile arrival counters
  int32_t *claims;          // claim counters of the 8 XCD shares, or null
  float *part;              // split-K: fp32 partial slot of unit u at u*BM*BN
};

// Experts with at most this many rows run on the 64-row-tile kernel.
constexpr int kSmallRows = 64;

// Floats per split-K partial slot of the workspace: one 128 x 256 tile.
constexpr int kSlotFloats = 128 * 256;

// Split-K choice handed from the plan kernel to the GEMM launch.
struct SplitPlan {
  int32_t *word;    // out: S for this launch (1 = no split); null: never split
  int32_t *ctr;     // [slots] per-tile arrival counters, zeroed when S > 1
  int below;        // split only while the 128-row class has fewer tiles
  int P;            // compute units
  int slots;        // partial slots in the workspace: tiles * S <= slots
  int smax;         // largest S
  int KT;           // K steps of the launch: each split gets >= kSplitMinKT
  float part_ratio; // bytes of one partial slot over a tile's weight bytes
};

constexpr int kSplitMinKT = 8;

// K ranges per tile for tw tiles of the large-row class with `cap` partial
// slots free (see gemm_plan_kernel).
__device__ __forceinline__ int choose_split(const SplitPlan &sp, int tw,
                                            int64_t cap) {
  int S = 1;
  if (tw > 0 && tw < sp.below) {
    float best = (float)((tw + sp.P - 1) / sp.P);  // waves at S = 1
    for (int c = 2; c <= sp.smax && c * kSplitMinKT <= sp.KT &&
                    (int64_t)tw * c <= cap;
         ++c) {
      const int waves = (tw * c + sp.P - 1) / sp.P;
      const float f = (float)waves / c * (1.f + (2 * c - 1) * sp.part_ratio);
      if (f < best) {
        best = f;
        S = c;
      }
    }
  }
  return S;
}

// Tile prefixes per row class: prefix_c[e+1] = prefix_c[e] + ceil(rows_e /
// BM_c) * NT_c when expert e belongs to class c.  Experts with at most
// kSmallRows rows form the small class (0), the others the wide class (1).
// With sp.word, S is chosen for the wide class: the S that minimises the
// time in units of one whole tile, ceil(tiles * S / P) / S (waves of units
// over the compute units, each 1/S of a tile), times the tile's bytes grown
// by the split's fp32 traffic (S slots written, S - 1 read back: (2S - 1)
// slots against the tile's weight bytes), the smaller S on ties; S = 1 once
// there are sp.below tiles.  Segments are cut at the row capacity
// r_cap; the error word `err` gets kDevErrRows when the offsets run past it
// or decrease, else 0.  The 8 claim counters (when given) are cleared.  One
// block.
__global__ __launch_bounds__(1024) void gemm_plan_kernel(
    const int32_t *__restrict__ offsets, int G, int r_cap, int32_t *err,
    const int32_t *__restrict__ group_w, int n_w, int bm_small, int nt_small,
    int bm_wide, int nt_wide, int32_t *__restrict__ prefix_small,
    int32_t *__restrict__ prefix_wide, SplitPlan sp, int32_t *claims) {
  __shared__ int32_t wsum[2][16];
  const int tid = threadIdx.x, nth = blockDim.x, nw = nth >> 6;
  if (claims && tid < 8) claims[tid] = 0;
  const int per = (G + nth - 1) / nth;
  const int e0 = min(G, tid * per), e1 = min(G, e0 + per);
  auto tiles = [&](int e, int32_t &t0, int32_t &t1) {
    int b, en;
    seg_rows(offsets, e, r_cap, b, en);
    const int n = en - b;
    t0 = n <= kSmallRows ? (n + bm_small - 1) / bm_small * nt_small : 0;
    t1 = n <= kSmallRows ? 0 : (n + bm_wide - 1) / bm_wide * nt_wide;
  };
  int32_t s[2] = {0, 0};
  int bad = 0;
  for (int e = e0; e < e1; ++e) {
    int32_t t[2];
    tiles(e, t[0], t[1]);
    s[0] += t[0];
    s[1] += t[1];
    bad |= seg_bad(offsets, e, r_cap) ? kDevErrRows : 0;
    if (group_w && (uint32_t)group_w[e] >= (uint32_t)n_w) bad |= kDevErrExpertIndex;
  }
  // Inclusive scan of s over the block: lane shuffles inside each
  // wavefront, then the 16 wavefront totals through LDS (one barrier).
  const int lane = tid & 63, wv = tid >> 6;
  int32_t x[2] = {s[0], s[1]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int32_t y = __shfl_up(x[c], off, 64);
      if (lane >= off) x[c] += y;
    }
  }
  if (lane == 63)
    for (int c = 0; c < 2; ++c) wsum[c][wv] = x[c];
  __syncthreads();
  int32_t r[2], total[2];
  for (int c = 0; c < 2; ++c) {
    int32_t before = 0, all = 0;
    for (int q = 0; q < nw; ++q) {
      const int32_t v = wsum[c][q];
      before += q < wv ? v : 0;
      all += v;
    }
    r[c] = before + x[c] - s[c];
    total[c] = all;
  }
  for (int e = e0; e < e1; ++e) {
    prefix_small[e] = r[0];
    prefix_wide[e] = r[1];
    int32_t t[2];
    tiles(e, t[0], t[1]);
    r[0] += t[0];
    r[1] += t[1];
  }
  if (tid == nth - 1) {
    prefix_small[G] = total[0];
    prefix_wide[G] = total[1];
  }
  if (sp.word) {
    // every thread makes the same choice from the block-wide total
    const int tw = total[1];
    const int S = choose_split(sp, tw, sp.slots);
    if (tid == 0) *sp.word = S;
    if (S > 1)
      for (int i = tid; i < tw; i += nth) sp.ctr[i] = 0;
  }
  // OR of the error bits over the block
  __shared__ int32_t bad_or;
  if (tid == 0) bad_or = 0;
  __syncthreads();
  if (bad) atomicOr(&bad_or, bad);
  __syncthreads();
  if (tid == 0) *err = bad_or;
}

// Wait until at most N of this wavefront's vector-memory loads are in flight
// and its LDS reads are done, then join the workgroup barrier.  The "memory"
// clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
               :: "i"(N) : "memory");
}

// Direct global -> LDS load of 16 bytes per lane: lane l's data goes to LDS
// byte address lds_base + 16 * l (lds_base uniform over the wavefront).
__device__ __forceinline__ void load_lds16(uint32_t lds_base, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory");
}

// Physical 16-byte chunk of logical chunk c of LDS row `row` (CPR chunks per
// row).  A ds_read_b128 serves 16 lanes (256 bytes of banks) at a time, and
// the fragment reads put 16 consecutive rows at one logical chunk in such a
// group: with 128-byte rows, rows of equal parity must get distinct chunks
// (c ^ (row/2 % 8)); with 64-byte rows, rows equal mod 4 must
// (c ^ (row/4 % 4)).  Either way the 16 reads cover all 16 bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  return CPR == 8 ? (c ^ ((row >> 1) & 7)) : (c ^ ((row >> 2) & 3));
}

// K steps of a whole tile may start at step rot (then wrap): K step ks of
// the loop reads step (ks + rot) mod KT, with rot = n-tile mod KT.
// Workgroups that start together and stream weights at the same rate would
// otherwise read the same 128-byte column of every weight row at the same
// time; with rows a power of two bytes apart (4 KiB at K = 2048, the down
// projection) those reads fall on the same few HBM channels.  Measured on
// the EP8 share (32 experts of 7-34 rows, weight-streaming): the down
// projection replayed in a graph 196 -> 172 us with a stride of 5 steps per
// n-tile; a stride of 1 (neighbouring n-tiles one step apart) took the step
// another 0.9% lower (strides 3, 7, 11, 13 and ones that add the expert
// index measured like 5; the full layer and the EP64 share did not move).
// The rotation depends only
// on the tile's n-tile and K, so every path that runs a tile whole sums in
// the same order (bit-equal results across the grouped, per-expert-loop and
// one-launch paths); split-K units are not rotated.
#ifndef MOE_KROT
#define MOE_KROT 1
#endif
__device__ __forceinline__ int rot_step(int ks, int rot, int KT) {
  const int r = ks + rot;
  return r >= KT ? r - KT : r;
}
__device__ __forceinline__ int tile_rot(int nt, int KT) {
  return MOE_KROT ? nt % KT : 0;
}

// Load the A and B fragments of k-substep kk (16 values of K) from one LDS
// stage: lane holds row (lane & 31) of each 32-row block, K chunk
// 2*kk + lane/32.
template <int CPR, int MV, int NB>
__device__ __forceinline__ void load_frags(const uint4 *As, const uint4 *Bs,
                                           int kk, int lane, int arow0,
                                           int brow0, bf16x8 (&af)[MV],
                                           bf16x8 (&bf)[NB]) {
  const int ch = 2 * kk + (lane >> 5);
#pragma unroll
  for (int m = 0; m < MV; ++m) {
    const int row = arow0 + m * 32 + (lane & 31);
    const uint4 v = As[row * CPR + swz<CPR>(row, ch)];
    af[m] = *(const bf16x8 *)&v;
  }
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int row = brow0 + n * 32 + (lane & 31);
    const uint4 v = Bs[row * CPR + swz<CPR>(row, ch)];
    bf[n] = *(const bf16x8 *)&v;
  }
}

// The K loop of one tile for a wavefront with MV valid 32-row blocks.
// Stages 0 .. STAGES-2 have been issued by the caller; every iteration
// issues one more (clamped to the last stage at the tail, a harmless
// re-read that keeps (STAGES-2)*L loads in flight at every wait).  The
// stage's L loads are spread over its MFMAs (scheduling barriers keep them
// there) instead of being issued in one burst, so the vector-memory queue
// never stalls the matrix work; fragment reads of k-substep kk+1 are issued
// before the MFMAs of kk.  The loop body has no data-dependent branches.
// Loop step ks reads K step rot_step(ks, rot, KT) (see tile_rot).
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int MV,
          bool FRONT>
__device__ __forceinline__ void gemm_kloop(
    f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
    const char *const (&gsrc)[(BM + BN) * (BK / 8) / (WM * WN * 64)],
    const uint4 *smem, uint32_t lds0, uint32_t wave_off, int KT, int lane,
    int arow0, int brow0, int rot = 0) {
  constexpr int CPR = BK / 8, NB = BN / WN / 32, KK = BK / 16;
  constexpr int STAGE_CHUNKS = (BM + BN) * CPR;
  constexpr int L = STAGE_CHUNKS / (WM * WN * 64);
  constexpr int NMF = MV * NB * KK;
  for (int kt = 0; kt < KT; ++kt) {
    wait_loads_barrier<(STAGES - 2) * L>();
    // Loads of stage kt + STAGES - 1 (clamped to the last stage at the tail:
    // the re-read is harmless and keeps the in-flight count fixed).
    const int ks = min(kt + STAGES - 1, KT - 1);
    const int st = (kt + STAGES - 1) % STAGES;
    const uint32_t sb = lds0 + (uint32_t)(st * STAGE_CHUNKS * 16) + wave_off;
    const int64_t koff = (int64_t)rot_step(ks, rot, KT) * (BK * 2);
    if constexpr (FRONT || MV == 0) {
#pragma unroll
      for (int i = 0; i < L; ++i)
        load_lds16(sb + (uint32_t)(i * 64 * 16), gsrc[i] + koff);
    }
    if constexpr (MV > 0) {
      const uint4 *As = smem + (kt % STAGES) * STAGE_CHUNKS;
      const uint4 *Bs = As + BM * CPR;
      bf16x8 a0[MV], b0[NB], a1[MV], b1[NB];
      load_frags<CPR, MV, NB>(As, Bs, 0, lane, arow0, brow0, a0, b0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          if (kk & 1) load_frags<CPR, MV, NB>(As, Bs, kk + 1, lane, arow0, brow0, a0, b0);
          else load_frags<CPR, MV, NB>(As, Bs, kk + 1, lane, arow0, brow0, a1, b1);
        }
#pragma unroll
        for (int m = 0; m < MV; ++m)
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                (kk & 1) ? a1[m] : a0[m], (kk & 1) ? b1[n] : b0[n], acc[m][n],
                0, 0, 0);
            if constexpr (!FRONT) {
              const int f = (kk * MV + m) * NB + n;
#pragma unroll
              for (int i = f * L / NMF; i < (f + 1) * L / NMF; ++i) {
                __builtin_amdgcn_sched_barrier(0);
                load_lds16(sb + (uint32_t)(i * 64 * 16), gsrc[i] + koff);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
      }
    }
  }
  wait_loads_barrier<0>();
}

// Split-K hand-over of one unit: K range ks of S of a tile whose units own
// the workspace slots slot0 .. slot0 + S - 1 (kSlotFloats floats apart) and
// the arrival counter ctr[ci].  Every unit stores its accumulators (the
// wavefront's valid 32-row blocks) to its slot with coherent stores, waits
// for them, and counts itself in; the unit that counts last returns true
// after replacing acc with the sum of the S partials taken in ks order (its
// own from registers).  The others return false.  Layout inside a slot: per
// wavefront, block (m, n), quarter q of the 16 accumulator values, half h
// of the quarter, lane: 8 bytes at float (((wid*MB + m)*NB + n)*4 + q)*256
// + h*128 + 2*lane, so each 8-byte store or load instruction covers 512
// contiguous bytes.
template <int MB, int NB>
__device__ __forceinline__ bool split_hand_over(f32x16 (&acc)[MB][NB],
                                                const GemmArgs &p, int slot0,
                                                int ci, int ks, int S, int wid,
                                                int lane, int mvalid,
                                                int *s_last) {
  static_assert(4 * MB * NB * 1024 <= kSlotFloats, "a slot holds the tile");
  {
    float *mine = p.part + (int64_t)(slot0 + ks) * kSlotFloats;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m >= mvalid) continue;
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float *d = mine + (((wid * MB + m) * NB + n) * 4 + q) * 256 + lane * 2;
          uint64_t lo, hi;
          const float v[4] = {acc[m][n][4 * q], acc[m][n][4 * q + 1],
                              acc[m][n][4 * q + 2], acc[m][n][4 * q + 3]};
          __builtin_memcpy(&lo, v, 8);
          __builtin_memcpy(&hi, v + 2, 8);
          store_coherent8(d, lo);
          store_coherent8(d + 128, hi);
        }
    }
  }
  wait_vmem();
  __syncthreads();
  if (wid == 0 && lane == 0) {
    // one atomic; its old value is the arrival number
    const int old = __hip_atomic_fetch_add(p.ctr + ci, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    *s_last = old == S - 1;
    // every unit of the tile has counted in: the counter goes back to zero
    // for a later launch that reuses it (the two launches of the grouped FFN)
    if (old == S - 1)
      __hip_atomic_store(p.ctr + ci, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(*s_last)) return false;
  const float *slots = p.part + (int64_t)slot0 * kSlotFloats;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= mvalid) continue;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      f32x16 sum;
      for (int j = 0; j < S; ++j) {
        f32x16 v;
        if (j == ks) {
          v = acc[m][n];
        } else {
          const float *src = slots + (int64_t)j * kSlotFloats;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float *d = src + (((wid * MB + m) * NB + n) * 4 + q) * 256 + lane * 2;
            const uint64_t lo = load_coherent8(d), hi = load_coherent8(d + 128);
            float w[4];
            __builtin_memcpy(w, &lo, 8);
            __builtin_memcpy(w + 2, &hi, 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 * q + i] = w[i];
          }
        }
        if (j == 0) sum = v;
        else
#pragma unroll
          for (int i = 0; i < 16; ++i) sum[i] += v[i];
      }
      acc[m][n] = sum;
    }
  }
  return true;
}

// Epilogue of one wavefront's WTM x WTN part of a tile (rows wrow0 ..
// of the tile, B-rows wn*WTN .. of its BN).  Lane holds column (lane & 31)
// of each 32x32 block and rows 8*(r/4) + 4*(lane/32) + (r%4), r < 16.  bf16
// outputs are staged in a per-wavefront LDS region (smem must be free) and
// leave as 16-byte row pieces.
// The routing-weight scale of each accumulator row of this lane (the
// SwiGLU epilogue's s), 1 where there is none: all of them loaded at once,
// ahead of the epilogue's arithmetic, instead of one load and one wait per
// row inside it.
template <int MB>
__device__ __forceinline__ void load_row_scales(const GemmArgs &p, int row0,
                                                int wrow0, int rows, int lane,
                                                int mvalid,
                                                float (&sc)[MB][16]) {
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = wrow0 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      sc[m][r] = (m < mvalid && i < rows && p.row_scale) ? p.row_scale[row0 + i] : 1.f;
    }
}

// sc: the rows' routing scales (SWIGLU; load_row_scales), unused otherwise.
template <int EPI, int BN, int MB, int NB, int WTM, int WTN>
__device__ __forceinline__ void tile_epilogue(f32x16 (&acc)[MB][NB],
                                              const GemmArgs &p, uint4 *smem,
                                              int wid, int wn, int lane,
                                              int mvalid, int nt, int row0,
                                              int wrow0, int rows,
                                              int32_t *dep, int di,
                                              const float (&sc)[MB][16]) {
  if (EPI == EPI_SWIGLU) {
    // B rows alternate 32 gate rows and the 32 matching up rows, so block
    // 2q holds g and block 2q+1 holds u of the same outputs in every lane.
    constexpr int W = WTN / 2;
    uint16_t *lw = (uint16_t *)smem + (size_t)wid * (WTM * W);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m >= mvalid) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rw = m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float s = sc[m][r];
#pragma unroll
        for (int q = 0; q < NB / 2; ++q) {
          const float g = acc[m][2 * q][r], u = acc[m][2 * q + 1][r];
          lw[rw * W + st_col<W>(rw, q * 32 + (lane & 31))] =
              (uint16_t)f32_to_bf16_bits(s * silu_f32(g) * u);
        }
      }
    }
    __syncthreads();
    if (dep == nullptr) {
      store_staged<W, WTM>(lw, (uint16_t *)p.C, p.ldc,
                           (int64_t)nt * (BN / 2) + wn * W, p.N, row0 + wrow0,
                           wrow0, rows, lane);
    } else {
      // a for other workgroups of this launch: coherent stores, waited for,
      // then the tile counts in
      store_staged_coherent<W, WTM>(lw, (uint16_t *)p.C, p.ldc,
                                    (int64_t)nt * (BN / 2) + wn * W, p.N,
                                    row0 + wrow0, wrow0, rows, lane);
      wait_vmem();
      __syncthreads();
      if (wid == 0 && lane == 0)
        __hip_atomic_fetch_add(dep + di, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (EPI == EPI_BF16) {
    uint16_t *lw = (uint16_t *)smem + (size_t)wid * (WTM * WTN);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m >= mvalid) continue;
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rw = m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          lw[rw * WTN + st_col<WTN>(rw, n * 32 + (lane & 31))] =
              (uint16_t)f32_to_bf16_bits(acc[m][n][r]);
        }
    }
    __syncthreads();
    store_staged<WTN, WTM>(lw, (uint16_t *)p.C, p.ldc,
                           (int64_t)nt * BN + wn * WTN, p.N, row0 + wrow0,
                           wrow0, rows, lane);
  } else {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m >= mvalid) continue;
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = wrow0 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = nt * BN + wn * WTN + n * 32 + (lane & 31);
          if (i < rows && col < p.N)
            ((float *)p.C)[(int64_t)(row0 + i) * p.ldc + col] =
                acc[m][n][r] + (p.bias ? p.bias[col] : 0.f);
        }
    }
  }
}

// Static shape facts of one tile configuration.
template <int BM, int BN, int WM, int WN, int BK, int STAGES>
struct TileCfg {
  static constexpr int NTH = WM * WN * 64;           // 4 or 8 wavefronts
  static constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MB = WTM / 32, NB = WTN / 32;
  static constexpr int STAGE_CHUNKS = (BM + BN) * CPR;
  static constexpr int L = STAGE_CHUNKS / NTH;       // loads per thread per stage
  static constexpr int RING = STAGES * STAGE_CHUNKS; // 16-byte LDS chunks
  static_assert(WM * WN == 4 || WM * WN == 8, "four or eight wavefronts");
  static_assert(MB >= 1 && NB >= 1, "wave tile is a multiple of 32x32");
  static_assert(BM * CPR % NTH == 0 && BN * CPR % NTH == 0, "load split");
  static_assert(STAGES * STAGE_CHUNKS * 16 >= WM * WN * WTM * WTN * 2,
                "the ring must hold every wavefront's epilogue region");
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(STAGES >= 2 && STAGES <= 6 && (STAGES - 2) * L <= 63,
                "vmcnt range");
};

// Tile t of a launch's class (BM-row tiles): its expert e, m-tile mt,
// n-tile nt and rows [row0, row0 + rows).
template <int BM>
__device__ __forceinline__ void tile_coords(const GemmArgs &p, int t, int &e,
                                            int &mt, int &nt, int &row0,
                                            int &rows) {
  int r_begin, r_end, local;
  if (p.offsets) {
    e = upper_bound_minus1(p.tile_prefix, p.G, t);
    seg_rows(p.offsets, e, p.r_cap, r_begin, r_end);
    local = t - p.tile_prefix[e];
  } else {
    e = 0; r_begin = 0; r_end = p.single_rows; local = t;
  }
  const int mtiles = (r_end - r_begin + BM - 1) / BM;
  banded_mn(local, mtiles, p.NT, 8, mt, nt);
  row0 = r_begin + mt * BM;
  rows = min(BM, r_end - row0);
}

// Global source of each of this thread's L loads per stage of tile t (K
// range starting at step kt0), and the tile's coordinates.  The stage is
// cut into groups of 64 chunks (one load instruction each); wavefront w
// issues groups [w*L, w*L + L), so with BM == BN two wavefronts load only A
// rows (mostly L2 hits) and two only B rows (weight stream): a wavefront's
// loads return in order, and this keeps the quick hits out of the queue
// behind slow misses.  Chunk q = (w*L + i)*64 + lane.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int EPI>
__device__ __forceinline__ void tile_sources(
    const GemmArgs &p, int t, int kt0, int wid, int lane,
    const char *(&gsrc)[TileCfg<BM, BN, WM, WN, BK, STAGES>::L], int &e,
    int &mt, int &nt, int &row0, int &rows) {
  using C = TileCfg<BM, BN, WM, WN, BK, STAGES>;
  constexpr int CPR = C::CPR, L = C::L;
  const int K = p.K;
  tile_coords<BM>(p, t, e, mt, nt, row0, rows);
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int q = (wid * L + i) * 64 + lane;
    const int row = q / CPR;
    if (row < BM) {
      const int kc = swz<CPR>(row, q % CPR);
      int64_t ar = row0 + min(row, rows - 1);
      if (p.a_rows) ar = min(p.a_rows[ar] / p.a_div, p.a_rows_max);
      gsrc[i] = (const char *)(p.A + ar * K + kc * 8);
    } else {
      const int j = row - BM;
      const int kc = swz<CPR>(j, q % CPR);
      const uint16_t *base;
      int col;
      if (EPI == EPI_SWIGLU) {
        const int w = j & 63;
        col = nt * (BN / 2) + (j >> 6) * 32 + (w & 31);
        base = w < 32 ? p.B0 : p.B1;
      } else {
        col = nt * BN + j;
        base = p.B0;
      }
      col = min(col, p.N - 1);
      const int we = p.group_w ? min(max(p.group_w[e], 0), p.n_w - 1) : e;
      gsrc[i] = (const char *)(base + (int64_t)we * p.b_stride + (int64_t)col * K + kc * 8);
    }
    gsrc[i] += (int64_t)kt0 * (BK * 2);
  }
}

// One unit of a launch's class: K range ks of S of tile t; split units
// hand over through slots slot0 .. slot0 + S - 1 and counter ctr[ci].  With
// dep non-null (gate/up inside the fused FFN) the epilogue writes a through
// device-coherent stores and then counts the tile in on dep[di].
// smem: the LDS ring (at least the configuration's RING chunks), free on
// entry; s_last: an LDS word for the split hand-over.
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int EPI>
__device__ __forceinline__ void gemm_unit(const GemmArgs &p, int t, int ks,
                                          int S, int slot0, int ci,
                                          int32_t *dep, int di, uint4 *smem,
                                          int *s_last) {
  using C = TileCfg<BM, BN, WM, WN, BK, STAGES>;
  constexpr int WTM = C::WTM, WTN = C::WTN, MB = C::MB, NB = C::NB,
                STAGE_CHUNKS = C::STAGE_CHUNKS, L = C::L;
  static_assert(EPI != EPI_SWIGLU || NB % 2 == 0,
                "SwiGLU pairs a gate block with the up block next to it");
  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int wm = wid / WN, wn = wid % WN;
  const int KT = p.K / BK;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  const int kt0 = ks * KT / S, KTs = (ks + 1) * KT / S - kt0;
  // The lane index, opaque to the compiler: otherwise, inside the caller's
  // persistent loop, it hoists every lane-dependent LDS address of the unit
  // out of the loop and keeps them all live (register spills).
  int lane;
  asm volatile("; lane index" : "=v"(lane) : "0"(tid & 63));
  int e, mt, nt, row0, rows;
  const char *gsrc[L];
  tile_sources<BM, BN, WM, WN, BK, STAGES, EPI>(p, t, kt0, wid, lane, gsrc, e,
                                                mt, nt, row0, rows);
  const uint32_t wave_off = (uint32_t)(wid * L * 64 * 16);
  const int rot = S == 1 ? tile_rot(nt, KTs) : 0;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  const int wrow0 = wm * WTM;
  const int mvalid = rows > wrow0 ? min(MB, (rows - wrow0 + 31) / 32) : 0;

  const int brow0 = wn * WTN;
  // prologue: stages 0 .. STAGES-2
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) {
    const uint32_t sb = lds0 + (uint32_t)(st * STAGE_CHUNKS * 16) + wave_off;
    const int64_t koff = (int64_t)rot_step(min(st, KTs - 1), rot, KTs) * (BK * 2);
#pragma unroll
    for (int i = 0; i < L; ++i)
      load_lds16(sb + (uint32_t)(i * 64 * 16), gsrc[i] + koff);
  }
  // the K loop, specialised for this wavefront's number of valid blocks
  // (a wavefront with none still keeps the loads and barriers going)
  // Split units stream weights with little MFMA work per step: they issue
  // each stage's loads at once, ahead of the MFMAs, which keeps more bytes
  // in flight; whole tiles spread the loads over the MFMAs.
  const bool front = MOE_SPLIT_FRONT && S > 1;
#define MOE_KLOOP_CASE(mv)                                                    \
    case mv:                                                                \
      if (mv <= MB) {                                                       \
        if (front)                                                          \
          gemm_kloop<BM, BN, WM, WN, BK, STAGES, (mv <= MB ? mv : 1), true>(\
              acc, gsrc, smem, lds0, wave_off, KTs, lane, wrow0, brow0);    \
        else                                                                \
          gemm_kloop<BM, BN, WM, WN, BK, STAGES, (mv <= MB ? mv : 1), false>(\
              acc, gsrc, smem, lds0, wave_off, KTs, lane, wrow0, brow0, rot);\
      }                                                                     \
      break;
  switch (mvalid) {
    MOE_KLOOP_CASE(1)
    MOE_KLOOP_CASE(2)
    MOE_KLOOP_CASE(3)
    MOE_KLOOP_CASE(4)
    default:
      gemm_kloop<BM, BN, WM, WN, BK, STAGES, 0, false>(
          acc, gsrc, smem, lds0, wave_off, KTs, lane, wrow0, brow0, rot);
  }
#undef MOE_KLOOP_CASE
  // every wavefront is done reading the ring before the next tile refills it
  wait_loads_barrier<0>();
  if (S == 1 || split_hand_over<MB, NB>(acc, p, slot0, ci, ks, S, wid, lane,
                                         mvalid, s_last)) {
    float sc[MB][16];
    if constexpr (EPI == EPI_SWIGLU)
      load_row_scales<MB>(p, row0, wrow0, rows, lane, mvalid, sc);
    tile_epilogue<EPI, BN, MB, NB, WTM, WTN>(acc, p, smem, wid, wn, lane,
                                             mvalid, nt, row0, wrow0, rows,
                                             dep, di, sc);
  }
}

// Walk the units [0, units) of a launch: XCD x (workgroups b with b % 8 ==
// x) takes the units [x*per, (x+1)*per) and its nx workgroups walk them in
// rounds of nx consecutive units, so the units that share an expert's rows
// or a weight strip run at the same time behind one L2.  With at least one
// workgroup per unit each does one unit.  Every loop condition is uniform
// over the workgroup.
template <typename F>
__device__ __forceinline__ void walk_units(int units, F &&run) {
  const int nx = gridDim.x >> 3, xcd = blockIdx.x & 7;
  const int per = (units + 7) >> 3;
#pragma nounroll
  for (int r = blockIdx.x >> 3; r < per; r += nx) {
    const int u = xcd * per + r;
    if (u >= units) break;
    __syncthreads();  // the previous unit's epilogue is done with the LDS ring
    run(u);
  }
}

// Claim the units [0, units) of a launch.  The units are cut into 8 shares
// ([z*per, (z+1)*per)), one per XCD.  On XCD x, workgroup j (of nx) starts
// with unit j of share x; after that its workgroups claim the share's
// remaining units in order through the counter claims[x], each claim made
// when the previous unit is done.  Units claimed one after the other
// start at about the same time, so tiles that share a weight strip or an
// expert's rows (consecutive units) stream them behind one L2 together.
// When its share is used up a workgroup reads all 8 counters at once and
// claims from a share that still has units.  Control flow is uniform:
// wavefront 0 claims with one lane's atomic and broadcasts the unit through
// LDS.
#ifndef MOE_CLAIMS
#define MOE_CLAIMS 1
#endif
// Units per workgroup from which a launch claims its units.
constexpr int kClaimRounds = 8;
template <typename F>
__device__ __forceinline__ void claim_units(int units, int32_t *claims,
                                            int *s_unit, F &&run) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nx = gridDim.x >> 3, xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int per = (units + 7) >> 3;
  auto share = [&](int z, int &lo, int &rest) {  // units past the first nx
    lo = min(units, z * per);
    rest = max(0, min(units, lo + per) - lo - nx);
  };
  int own_lo, own_rest;
  share(xcd, own_lo, own_rest);
  const int own_size = min(units, own_lo + per) - own_lo;
  int next = j < own_size ? own_lo + j : -1;
  bool own_done = false;
#pragma nounroll
  for (;;) {
    __syncthreads();  // the previous unit is done with LDS and s_unit
    if (wid == 0) {
      int unit = next;
      next = -1;
      if (unit < 0 && !own_done) {
        int v = 0;
        if (lane == 0)
          v = __hip_atomic_fetch_add(claims + xcd, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        v = __builtin_amdgcn_readfirstlane(v);
        if (v < own_rest) unit = own_lo + nx + v;
        else own_done = true;
      }
      // the own share is used up: claim from another that has units left
      while (unit < 0) {
        int lo = 0, rest = 0, c = 0;
        if (lane < 8) {
          share(lane, lo, rest);
          c = __hip_atomic_load(claims + lane, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint64_t open = __ballot(lane < 8 && c < rest) & 0xffull;
        if (open == 0) break;
        // the first open share after this XCD's, in ring order
        const uint64_t rot = ((open >> xcd) | (open << (8 - xcd))) & 0xffull;
        const int z = (xcd + __builtin_ctzll(rot)) & 7;
        int zlo, zrest;
        share(z, zlo, zrest);
        int v = 0;
        if (lane == 0)
          v = __hip_atomic_fetch_add(claims + z, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        v = __builtin_amdgcn_readfirstlane(v);
        if (v < zrest) unit = zlo + nx + v;
      }
      if (lane == 0) *s_unit = unit < 0 ? units : unit;
    }
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(*s_unit);
    if (u >= units) break;
    run(u);
  }
}

// One class of tiles (the router GEMM: one group, rows p.single_rows).
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ uint4 smem[TileCfg<BM, BN, WM, WN, BK, STAGES>::RING];
  __shared__ int s_last;
  int total;
  if (p.offsets) total = p.tile_prefix[p.G];
  else total = (p.single_rows + BM - 1) / BM * p.NT;
  const int S = p.split ? *p.split : 1;
  walk_units(total * S, [&](int u) {
    const int t = u / S;
    gemm_unit<BM, BN, WM, WN, BK, STAGES, EPI>(p, t, u - t * S, S, t * S, t,
                                               nullptr, 0, smem, &s_last);
  });
}

// Both row classes of a grouped GEMM in one launch: the small-row class's
// tiles (ps, 64 x 256, never split) are units [0, us), the large-row
// class's units (pw, 128 x 256, S K ranges per tile) follow.  One launch
// instead of two saves the launch of whichever class has no tiles.
#ifndef MOE_WIDE_CFG
#define MOE_WIDE_CFG 128, 256, 2, 2, 64, 3
#endif
#ifndef MOE_SMALL_CFG
#define MOE_SMALL_CFG 64, 256, 1, 4, 64, 3
#endif
template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm2_kernel(GemmArgs ps,
                                                            GemmArgs pw) {
  constexpr int RS = TileCfg<MOE_SMALL_CFG>::RING;
  constexpr int RW = TileCfg<MOE_WIDE_CFG>::RING;
  static_assert(TileCfg<MOE_SMALL_CFG>::NTH == 256 &&
                TileCfg<MOE_WIDE_CFG>::NTH == 256, "256 threads");
  __shared__ uint4 smem[RS > RW ? RS : RW];
  __shared__ int s_last, s_unit;
  const int us = ps.tile_prefix[ps.G];
  const int S = pw.split ? *pw.split : 1;
  const int uw = pw.tile_prefix[pw.G] * S;
  auto run = [&](int u) {
    if (u < us) {
      gemm_unit<MOE_SMALL_CFG, EPI>(ps, u, 0, 1, 0, 0, nullptr, 0, smem,
                                    &s_last);
    } else {
      const int t = (u - us) / S;
      gemm_unit<MOE_WIDE_CFG, EPI>(pw, t, u - us - t * S, S, t * S, t,
                                   nullptr, 0, smem, &s_last);
    }
  };
  // Many rounds of units per workgroup: claims (partners stay in step over
  // the rounds); a few: the static walk, which costs no atomics.
  if (MOE_CLAIMS && pw.claims && us + uw >= kClaimRounds * (int)gridDim.x)
    claim_units(us + uw, pw.claims, &s_unit, run);
  else
    walk_units(us + uw, run);
}

namespace {

// BM, BN, WM, WN, BK, STAGES of the large-expert shape: MOE_WIDE_CFG.
constexpr int kWideCfg[6] = {MOE_WIDE_CFG};
constexpr int kWideBM = kWideCfg[0], kWideBN = kWideCfg[1];
constexpr int kSmallCfg[6] = {MOE_SMALL_CFG};
constexpr int kSmallBN = kSmallCfg[1];
static_assert(kSmallCfg[0] == kSmallRows, "the small class is one m-tile");

// Largest K split, and the most partial slots a workspace carries (at
// 128 KiB each: 64 MiB).
#ifndef MOE_SPLITK_MAX
#define MOE_SPLITK_MAX 4
#endif
constexpr int kSplitMax = MOE_SPLITK_MAX;
constexpr int64_t kSplitSlotsMax = 512;
constexpr size_t kSlotBytes = (size_t)kWideBM * kWideBN * 4;

// Threads of a one-block plan kernel over G experts: one per expert, in
// whole wavefronts, at most 1024 (a small launch starts and ends sooner).
unsigned plan_threads(int G) {
  return (unsigned)std::min(1024, std::max(64, (G + 63) / 64 * 64));
}

int ntiles(int N, int BN, bool swiglu) {
  const int cols = swiglu ? BN / 2 : BN;
  return (N + cols - 1) / cols;
}

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

// Partial slots of the workspace: kSplitMax splits of every wide tile that
// rows up to R_cap over n_local experts can give for either GEMM of the FFN
// (gate/up: 128 a-columns per tile; down: 256 output columns), at most
// kSplitSlotsMax.
int64_t split_slots(int64_t n_local, int64_t R_cap, int64_t H, int64_t I) {
  if (R_cap <= kSmallRows) return 0;
  const int64_t mt = (R_cap + kWideBM - 1) / kWideBM + n_local;
  const int64_t nt = std::max<int64_t>(ntiles((int)I, kWideBN, true),
                                       ntiles((int)H, kWideBN, false));
  return std::min(kSplitSlotsMax, kSplitMax * std::min(mt * nt, kSplitSlotsMax));
}

// The grouped GEMM's part of a tile workspace (int32 words from ws): error
// header, the two class prefixes and the split word, then the split-K
// counters and partial slots.
struct TileWs {
  int32_t *err, *pre_s, *pre_w, *split, *claims, *ctr;
  float *part;
  int slots;
};

// int32 words after the error header: two prefixes, the split word and the
// eight claim counters
int64_t tile_head_words(int64_t n_local) { return 2 * (n_local + 1) + 1 + 8; }

TileWs tile_ws(int32_t *ws, int64_t n_local, int64_t slots) {
  TileWs w;
  w.err = ws;
  w.pre_s = ws + kErrHeaderBytes / 4;
  w.pre_w = w.pre_s + (n_local + 1);
  w.split = w.pre_w + (n_local + 1);
  w.claims = w.split + 1;
  const int64_t head = kErrHeaderBytes + align256(tile_head_words(n_local) * 4);
  w.ctr = ws + head / 4;
  w.part = (float *)((char *)ws + head + align256(slots * 4));
  w.slots = (int)slots;
  return w;
}

// Grid of a grouped GEMM launch: one workgroup per unit up to one per
// compute unit (each kernel's LDS ring allows one workgroup per CU); past
// that the workgroups stay resident and walk the units (persistent).
template <int BM, int BN, int WM, int WN, int BK, int ST, int EPI>
hipError_t launch_one(GemmArgs p, int64_t max_units, int num_cus,
                      hipStream_t s) {
  int64_t grid = tile_grid(max_units);
  if (MOE_GEMM_PERSISTENT)
    grid = std::min<int64_t>(grid, std::max(8, num_cus / 8 * 8));
  grouped_gemm_kernel<BM, BN, WM, WN, BK, ST, EPI>
      <<<(unsigned)grid, WM * WN * 64, 0, s>>>(p);
  return hipGetLastError();
}

// Tile shapes.  Large experts: 128 rows x 256 B-rows (BK 64, 3 stages), split
// along K when the plan kernel finds too few tiles for the chip.  Small
// experts: 64 x 256 (BK 64, 3 stages).  One plan kernel, then one launch
// that runs both classes.
// host_rows >= 0: the launch covers one group whose row count the host
// knows (the per-expert loop); the grid is sized for it.
template <int EPI>
hipError_t launch_grouped(GemmArgs p, int num_cus, const TileWs &ws,
                          int64_t R_cap, hipStream_t s,
                          int64_t host_rows = -1) {
  const bool sw = EPI == EPI_SWIGLU;
  const int nt_w = ntiles(p.N, kWideBN, sw);
  const int nt_s = ntiles(p.N, kSmallBN, sw);
  const int64_t grid_rows = host_rows >= 0 ? host_rows : R_cap;
  p.r_cap = (int)R_cap;
  SplitPlan sp{};
  if (ws.slots >= 2) {
    sp.word = ws.split;
    sp.ctr = ws.ctr;
    sp.below = 2 * num_cus;
    sp.P = num_cus;
    sp.slots = ws.slots;
    sp.smax = kSplitMax;
    sp.KT = p.K / kWideCfg[4];
    // slot: BM x BN fp32; the tile's weights: BN rows of K bf16
    sp.part_ratio = (float)(kWideBM * 4) / (float)(p.K * 2);
  }
  gemm_plan_kernel<<<1, plan_threads(p.G), 0, s>>>(p.offsets, p.G, p.r_cap, ws.err,
                                      p.group_w, p.n_w, 64, nt_s, kWideBM,
                                      nt_w, ws.pre_s, ws.pre_w, sp,
                                      ws.claims);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // both row classes in one launch
  GemmArgs ps = p;
  ps.tile_prefix = ws.pre_s;
  ps.NT = nt_s;
  GemmArgs pw = p;
  pw.tile_prefix = ws.pre_w;
  pw.NT = nt_w;
  pw.claims = ws.claims;
  // units: the small class's tiles (an expert of at most 64 rows has one
  // m-tile) plus the large class's tiles or split units
  const int64_t small_units =
      host_rows >= 0 ? (host_rows <= kSmallRows ? nt_s : 0) : (int64_t)p.G * nt_s;
  int64_t wide_units =
      host_rows >= 0 && host_rows <= kSmallRows
          ? 0
          : ((grid_rows + kWideBM - 1) / kWideBM + p.G) * (int64_t)nt_w;
  if (sp.word) {
    pw.split = ws.split;
    pw.ctr = ws.ctr;
    pw.part = ws.part;
    if (wide_units > 0) wide_units = std::max<int64_t>(wide_units, ws.slots);
  }
  int64_t grid = tile_grid(small_units + wide_units);
  if (MOE_GEMM_PERSISTENT)
    grid = std::min<int64_t>(grid, std::max(8, num_cus / 8 * 8));
  grouped_gemm2_kernel<EPI><<<(unsigned)grid, 256, 0, s>>>(ps, pw);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t n_local, int64_t R_cap, int64_t H,
                            int64_t I) {
  const int64_t slots = split_slots(n_local, R_cap, H, I);
  return kErrHeaderBytes + align256(tile_head_words(n_local) * 4) +
         align256(slots * 4) + slots * kSlotBytes;
}

hipError_t launch_gate_up_bf16(const uint16_t *x_perm, const int32_t *offsets,
                               const float *s_perm, int n_local, int64_t R_cap,
                               int H, int I, const uint16_t *w_gate,
                               const uint16_t *w_up, uint16_t *a,
                               int32_t *tile_ws, int num_cus, hipStream_t s,
                               const int32_t *row_src, int k, int64_t T,
                               const int32_t *group_w, int n_w) {
  GemmArgs p{};
  p.group_w = group_w; p.n_w = n_w;
  p.A = x_perm; p.B0 = w_gate; p.B1 = w_up;
  p.a_rows = row_src; p.a_div = k; p.a_rows_max = (int)(T - 1);
  p.b_stride = (int64_t)I * H;
  p.C = a; p.ldc = I; p.row_scale = s_perm;
  p.offsets = offsets; p.G = n_local; p.N = I; p.K = H;
  const TileWs ws = moe::tile_ws(tile_ws, n_local,
                                 split_slots(n_local, R_cap, H, I));
  return launch_grouped<EPI_SWIGLU>(p, num_cus, ws, R_cap, s);
}

hipError_t launch_down_bf16(const uint16_t *a, const int32_t *offsets,
                            int n_local, int64_t R_cap, int H, int I,
                            const uint16_t *w_down, uint16_t *y,
                            int32_t *tile_ws, int num_cus, hipStream_t s,
                            const int32_t *group_w, int n_w) {
  GemmArgs p{};
  p.group_w = group_w; p.n_w = n_w;
  p.A = a; p.B0 = w_down; p.B1 = nullptr;
  p.b_stride = (int64_t)H * I;
  p.C = y; p.ldc = H;
  p.offsets = offsets; p.G = n_local; p.N = H; p.K = I;
  const TileWs ws = moe::tile_ws(tile_ws, n_local,
                                 split_slots(n_local, R_cap, H, I));
  return launch_grouped<EPI_BF16>(p, num_cus, ws, R_cap, s);
}

hipError_t launch_ffn_loop_bf16(const uint16_t *x_perm, const int32_t *offsets,
                               const int32_t *host_counts, const float *s_perm,
                               int n_local, int64_t R_cap, int H, int I,
                               const uint16_t *w_gate, const uint16_t *w_up,
                               const uint16_t *w_down, uint16_t *a,
                               uint16_t *y, int32_t *tile_ws, int num_cus,
                               hipStream_t s) {
  const int64_t IH = (int64_t)I * H;
  const TileWs ws = moe::tile_ws(tile_ws, n_local,
                                 split_slots(n_local, R_cap, H, I));
  for (int e = 0; e < n_local; ++e) {
    const int64_t n = host_counts[e];
    if (n <= 0) continue;
    // one group: rows [offsets[e], offsets[e+1]) read through offsets + e
    GemmArgs g{};
    g.A = x_perm; g.B0 = w_gate + e * IH; g.B1 = w_up + e * IH;
    g.b_stride = 0;
    g.C = a; g.ldc = I; g.row_scale = s_perm;
    g.offsets = offsets + e; g.G = 1; g.N = I; g.K = H;
    hipError_t err = launch_grouped<EPI_SWIGLU>(g, num_cus, ws, R_cap, s, n);
    if (err != hipSuccess) return err;
    GemmArgs d{};
    d.A = a; d.B0 = w_down + e * IH; d.B1 = nullptr;
    d.b_stride = 0;
    d.C = y; d.ldc = H;
    d.offsets = offsets + e; d.G = 1; d.N = H; d.K = I;
    err = launch_grouped<EPI_BF16>(d, num_cus, ws, R_cap, s, n);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_router_gemm_bf16(const uint16_t *x, const uint16_t *w,
                                   const float *bias, float *logits, int64_t T,
                                   int H, int E, int num_cus, hipStream_t s) {
  GemmArgs p{};
  p.A = x; p.B0 = w; p.b_stride = 0;
  p.C = logits; p.ldc = E;
  p.bias = bias;
  p.offsets = nullptr; p.single_rows = (int)T; p.G = 1; p.N = E; p.K = H;
  // 64 x 128 tiles, 4 stages: at 8192 tokens x 256 experts x 7168 that is
  // one tile per CU and each token row read twice (64 x 64 tiles: 9% slower)
  p.NT = ntiles(E, 128, false);
  const int64_t max_tiles = (T + 63) / 64 * (int64_t)p.NT;
  return launch_one<64, 128, 2, 2, 64, 4, EPI_F32_BIAS>(p, max_tiles, num_cus,
                                                        s);
}

// ---- the FFN in one launch (decode fusion) ---------------------------------
// Gate/up and down of the grouped FFN as one persistent launch, on the same
// tiles, unit bodies and split-K hand-over as the two grouped launches.
// The units of each phase (every gate/up unit: small-row class, then
// large-row class; then every down unit) are cut into 8 contiguous shares,
// one per XCD, each with a claim counter; a workgroup claims from its XCD's
// share and, when that is used up, from the others'.  It moves on to the
// down phase only after finding every gate/up share used up.  A
// gate/up tile writes its columns of a through device-coherent stores and
// counts in on its (expert, m-tile) counter; a down tile of that expert and
// m-tile (same row class, so the same rows) waits until all nt_gu gate/up
// tiles of those rows have counted in, then reads a through its direct-to-LDS
// loads: its lines of a were never read before in this launch, so no cache
// holds a stale copy (rows of a are whole cache lines: I % 64 == 0).  Every
// unit a waiting workgroup depends on was claimed before it by a running
// workgroup that never waits, so each wait ends; a wall-clock bound on it
// sets kDevErrWait instead of hanging.  Shares by XCD keep the tiles that
// share a weight strip or an expert's rows behind one L2, as in the grouped
// launches.  Control flow is uniform per workgroup: the claims go through
// all of wavefront 0's lanes and readfirstlane.

// Per (class, GEMM) launch state, then the hand-over state.
struct FfnArgs {
  GemmArgs g[4];            // gate/up small, gate/up large, down small, down large
  const int32_t *mpre_s;    // [G + 1] m-tile prefix of the small-row class
  const int32_t *mpre_w;    // [G + 1] m-tile prefix of the large-row class
  int32_t *words;           // [0..15] claim counters (gate/up, then down,
                            //   per XCD share); [16] S gate/up, [17] S down
  int32_t *dep;             // per m-tile (small class, then large) counters
  int32_t *err;             // error word (kDevErrWait on a wait that gave up)
  int nt_gu;                // gate/up tiles per m-tile
};

// Bound on one wait, in ticks of the 100 MHz constant clock (0.2 s).
constexpr uint64_t kFfnWaitTicks = 20000000;

// Wavefront 0 polls *cnt until it reaches target (bounded), then the
// workgroup goes on.
__device__ __forceinline__ void ffn_wait(const int32_t *cnt, int target,
                                         int32_t *err, int wid, int lane) {
  if (wid == 0) {
    const uint64_t t0 = wall_clock64();
    for (;;) {
      const int v = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
          cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (v >= target) break;
      if (wall_clock64() - t0 > kFfnWaitTicks) {
        if (lane == 0) atomicOr(err, kDevErrWait);
        break;
      }
      // about a microsecond between polls: waits last up to a gate/up
      // tile's time, and denser polling of one address slows the weight
      // stream of the tiles being waited for
      __builtin_amdgcn_s_sleep(32);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void grouped_ffn_kernel(FfnArgs f) {
  constexpr int RS = TileCfg<MOE_SMALL_CFG>::RING;
  constexpr int RW = TileCfg<MOE_WIDE_CFG>::RING;
  __shared__ uint4 smem[RS > RW ? RS : RW];
  __shared__ int s_last, s_unit;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = f.g[0].G;
  const int Gs = f.g[0].tile_prefix[G], Gw = f.g[1].tile_prefix[G];
  const int Ds = f.g[2].tile_prefix[G], Dw = f.g[3].tile_prefix[G];
  const int Sg = f.words[16], Sd = f.words[17];
  const int Ms = f.mpre_s[G];
  const int n0 = Gs, n1 = n0 + Gw * Sg, n2 = n1 + Ds, n3 = n2 + Dw * Sd;
  const int xcd = blockIdx.x & 7;
  int phase = 0;  // wavefront 0's: 0 gate/up, 1 down, 2 done
  for (;;) {
    __syncthreads();  // the previous unit is done with LDS and s_unit
    if (wid == 0) {
      int unit = -1;
      while (phase < 2 && unit < 0) {
        const int base = phase == 0 ? 0 : n1;
        const int n = phase == 0 ? n1 : n3 - n1;
        const int per = (n + 7) >> 3;
        for (int y = 0; y < 8 && unit < 0; ++y) {
          const int z = (xcd + y) & 7;
          const int lo = min(n, z * per), size = min(n, lo + per) - lo;
          if (size == 0) continue;
          // one atomic, from lane 0 (a branch without barriers or loops
          // inside); its old value is the claim
          int v = 0;
          if (lane == 0)
            v = __hip_atomic_fetch_add(f.words + phase * 8 + z, 1,
                                       __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
          v = __builtin_amdgcn_readfirstlane(v);
          if (v < size) unit = base + lo + v;
        }
        if (unit < 0) ++phase;  // every share of this phase is used up
      }
      if (lane == 0) s_unit = unit < 0 ? n3 : unit;
    }
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(s_unit);
    if (u >= n3) break;
    int e, mt, nt, row0, rows;
    if (u < n0) {
      tile_coords<64>(f.g[0], u, e, mt, nt, row0, rows);
      gemm_unit<MOE_SMALL_CFG, EPI_SWIGLU>(f.g[0], u, 0, 1, 0, 0, f.dep,
                                           f.mpre_s[e] + mt, smem, &s_last);
    } else if (u < n1) {
      const int t = (u - n0) / Sg;
      tile_coords<128>(f.g[1], t, e, mt, nt, row0, rows);
      gemm_unit<MOE_WIDE_CFG, EPI_SWIGLU>(f.g[1], t, u - n0 - t * Sg, Sg,
                                          t * Sg, t, f.dep,
                                          Ms + f.mpre_w[e] + mt, smem, &s_last);
    } else if (u < n2) {
      const int t = u - n1;
      tile_coords<64>(f.g[2], t, e, mt, nt, row0, rows);
      ffn_wait(f.dep + f.mpre_s[e] + mt, f.nt_gu, f.err, wid, lane);
      gemm_unit<MOE_SMALL_CFG, EPI_BF16>(f.g[2], t, 0, 1, 0, 0, nullptr, 0,
                                         smem, &s_last);
    } else {
      const int t = (u - n2) / Sd;
      tile_coords<128>(f.g[3], t, e, mt, nt, row0, rows);
      ffn_wait(f.dep + Ms + f.mpre_w[e] + mt, f.nt_gu, f.err, wid, lane);
      gemm_unit<MOE_WIDE_CFG, EPI_BF16>(f.g[3], t, u - n2 - t * Sd, Sd,
                                        Gw * Sg + t * Sd, Gw + t, nullptr, 0,
                                        smem, &s_last);
    }
  }
}

// Plan of the FFN's two GEMMs, one block: per expert the tiles of both row
// classes for both GEMMs and the m-tiles of both classes, as exclusive
// prefixes (G + 1 entries each); the split of each GEMM's large-row class;
// the claim counters, the m-tile counters and the split counters in use
// cleared; the error word (kDevErrRows for offsets past r_cap or
// decreasing, else 0).  For the one-launch FFN (independent == 0) both
// GEMMs' units share the partial slots (gate/up first, down with the slots
// gate/up leaves) and down's tiles count in on the counters after gate/up's.
// For the grouped FFN's two launches (independent == 1) each GEMM chooses
// its split as its own launch would and both start at slot and counter 0:
// the gate/up launch has handed over (and reset its counters) before the
// down launch starts.
struct FfnPlanArgs {
  const int32_t *offsets;
  int G, r_cap;
  int nt[4];                // n-tiles: gate/up small, gate/up large, down small, down large
  int32_t *pre[4];          // tile prefixes, same order
  int32_t *mpre[2];         // m-tile prefixes: small, large
  int32_t *words, *dep, *err;
  SplitPlan gu, dn;         // split choice of each GEMM (word unused)
  int independent;          // 1: the two GEMMs run as separate launches
};

__global__ __launch_bounds__(1024) void ffn_plan_kernel(FfnPlanArgs a) {
  constexpr int NC = 6;     // 4 tile counts, 2 m-tile counts
  __shared__ int32_t wsum[NC][16];
  __shared__ int32_t bad_or;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nth = blockDim.x, nw = nth >> 6;
  if (tid == 0) bad_or = 0;
  const int G = a.G;
  const int per = (G + nth - 1) / nth;
  const int e0 = min(G, tid * per), e1 = min(G, e0 + per);
  auto counts = [&](int e, int32_t (&c)[NC]) {
    int b, en;
    seg_rows(a.offsets, e, a.r_cap, b, en);
    const int n = en - b;
    const int ms = n <= kSmallRows ? (n + 63) / 64 : 0;
    const int mw = n <= kSmallRows ? 0 : (n + 127) / 128;
    c[0] = ms * a.nt[0]; c[1] = mw * a.nt[1];
    c[2] = ms * a.nt[2]; c[3] = mw * a.nt[3];
    c[4] = ms; c[5] = mw;
  };
  int32_t s[NC] = {};
  int bad = 0;
  for (int e = e0; e < e1; ++e) {
    int32_t c[NC];
    counts(e, c);
    for (int i = 0; i < NC; ++i) s[i] += c[i];
    bad |= seg_bad(a.offsets, e, a.r_cap) ? kDevErrRows : 0;
  }
  int32_t x[NC];
  for (int i = 0; i < NC; ++i) x[i] = s[i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int32_t y = __shfl_up(x[i], off, 64);
      if (lane >= off) x[i] += y;
    }
  }
  if (lane == 63)
    for (int i = 0; i < NC; ++i) wsum[i][wv] = x[i];
  __syncthreads();
  int32_t r[NC], total[NC];
  for (int i = 0; i < NC; ++i) {
    int32_t before = 0, all = 0;
    for (int q = 0; q < nw; ++q) {
      const int32_t v = wsum[i][q];
      before += q < wv ? v : 0;
      all += v;
    }
    r[i] = before + x[i] - s[i];
    total[i] = all;
  }
  for (int e = e0; e < e1; ++e) {
    for (int i = 0; i < 4; ++i) a.pre[i][e] = r[i];
    a.mpre[0][e] = r[4];
    a.mpre[1][e] = r[5];
    int32_t c[NC];
    counts(e, c);
    for (int i = 0; i < NC; ++i) r[i] += c[i];
  }
  if (tid == nth - 1) {
    for (int i = 0; i < 4; ++i) a.pre[i][G] = total[i];
    a.mpre[0][G] = total[4];
    a.mpre[1][G] = total[5];
  }
  // splits of the large-row class (every thread chooses the same)
  const int gw = total[1], dw = total[3];
  int Sg = 1, Sd = 1;
  if (a.independent) {
    if (a.gu.slots >= 2) {
      Sg = choose_split(a.gu, gw, a.gu.slots);
      Sd = choose_split(a.dn, dw, a.dn.slots);
    }
  } else if (a.gu.slots >= 2 && (int64_t)gw + dw <= a.gu.slots) {
    // gate/up's units take slots [0, gw*Sg), down's the ones after
    Sg = choose_split(a.gu, gw, a.gu.slots);
    Sd = choose_split(a.dn, dw, (int64_t)a.dn.slots - (int64_t)gw * Sg);
  }
  if (tid < 16) a.words[tid] = 0;
  if (tid == 0) {
    a.words[16] = Sg;
    a.words[17] = Sd;
  }
  const int nm = total[4] + total[5];
  for (int i = tid; i < nm; i += nth) a.dep[i] = 0;
  // split counters: gate/up tiles [0, gw), down tiles [gw, gw + dw) (one
  // launch) or [0, dw) (two launches)
  const int nc = a.independent ? max(Sg > 1 ? gw : 0, Sd > 1 ? dw : 0)
                               : ((Sg > 1 || Sd > 1) ? gw + dw : 0);
  for (int i = tid; i < nc; i += nth) a.gu.ctr[i] = 0;
  if (bad) atomicOr(&bad_or, bad);
  __syncthreads();
  if (tid == 0) *a.err = bad_or;
}

namespace {

// The fused FFN's arrays after the grouped GEMM's part of the workspace.
struct FfnWs {
  int32_t *pre_ds, *pre_dw, *mpre_s, *mpre_w, *words, *dep;
};

int64_t ffn_extra_words(int64_t n_local, int64_t R_cap) {
  // 4 prefixes, 20 words, m-tile counters: at most n_local small m-tiles
  // and R_cap / 128 + n_local large ones
  return 4 * (n_local + 1) + 20 + 2 * n_local + R_cap / 128 + 1;
}

FfnWs ffn_ws(const TileWs &w, int64_t n_local) {
  FfnWs f;
  int32_t *x = (int32_t *)(w.part + (int64_t)w.slots * kSlotFloats);
  f.pre_ds = x;
  f.pre_dw = f.pre_ds + (n_local + 1);
  f.mpre_s = f.pre_dw + (n_local + 1);
  f.mpre_w = f.mpre_s + (n_local + 1);
  f.words = f.mpre_w + (n_local + 1);
  f.dep = f.words + 20;
  return f;
}

}  // namespace

size_t ffn_fused_workspace_bytes(int64_t n_local, int64_t R_cap, int64_t H,
                                 int64_t I) {
  return gemm_workspace_bytes(n_local, R_cap, H, I) +
         (size_t)align256(ffn_extra_words(n_local, R_cap) * 4);
}

namespace {

// Arguments of both GEMMs of the FFN and of their plan kernel, over the
// workspace laid out as the one-launch FFN's (the grouped FFN's two launches
// use the same layout).
struct FfnSetup {
  FfnArgs f;
  FfnPlanArgs pa;
  TileWs w;
  FfnWs fw;
};

FfnSetup ffn_setup(const uint16_t *x, const int32_t *row_src, int k,
                   int64_t T, const int32_t *offsets, const float *s_perm,
                   int n_local, int64_t R_cap, int H, int I,
                   const uint16_t *w_gate, const uint16_t *w_up,
                   const uint16_t *w_down, uint16_t *a, uint16_t *y,
                   int32_t *ws, int num_cus, int independent) {
  FfnSetup st{};
  const int64_t slots = split_slots(n_local, R_cap, H, I);
  st.w = moe::tile_ws(ws, n_local, slots);
  st.fw = ffn_ws(st.w, n_local);
  const TileWs &w = st.w;
  const FfnWs &fw = st.fw;
  FfnArgs &f = st.f;
  // gate/up: x (gathered through row_src, or x_perm) against W_gate / W_up
  GemmArgs gu{};
  gu.A = x; gu.B0 = w_gate; gu.B1 = w_up;
  gu.a_rows = row_src; gu.a_div = row_src ? k : 1;
  gu.a_rows_max = row_src ? (int)(T - 1) : (int)R_cap - 1;
  gu.b_stride = (int64_t)I * H;
  gu.C = a; gu.ldc = I; gu.row_scale = s_perm;
  gu.offsets = offsets; gu.G = n_local; gu.N = I; gu.K = H;
  gu.r_cap = (int)R_cap;
  gu.ctr = w.ctr; gu.part = w.part;
  GemmArgs dn{};
  dn.A = a; dn.B0 = w_down;
  dn.b_stride = (int64_t)H * I;
  dn.C = y; dn.ldc = H;
  dn.offsets = offsets; dn.G = n_local; dn.N = H; dn.K = I;
  dn.r_cap = (int)R_cap;
  dn.ctr = w.ctr; dn.part = w.part;
  const int nt[4] = {ntiles(I, kSmallBN, true), ntiles(I, kWideBN, true),
                     ntiles(H, kSmallBN, false), ntiles(H, kWideBN, false)};
  int32_t *pre[4] = {w.pre_s, w.pre_w, fw.pre_ds, fw.pre_dw};
  for (int i = 0; i < 4; ++i) {
    f.g[i] = i < 2 ? gu : dn;
    f.g[i].tile_prefix = pre[i];
    f.g[i].NT = nt[i];
  }
  f.mpre_s = fw.mpre_s; f.mpre_w = fw.mpre_w;
  f.words = fw.words; f.dep = fw.dep; f.err = w.err;
  f.nt_gu = nt[0];
  FfnPlanArgs &pa = st.pa;
  pa.offsets = offsets; pa.G = n_local; pa.r_cap = (int)R_cap;
  for (int i = 0; i < 4; ++i) { pa.nt[i] = nt[i]; pa.pre[i] = pre[i]; }
  pa.mpre[0] = fw.mpre_s; pa.mpre[1] = fw.mpre_w;
  pa.words = fw.words; pa.dep = fw.dep; pa.err = w.err;
  pa.independent = independent;
  for (int i = 0; i < 2; ++i) {
    SplitPlan &sp = i == 0 ? pa.gu : pa.dn;
    const int K = i == 0 ? H : I;
    if (slots >= 2) {
      sp.ctr = w.ctr;
      sp.below = 2 * num_cus;
      sp.P = num_cus;
      sp.slots = (int)slots;
      sp.smax = kSplitMax;
      sp.KT = K / kWideCfg[4];
      sp.part_ratio = (float)(kWideBM * 4) / (float)(K * 2);
    }
  }
  return st;
}

// Workgroups of a grouped GEMM launch over n_local experts and rows up to
// R_cap (units of both classes; the wide class at least as many as the
// partial slots when it may split), one per compute unit at most.
int64_t gemm2_grid(int N, bool swiglu, int n_local, int64_t R_cap,
                   int slots, int num_cus) {
  const int64_t small_units = (int64_t)n_local * ntiles(N, kSmallBN, swiglu);
  int64_t wide_units = ((R_cap + kWideBM - 1) / kWideBM + n_local) *
                       (int64_t)ntiles(N, kWideBN, swiglu);
  if (slots >= 2) wide_units = std::max<int64_t>(wide_units, slots);
  int64_t grid = tile_grid(small_units + wide_units);
  if (MOE_GEMM_PERSISTENT)
    grid = std::min<int64_t>(grid, std::max(8, num_cus / 8 * 8));
  return grid;
}

}  // namespace

hipError_t launch_ffn_fused_bf16(const uint16_t *x, const int32_t *row_src,
                                 int k, int64_t T, const int32_t *offsets,
                                 const float *s_perm, int n_local,
                                 int64_t R_cap, int H, int I,
                                 const uint16_t *w_gate, const uint16_t *w_up,
                                 const uint16_t *w_down, uint16_t *a,
                                 uint16_t *y, int32_t *ws, int num_cus,
                                 hipStream_t s) {
  const FfnSetup st = ffn_setup(x, row_src, k, T, offsets, s_perm, n_local,
                                R_cap, H, I, w_gate, w_up, w_down, a, y, ws,
                                num_cus, 0);
  ffn_plan_kernel<<<1, plan_threads(n_local), 0, s>>>(st.pa);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // one resident workgroup per CU (the LDS ring allows one), a multiple of
  // 8 so that every XCD has as many; a grid larger than the work only adds
  // workgroups that claim nothing
  grouped_ffn_kernel<<<(unsigned)std::max(8, num_cus / 8 * 8), 256, 0, s>>>(
      st.f);
  return hipGetLastError();
}

hipError_t launch_ffn_grouped_bf16(const uint16_t *x, const int32_t *row_src,
                                   int k, int64_t T, const int32_t *offsets,
                                   const float *s_perm, int n_local,
                                   int64_t R_cap, int H, int I,
                                   const uint16_t *w_gate,
                                   const uint16_t *w_up,
                                   const uint16_t *w_down, uint16_t *a,
                                   uint16_t *y, int32_t *ws, int num_cus,
                                   hipStream_t s) {
  const FfnSetup st = ffn_setup(x, row_src, k, T, offsets, s_perm, n_local,
                                R_cap, H, I, w_gate, w_up, w_down, a, y, ws,
                                num_cus, 1);
  ffn_plan_kernel<<<1, plan_threads(n_local), 0, s>>>(st.pa);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const bool split = st.w.slots >= 2;
  for (int d = 0; d < 2; ++d) {
    GemmArgs ps = st.f.g[2 * d], pw = st.f.g[2 * d + 1];
    pw.claims = st.fw.words + 8 * d;
    if (split) pw.split = st.fw.words + 16 + d;
    else { pw.ctr = nullptr; pw.part = nullptr; }
    const int64_t grid = gemm2_grid(d == 0 ? I : H, d == 0, n_local, R_cap,
                                    st.w.slots, num_cus);
    if (d == 0)
      grouped_gemm2_kernel<EPI_SWIGLU><<<(unsigned)grid, 256, 0, s>>>(ps, pw);
    else
      grouped_gemm2_kernel<EPI_BF16><<<(unsigned)grid, 256, 0, s>>>(ps, pw);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
