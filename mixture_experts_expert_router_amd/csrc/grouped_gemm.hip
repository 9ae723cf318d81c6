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
// Design (one launch per expert-size class, all experts of that class):
//   * C[r, n] = sum_k A[r, k] * B_e[n, k] for the rows r of expert e's
//     segment [offsets[e], offsets[e+1]); A and B are K-contiguous bf16.
//   * Work unit = tile of BM rows x BN B-rows of one expert.  A plan kernel
//     turns the device-side offsets into tile prefixes for two classes of
//     experts: those with at most kSmallRows rows (decode-like shares, run
//     with 64-row tiles) and the rest (128- or 256-row tiles).  Each class has
//     its own launch; the host never needs the per-expert counts.
//   * One tile per workgroup; the grid is launched for an upper bound and
//     each workgroup derives its tile from the device-side count (xcd_tile):
//     XCD x (workgroup id mod 8) takes a contiguous tile range in dispatch
//     order, and inside an expert tiles run in bands of 8 m-tiles with the
//     m-tile fastest (banded_mn), so workgroups running together on one L2
//     share the weight strip and the expert's rows.
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
//   * Gather on load (gate/up): A rows may be read straight from the token
//     rows x[row_src[r] / k] instead of a permuted copy.
//   * Epilogues: SWIGLU (B rows alternate 32 gate and the 32 matching up
//     rows, so each lane holds g and u of the same outputs; writes
//     a = s * SiLU(g) * u in bf16), BF16 (plain store) and F32_BIAS (router
//     logits + bias).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

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
  int G;                    // groups
  int N;                    // output columns (a-columns for SWIGLU)
  int K;
  int NT;                   // n-tiles per m-tile
};

// Experts with at most this many rows run on the 64-row-tile kernel.
constexpr int kSmallRows = 64;

// Tile prefixes per row class: prefix_c[e+1] = prefix_c[e] + ceil(rows_e /
// BM_c) * NT_c when expert e belongs to class c.  Experts with at most
// kSmallRows rows form the small class (0); the others are tiled either with
// the wide shape (1) or with the narrow one (2).  Without prefix_narrow the
// wide shape is used.  Otherwise the narrow one is used when the wide shape
// would give fewer than wide_min tiles in all, and its tiles fit in
// narrow_cap; the other shape's prefix is then all zeros.  One block.
__global__ __launch_bounds__(1024) void gemm_plan_kernel(
    const int32_t *__restrict__ offsets, int G, int bm_small, int nt_small,
    int bm_wide, int nt_wide, int bm_narrow, int nt_narrow, int wide_min,
    int narrow_cap, int32_t *__restrict__ prefix_small,
    int32_t *__restrict__ prefix_wide, int32_t *__restrict__ prefix_narrow) {
  __shared__ int32_t wsum[3][16];
  const int tid = threadIdx.x;
  const int per = (G + 1023) / 1024;
  const int e0 = min(G, tid * per), e1 = min(G, e0 + per);
  auto tiles = [&](int e, int32_t &t0, int32_t &t1, int32_t &t2) {
    const int n = offsets[e + 1] - offsets[e];
    t0 = t1 = t2 = 0;
    if (n <= kSmallRows) {
      t0 = (n + bm_small - 1) / bm_small * nt_small;
    } else {
      t1 = (n + bm_wide - 1) / bm_wide * nt_wide;
      t2 = (n + bm_narrow - 1) / bm_narrow * nt_narrow;
    }
  };
  int32_t s[3] = {0, 0, 0};
  for (int e = e0; e < e1; ++e) {
    int32_t t[3];
    tiles(e, t[0], t[1], t[2]);
    for (int c = 0; c < 3; ++c) s[c] += t[c];
  }
  // Inclusive scan of s over the block: lane shuffles inside each
  // wavefront, then the 16 wavefront totals through LDS (one barrier).
  const int lane = tid & 63, wv = tid >> 6;
  int32_t x[3] = {s[0], s[1], s[2]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int32_t y = __shfl_up(x[c], off, 64);
      if (lane >= off) x[c] += y;
    }
  }
  if (lane == 63)
    for (int c = 0; c < 3; ++c) wsum[c][wv] = x[c];
  __syncthreads();
  int32_t incl[3], total[3];
  for (int c = 0; c < 3; ++c) {
    int32_t before = 0, all = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int32_t v = wsum[c][q];
      before += q < wv ? v : 0;
      all += v;
    }
    incl[c] = before + x[c];
    total[c] = all;
  }
  const bool narrow = prefix_narrow != nullptr && total[1] < wide_min &&
                      total[2] <= narrow_cap;
  int32_t r[3];
  for (int c = 0; c < 3; ++c) r[c] = incl[c] - s[c];
  for (int e = e0; e < e1; ++e) {
    prefix_small[e] = r[0];
    prefix_wide[e] = narrow ? 0 : r[1];
    if (prefix_narrow) prefix_narrow[e] = narrow ? r[2] : 0;
    int32_t t[3];
    tiles(e, t[0], t[1], t[2]);
    for (int c = 0; c < 3; ++c) r[c] += t[c];
  }
  if (tid == 1023) {
    prefix_small[G] = total[0];
    prefix_wide[G] = narrow ? 0 : total[1];
    if (prefix_narrow) prefix_narrow[G] = narrow ? total[2] : 0;
  }
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
template <int BM, int BN, int WM, int WN, int BK, int STAGES, int MV>
__device__ __forceinline__ void gemm_kloop(
    f32x16 (&acc)[BM / WM / 32][BN / WN / 32],
    const char *const (&gsrc)[(BM + BN) * (BK / 8) / (WM * WN * 64)],
    const uint4 *smem, uint32_t lds0, uint32_t wave_off, int KT, int lane,
    int arow0, int brow0) {
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
    const int64_t koff = (int64_t)ks * (BK * 2);
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
            const int f = (kk * MV + m) * NB + n;
#pragma unroll
            for (int i = f * L / NMF; i < (f + 1) * L / NMF; ++i) {
              __builtin_amdgcn_sched_barrier(0);
              load_lds16(sb + (uint32_t)(i * 64 * 16), gsrc[i] + koff);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < L; ++i)
        load_lds16(sb + (uint32_t)(i * 64 * 16), gsrc[i] + koff);
    }
  }
  wait_loads_barrier<0>();
}

template <int BM, int BN, int WM, int WN, int BK, int STAGES, int EPI>
__global__ __launch_bounds__(WM * WN * 64) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int NTH = WM * WN * 64;            // 4 or 8 wavefronts
  constexpr int CPR = BK / 8;                  // 16-byte chunks per row
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int STAGE_CHUNKS = (BM + BN) * CPR;
  constexpr int L = STAGE_CHUNKS / NTH;        // loads per thread per stage
  static_assert(WM * WN == 4 || WM * WN == 8, "four or eight wavefronts");
  static_assert(MB >= 1 && NB >= 1, "wave tile is a multiple of 32x32");
  static_assert(EPI != EPI_SWIGLU || NB % 2 == 0,
                "SwiGLU pairs a gate block with the up block next to it");
  static_assert(BM * CPR % NTH == 0 && BN * CPR % NTH == 0, "load split");
  static_assert(STAGES * STAGE_CHUNKS * 16 >= WM * WN * WTM * WTN * 2,
                "the ring must hold every wavefront's epilogue region");
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(STAGES >= 2 && STAGES <= 6 && (STAGES - 2) * L <= 63,
                "vmcnt range");
  __shared__ uint4 smem[STAGES * STAGE_CHUNKS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int wm = wid / WN, wn = wid % WN;
  const int K = p.K;
  const int KT = K / BK;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  int total;
  if (p.offsets) total = p.tile_prefix[p.G];
  else total = (p.single_rows + BM - 1) / BM * p.NT;

  const int t = xcd_tile(blockIdx.x, total);
  if (t < 0) return;
  {
    int e, r_begin, r_end, local;
    if (p.offsets) {
      e = upper_bound_minus1(p.tile_prefix, p.G, t);
      r_begin = p.offsets[e];
      r_end = p.offsets[e + 1];
      local = t - p.tile_prefix[e];
    } else {
      e = 0; r_begin = 0; r_end = p.single_rows; local = t;
    }
    const int mtiles = (r_end - r_begin + BM - 1) / BM;
    int mt, nt;
    banded_mn(local, mtiles, p.NT, 8, mt, nt);
    const int row0 = r_begin + mt * BM;
    const int rows = min(BM, r_end - row0);

    // Global source of each of this thread's L loads per stage.  The stage
    // is cut into groups of 64 chunks (one load instruction each); wavefront
    // w issues groups [w*L, w*L + L), so with BM == BN two wavefronts load
    // only A rows (mostly L2 hits) and two only B rows (weight stream): a
    // wavefront's loads return in order, and this keeps the quick hits out
    // of the queue behind slow misses.  Chunk q = (w*L + i)*64 + lane.
    const char *gsrc[L];
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
        gsrc[i] = (const char *)(base + (int64_t)e * p.b_stride + (int64_t)col * K + kc * 8);
      }
    }
    const uint32_t wave_off = (uint32_t)(wid * L * 64 * 16);

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
      const int64_t koff = (int64_t)min(st, KT - 1) * (BK * 2);
#pragma unroll
      for (int i = 0; i < L; ++i)
        load_lds16(sb + (uint32_t)(i * 64 * 16), gsrc[i] + koff);
    }
    // the K loop, specialised for this wavefront's number of valid blocks
    // (a wavefront with none still keeps the loads and barriers going)
    switch (mvalid) {
#define MOE_KLOOP_CASE(mv)                                                    \
      case mv:                                                                \
        if (mv <= MB)                                                         \
          gemm_kloop<BM, BN, WM, WN, BK, STAGES, (mv <= MB ? mv : 1)>(        \
              acc, gsrc, smem, lds0, wave_off, KT, lane, wrow0, brow0);       \
        break;
      MOE_KLOOP_CASE(1)
      MOE_KLOOP_CASE(2)
      MOE_KLOOP_CASE(3)
      MOE_KLOOP_CASE(4)
#undef MOE_KLOOP_CASE
      default:
        gemm_kloop<BM, BN, WM, WN, BK, STAGES, 0>(
            acc, gsrc, smem, lds0, wave_off, KT, lane, wrow0, brow0);
    }
    // every wavefront is done reading the ring before the next tile refills it
    wait_loads_barrier<0>();

    // Epilogue.  Lane holds column (lane & 31) of each 32x32 block and rows
    // 8*(r/4) + 4*(lane/32) + (r%4), r < 16.  bf16 outputs are staged in a
    // per-wavefront LDS region and leave as 16-byte row pieces.
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
          const int i = wrow0 + rw;
          const float s = (i < rows && p.row_scale) ? p.row_scale[row0 + i] : 1.f;
#pragma unroll
          for (int q = 0; q < NB / 2; ++q) {
            const float g = acc[m][2 * q][r], u = acc[m][2 * q + 1][r];
            lw[rw * W + st_col<W>(rw, q * 32 + (lane & 31))] =
                (uint16_t)f32_to_bf16_bits(s * silu_f32(g) * u);
          }
        }
      }
      __syncthreads();
      store_staged<W, WTM>(lw, (uint16_t *)p.C, p.ldc,
                           (int64_t)nt * (BN / 2) + wn * W, p.N, row0 + wrow0,
                           wrow0, rows, lane);
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
}

namespace {

// BM, BN, WM, WN, BK, STAGES of the wide large-expert shape.
#ifndef MOE_NARROW_CFG
#define MOE_NARROW_CFG 256, 64, 4, 1, 64, 3
#endif
#ifndef MOE_WIDE_CFG
#define MOE_WIDE_CFG 128, 256, 2, 2, 64, 3
#endif

int ntiles(int N, int BN, bool swiglu) {
  const int cols = swiglu ? BN / 2 : BN;
  return (N + cols - 1) / cols;
}

template <int BM, int BN, int WM, int WN, int BK, int ST, int EPI>
hipError_t launch_one(GemmArgs p, int num_cus, int64_t max_tiles,
                      hipStream_t s) {
  (void)num_cus;
  grouped_gemm_kernel<BM, BN, WM, WN, BK, ST, EPI>
      <<<(unsigned)tile_grid(max_tiles), WM * WN * 64, 0, s>>>(p);
  return hipGetLastError();
}

// Tile shapes.  Large experts: 128 rows x 256 B-rows (BK 64, 3 stages), or
// 256 x 64 (BK 64, 3 stages) when the wide shape would give fewer than two
// tiles per CU.  Small experts: 64 x 256 (BK 64, 3 stages).  When the host
// cannot rule the narrow shape out (few experts times n-tiles), the plan
// kernel chooses from the actual rows and both kernels are launched; the one
// not chosen finds no tiles.
template <int EPI>
hipError_t launch_grouped(GemmArgs p, int num_cus, int32_t *tile_ws,
                          int64_t R_cap, hipStream_t s) {
  const bool sw = EPI == EPI_SWIGLU;
  constexpr int wide_cfg[6] = {MOE_WIDE_CFG};
  constexpr int narrow_cfg[6] = {MOE_NARROW_CFG};
  constexpr int WBM = wide_cfg[0], WBN = wide_cfg[1];
  constexpr int NBM = narrow_cfg[0], NBN = narrow_cfg[1];
  const int wide_min = 2 * num_cus;
  const int nt_w = ntiles(p.N, WBN, sw), nt_n = ntiles(p.N, NBN, sw);
  const int nt_s = ntiles(p.N, 256, sw);
  const bool wide_sure = (int64_t)p.G * nt_w >= wide_min;
  // The narrow kernel's grid; the plan kernel keeps the wide shape when the
  // narrow one would need more tiles than this.
  const int64_t max_n = ((R_cap + NBM - 1) / NBM + p.G) * (int64_t)nt_n;
  const int narrow_cap = (int)std::min<int64_t>(max_n, 8LL * num_cus);
  int32_t *pre_s = tile_ws;
  int32_t *pre_w = tile_ws + (p.G + 1);
  int32_t *pre_n = tile_ws + 2 * (p.G + 1);
  gemm_plan_kernel<<<1, 1024, 0, s>>>(p.offsets, p.G, 64, nt_s, WBM, nt_w,
                                      NBM, nt_n, wide_min, narrow_cap, pre_s,
                                      pre_w, wide_sure ? nullptr : pre_n);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // small-row class
  GemmArgs ps = p;
  ps.tile_prefix = pre_s;
  ps.NT = nt_s;
  err = launch_one<64, 256, 1, 4, 64, 3, EPI>(ps, num_cus,
                                              (int64_t)p.G * nt_s, s);
  if (err != hipSuccess) return err;
  // large-row class
  if (!wide_sure) {
    GemmArgs pn = p;
    pn.tile_prefix = pre_n;
    pn.NT = nt_n;
    err = launch_one<MOE_NARROW_CFG, EPI>(pn, num_cus, narrow_cap, s);
    if (err != hipSuccess) return err;
  }
  GemmArgs pw = p;
  pw.tile_prefix = pre_w;
  pw.NT = nt_w;
  const int64_t max_w = ((R_cap + WBM - 1) / WBM + p.G) * (int64_t)nt_w;
  return launch_one<MOE_WIDE_CFG, EPI>(pw, num_cus, max_w, s);
}

}  // namespace

size_t gemm_workspace_bytes(int64_t n_local) {
  return (size_t)((3 * (n_local + 1) * 4 + 255) / 256 * 256);
}

hipError_t launch_gate_up_bf16(const uint16_t *x_perm, const int32_t *offsets,
                               const float *s_perm, int n_local, int64_t R_cap,
                               int H, int I, const uint16_t *w_gate,
                               const uint16_t *w_up, uint16_t *a,
                               int32_t *tile_ws, int num_cus, hipStream_t s,
                               const int32_t *row_src, int k, int64_t T) {
  GemmArgs p{};
  p.A = x_perm; p.B0 = w_gate; p.B1 = w_up;
  p.a_rows = row_src; p.a_div = k; p.a_rows_max = (int)(T - 1);
  p.b_stride = (int64_t)I * H;
  p.C = a; p.ldc = I; p.row_scale = s_perm;
  p.offsets = offsets; p.G = n_local; p.N = I; p.K = H;
  return launch_grouped<EPI_SWIGLU>(p, num_cus, tile_ws, R_cap, s);
}

hipError_t launch_down_bf16(const uint16_t *a, const int32_t *offsets,
                            int n_local, int64_t R_cap, int H, int I,
                            const uint16_t *w_down, uint16_t *y,
                            int32_t *tile_ws, int num_cus, hipStream_t s) {
  GemmArgs p{};
  p.A = a; p.B0 = w_down; p.B1 = nullptr;
  p.b_stride = (int64_t)H * I;
  p.C = y; p.ldc = H;
  p.offsets = offsets; p.G = n_local; p.N = H; p.K = I;
  return launch_grouped<EPI_BF16>(p, num_cus, tile_ws, R_cap, s);
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
  return launch_one<64, 128, 2, 2, 64, 4, EPI_F32_BIAS>(p, num_cus, max_tiles, s);
}

}  // namespace moe
