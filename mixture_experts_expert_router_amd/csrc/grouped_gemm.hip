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
// Design (one launch per GEMM, all experts):
//   * C[r, n] = sum_k A[r, k] * B_e[n, k] for the rows r of expert e's
//     segment [offsets[e], offsets[e+1]); A and B are K-contiguous bf16.
//   * Work unit = tile of BM rows x BN B-rows of one expert.  A small plan
//     kernel turns the device-side offsets into a tile prefix, so the host
//     never needs the per-expert counts.
//   * Persistent grid: every workgroup walks the tile list with stride
//     gridDim.x.  Workgroups are renumbered so that consecutive logical
//     workgroups sit on the same XCD (hardware places workgroup b on XCD
//     b % 8), and tiles are ordered (expert, n-tile, m-tile): the m-tiles of
//     one weight strip, and the n-tiles next to them, run at the same time on
//     one XCD and share its L2.
//   * 256 threads = 4 wavefronts in a WM x WN grid; each wavefront owns a
//     (BM/WM) x (BN/WN) sub-tile made of 32x32 blocks computed with
//     v_mfma_f32_32x32x16_bf16 (fp32 accumulators in registers).
//   * K is walked in steps of 64: global -> registers -> LDS (double buffer),
//     the next step's global loads in flight while the current one computes.
//     LDS rows are 128 B; 16-byte chunks are XOR-swizzled by (row & 7) so the
//     fragment reads of 8 consecutive rows hit distinct banks.
//   * 32-row sub-tiles past the end of an expert's segment are skipped (the
//     branch is uniform per wavefront), so a tile with 16 rows costs one
//     32-row MFMA pass, not BM/32.
//   * Epilogues: SWIGLU (B rows interleaved as 16 gate + 16 up per 32-row
//     block, so one lane swap pairs g and u of the same output; writes
//     a = s * SiLU(g) * u in bf16), BF16 (plain store) and F32_BIAS (router
//     logits + bias).
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
  const int32_t *tile_prefix;  // [G + 1] tile prefix (grouped mode)
  int single_rows;          // rows of the single group (offsets == null)
  int G;                    // groups
  int N;                    // output columns (a-columns for SWIGLU)
  int K;
  int NT;                   // n-tiles per m-tile
};

constexpr int BK = 64;

// tile_prefix[e+1] = tile_prefix[e] + ceil(rows_e / BM) * NT, one block.
__global__ __launch_bounds__(1024) void gemm_plan_kernel(
    const int32_t *__restrict__ offsets, int G, int BM, int NT,
    int32_t *__restrict__ tile_prefix) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (G + 1023) / 1024;
  const int e0 = min(G, tid * per), e1 = min(G, e0 + per);
  int32_t s = 0;
  for (int e = e0; e < e1; ++e)
    s += (offsets[e + 1] - offsets[e] + BM - 1) / BM * NT;
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - s;
  for (int e = e0; e < e1; ++e) {
    tile_prefix[e] = run;
    run += (offsets[e + 1] - offsets[e] + BM - 1) / BM * NT;
  }
  if (tid == 1023) tile_prefix[G] = part[1023];
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs p) {
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int CPR = BK / 8;  // 16-byte chunks per LDS row
  constexpr int A_PER_T = BM * CPR / 256, B_PER_T = BN * CPR / 256;
  static_assert(WM * WN == 4, "four wavefronts");
  static_assert(MB >= 1 && NB >= 1, "wave tile is a multiple of 32x32");
  static_assert(A_PER_T >= 1 && B_PER_T >= 1, "tile too small");
  __shared__ uint4 smem[2][(BM + BN) * CPR];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int K = p.K;
  const int KT = K / BK;

  int total;
  if (p.offsets) total = p.tile_prefix[p.G];
  else total = (p.single_rows + BM - 1) / BM * p.NT;

  const int nwg = gridDim.x, bid = blockIdx.x;
  const int L = (bid & 7) * (nwg >> 3) + (bid >> 3);

  for (int t = L; t < total; t += nwg) {
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
    const int nt = local / mtiles, mt = local - nt * mtiles;
    const int row0 = r_begin + mt * BM;
    const int rows = min(BM, r_end - row0);

    // Per-thread global source pointers for the A and B chunks it loads.
    const uint16_t *a_src[A_PER_T];
    const uint16_t *b_src[B_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int c = tid + i * 256, row = c / CPR, kc = c % CPR;
      a_src[i] = p.A + (int64_t)(row0 + min(row, rows - 1)) * K + kc * 8;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int c = tid + i * 256, j = c / CPR, kc = c % CPR;
      const uint16_t *base;
      int col;
      if (EPI == EPI_SWIGLU) {
        const int w = j & 31;
        col = nt * (BN / 2) + (j >> 5) * 16 + (w & 15);
        base = w < 16 ? p.B0 : p.B1;
      } else {
        col = nt * BN + j;
        base = p.B0;
      }
      col = min(col, p.N - 1);
      b_src[i] = base + (int64_t)e * p.b_stride + (int64_t)col * K + kc * 8;
    }

    f32x16 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

    uint4 ra[A_PER_T], rb[B_PER_T];
#define MOE_GLOAD(kt_)                                                    \
  {                                                                       \
    _Pragma("unroll") for (int i = 0; i < A_PER_T; ++i) ra[i] =           \
        *(const uint4 *)(a_src[i] + (kt_) * BK);                          \
    _Pragma("unroll") for (int i = 0; i < B_PER_T; ++i) rb[i] =           \
        *(const uint4 *)(b_src[i] + (kt_) * BK);                          \
  }
#define MOE_SSTORE(buf_)                                                  \
  {                                                                       \
    _Pragma("unroll") for (int i = 0; i < A_PER_T; ++i) {                 \
      const int c = tid + i * 256, row = c / CPR, kc = c % CPR;           \
      smem[buf_][row * CPR + (kc ^ (row & 7))] = ra[i];                   \
    }                                                                     \
    _Pragma("unroll") for (int i = 0; i < B_PER_T; ++i) {                 \
      const int c = tid + i * 256, row = c / CPR, kc = c % CPR;           \
      smem[buf_][(BM + row) * CPR + (kc ^ (row & 7))] = rb[i];            \
    }                                                                     \
  }

    // number of valid 32-row blocks of this wavefront
    const int wrow0 = wm * WTM;
    const int mvalid = rows > wrow0 ? min(MB, (rows - wrow0 + 31) / 32) : 0;

    MOE_GLOAD(0);
    MOE_SSTORE(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) MOE_GLOAD(kt + 1);
      if (mvalid > 0) {
        const uint4 *As = smem[buf];
        const uint4 *Bs = smem[buf] + BM * CPR;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int ch = 2 * kk + (lane >> 5);
          bf16x8 af[MB], bfr[NB];
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const int row = wrow0 + m * 32 + (lane & 31);
            const uint4 v = As[row * CPR + (ch ^ (row & 7))];
            af[m] = *(const bf16x8 *)&v;
          }
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int row = wn * WTN + n * 32 + (lane & 31);
            const uint4 v = Bs[row * CPR + (ch ^ (row & 7))];
            bfr[n] = *(const bf16x8 *)&v;
          }
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            if (m < mvalid) {
#pragma unroll
              for (int n = 0; n < NB; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    af[m], bfr[n], acc[m][n], 0, 0, 0);
            }
          }
        }
      }
      if (kt + 1 < KT) MOE_SSTORE(buf ^ 1);
      __syncthreads();
    }
#undef MOE_GLOAD
#undef MOE_SSTORE

    // Epilogue.  Lane holds column (lane & 31) of each 32x32 block and rows
    // 8*(r/4) + 4*(lane/32) + (r%4), r < 16.
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m >= mvalid) continue;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = wrow0 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const float v = acc[m][n][r];
          if (EPI == EPI_SWIGLU) {
            const float other = __shfl_xor(v, 16, 64);
            if ((lane & 31) < 16 && i < rows) {
              const int col = nt * (BN / 2) + (wn * WTN + n * 32) / 2 + (lane & 15);
              if (col < p.N) {
                const float s = p.row_scale ? p.row_scale[row0 + i] : 1.f;
                const float a = s * silu_f32(v) * other;
                ((uint16_t *)p.C)[(int64_t)(row0 + i) * p.ldc + col] =
                    (uint16_t)f32_to_bf16_bits(a);
              }
            }
          } else {
            const int col = nt * BN + wn * WTN + n * 32 + (lane & 31);
            if (i < rows && col < p.N) {
              if (EPI == EPI_BF16)
                ((uint16_t *)p.C)[(int64_t)(row0 + i) * p.ldc + col] =
                    (uint16_t)f32_to_bf16_bits(v);
              else
                ((float *)p.C)[(int64_t)(row0 + i) * p.ldc + col] =
                    v + (p.bias ? p.bias[col] : 0.f);
            }
          }
        }
      }
    }
  }
}

namespace {

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_cfg(GemmArgs p, int num_cus, int32_t *tile_ws,
                      int64_t max_rows, hipStream_t s) {
  p.NT = EPI == EPI_SWIGLU ? (p.N + BN / 2 - 1) / (BN / 2)
                           : (p.N + BN - 1) / BN;
  int64_t max_tiles;
  if (p.offsets) {
    p.tile_prefix = tile_ws;
    gemm_plan_kernel<<<1, 1024, 0, s>>>(p.offsets, p.G, BM, p.NT, tile_ws);
    max_tiles = ((max_rows + BM - 1) / BM + p.G) * (int64_t)p.NT;
  } else {
    max_tiles = (max_rows + BM - 1) / BM * (int64_t)p.NT;
  }
  int64_t grid = num_cus;  // one 256-thread workgroup per CU
  if (max_tiles < grid) grid = (max_tiles + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  grouped_gemm_kernel<BM, BN, WM, WN, EPI><<<(unsigned)grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_bf16(const uint16_t *x_perm, const int32_t *offsets,
                               const float *s_perm, int n_local, int64_t R_cap,
                               int H, int I, const uint16_t *w_gate,
                               const uint16_t *w_up, uint16_t *a,
                               int32_t *tile_ws, int num_cus, hipStream_t s) {
  GemmArgs p{};
  p.A = x_perm; p.B0 = w_gate; p.B1 = w_up;
  p.b_stride = (int64_t)I * H;
  p.C = a; p.ldc = I; p.row_scale = s_perm;
  p.offsets = offsets; p.G = n_local; p.N = I; p.K = H;
  return launch_cfg<128, 256, 2, 2, EPI_SWIGLU>(p, num_cus, tile_ws, R_cap, s);
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
  return launch_cfg<128, 256, 2, 2, EPI_BF16>(p, num_cus, tile_ws, R_cap, s);
}

hipError_t launch_router_gemm_bf16(const uint16_t *x, const uint16_t *w,
                                   const float *bias, float *logits, int64_t T,
                                   int H, int E, int num_cus, hipStream_t s) {
  GemmArgs p{};
  p.A = x; p.B0 = w; p.b_stride = 0;
  p.C = logits; p.ldc = E;
  p.bias = bias;
  p.offsets = nullptr; p.single_rows = (int)T; p.G = 1; p.N = E; p.K = H;
  return launch_cfg<64, 64, 2, 2, EPI_F32_BIAS>(p, num_cus, nullptr, T, s);
}

}  // namespace moe
