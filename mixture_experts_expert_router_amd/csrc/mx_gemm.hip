// MXFP8 grouped GEMM on gfx950: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3
// operands and one E8M0 scale per 32 values along K (BioNeMo MoE article,
// "MXFP8 Precision Reduces Memory Footprint for Biological Models", and
// "GroupedLinear Optimizes Expert Computation in MoE Models" for grouping and
// the fused GroupedLinear -> ScaledSwiGLU -> GroupedLinear forward/backward).
// Dequantisation happens inside the matrix instruction (each lane half hands
// the scale byte of one 32-value block of its rows), so no dequantised copy
// exists.
//
// C[m, n] = sum_k A[m, k] * B[n, k] * 2^(sa - 127) * 2^(sb - 127)
// A: codes [rows, lda] bytes, K-contiguous, scales [rows, ldas] (byte per 32)
// B: per group g, codes B + g*b_stride, rows [N, ldb]; scales likewise.
// Two grouping modes:
//   ROWSEG: rows of A grouped into expert segments by offsets (forward and
//           data gradients); K fixed.  Tiles listed by a plan kernel.
//   KSEG:   every group has all M x N outputs and its own K range
//           [kseg[g], kseg[g+1]) of transposed operands (weight gradients:
//           K runs over an expert's rows, zero-padded to 256 or 512).
// KSPLIT (data gradient through gate and up): B rows are [B0 row | B1 row]
// along K, the switch at `ksplit`.
//
// Pipeline: BM x BN tiles on 4 wavefronts (each a (BM/WM) x (BN/WN) block of
// 32x32 MFMA tiles; 128 x 128 per wavefront at the 256 x 256 shape, which
// halves the LDS bytes read per FLOP against 64 x 64), K advancing BKB
// values per stage through a STAGES-deep LDS ring filled by direct
// global->LDS loads from inline assembly (explicit vmcnt waits).  A stage
// holds the A and B code rows (BKB bytes each, 16-byte chunks XOR-swizzled
// against bank conflicts) and, per row, the scale dword of the 128 values
// the stage lies in (one dword load per row, packed row after row).  The
// loads run STAGES-1 stages ahead, spread over the MFMAs of the stage being
// computed.  Two 128-value stages measured faster than four 64-value ones
// (fewer barriers per K, twice the MFMAs per stage).  K must be a multiple
// of 128.
//
// Gradient option: FA = kMxE5M2 makes A's elements E5M2 (the matrix
// instruction's A-format field selects bf8), for the backward GEMMs whose A
// operand is a gradient (dY, [dg | du] and their transposes); B stays E4M3.
// The SwiGLU-backward epilogue then also writes the codes of dg and du in
// E5M2, while the codes of a (an activation) stay E4M3.
#include "common.hpp"
#include "mx_codec.hpp"
#include "kernels.hpp"

namespace moe {

struct MxArgs {
  const uint8_t *A, *As;
  int64_t lda, ldas;
  const uint8_t *B0, *B0s, *B1, *B1s;
  int64_t ldb, ldbs, b_stride, bs_stride;
  const int32_t *offsets;       // ROWSEG: [G + 1]
  const int32_t *tile_prefix;   // ROWSEG: [G + 1]
  const int32_t *kseg;          // KSEG: [G + 1] K ranges (multiples of 128)
  int G, M, N, K, NT, MT;
  int r_cap;                    // ROWSEG: row capacity (segments cut at it)
  void *C;
  int64_t ldc, c_stride;
  const float *row_scale;       // SWIGLU, SWIGLU_BWD: s per row (or null)
  float *gu;                    // SWIGLU: g, u out; SWIGLU_BWD: g, u in (fp32)
  int64_t ldgu;                 // u at column offset N of gu (and of dgu)
  uint16_t *dgu;                // SWIGLU_BWD: dg, du out in bf16 (or null)
  float *ds_part;               // SWIGLU_BWD: [rows, NT * WN]
  int ksplit;                   // KSPLIT: K of the B0 part (0 = none)
  uint8_t *q, *qs;              // SWIGLU: row-wise MX codes of a; SWIGLU_BWD:
  int64_t ldq, ldqs;            //   of [dg | du]; from fp32 (null: none)
  // SWIGLU_BWD: column-wise MX copies of dg (t0), du (t1) and a (t2) for the
  // weight gradients, from fp32: codes [N, ldt], scales [N, ldts]; row r of
  // expert e lands at position tpad[e] + (r - first row of e) (segments
  // padded to BM rows).  Null: not written.
  uint8_t *t0, *t0s, *t1, *t1s, *t2, *t2s;
  int64_t ldt, ldts;
  const int32_t *tpad;
};

enum MxMode { MX_ROWSEG = 0, MX_KSEG = 1 };
enum MxEpi { MX_EPI_BF16 = 0, MX_EPI_SWIGLU = 1, MX_EPI_SWIGLU_BWD = 2 };

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// Direct global -> LDS loads: lane l's 16 (or 4) bytes go to LDS byte
// address lds_base + 16 * l (or 4 * l); lds_base is uniform.
__device__ __forceinline__ void mx_load_lds16(uint32_t lds_base, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory");
}
// A pointer the wavefront holds in common, in scalar registers.
template <typename T>
__device__ __forceinline__ T *mx_uniform(T *q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// The same 16 bytes per lane from sbase + voff: a uniform base and a 32-bit
// byte offset per lane (the instruction's SGPR-address form).
__device__ __forceinline__ void mx_load_lds16_so(uint32_t lds_base,
                                                 const void *sbase,
                                                 uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void mx_load_lds4(uint32_t lds_base, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_base), "v"(g) : "memory");
}

template <int N>
__device__ __forceinline__ void mx_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
               :: "i"(N) : "memory");
}

// Physical 16-byte chunk of logical chunk c of an LDS code row with CPR
// chunks: 16 consecutive rows at one logical chunk hit 16 bank groups
// (128-byte rows: rows of equal parity get distinct chunks; 64-byte rows:
// rows equal mod 4 do).
template <int CPR>
__device__ __forceinline__ int mx_swz(int row, int c) {
  return CPR == 8 ? (c ^ ((row >> 1) & 7)) : (c ^ ((row >> 2) & 3));
}

// tile_prefix[e+1] = tile_prefix[e] + ceil(rows_e / BM) * NT, with the
// segments cut at the row capacity r_cap; *err = kDevErrRows when the
// offsets run past it or decrease, else 0 (err may be null).  One block.
__global__ __launch_bounds__(1024) void mx_plan_kernel(
    const int32_t *__restrict__ offsets, int G, int r_cap, int BM, int NT,
    int32_t *__restrict__ prefix, int32_t *__restrict__ err) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (G + 1023) / 1024;
  const int e0 = min(G, tid * per), e1 = min(G, e0 + per);
  auto tiles = [&](int e) {
    int b, en;
    seg_rows(offsets, e, r_cap, b, en);
    return (en - b + BM - 1) / BM * NT;
  };
  int32_t s = 0;
  int bad = 0;
  for (int e = e0; e < e1; ++e) {
    s += tiles(e);
    bad |= seg_bad(offsets, e, r_cap);
  }
  bad = __syncthreads_or(bad);
  if (tid == 0 && err) *err = bad ? kDevErrRows : 0;
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
    prefix[e] = run;
    run += tiles(e);
  }
  if (tid == 1023) prefix[G] = part[1023];
}

// Source row of B-tile row j (0 <= j < BN) and whether it comes from B1:
// SWIGLU alternates 32 gate rows and the 32 matching up rows, so one tile
// yields both operands of SwiGLU for BN/2 output columns, and MFMA blocks
// 2q and 2q+1 of a wavefront hold g and u of the same outputs in each lane.
template <int EPI, int BN>
__device__ __forceinline__ int mx_brow(int nt, int j, int N, bool &up) {
  int col;
  if (EPI == MX_EPI_SWIGLU) {
    const int w = j & 63;
    col = nt * (BN / 2) + (j >> 6) * 32 + (w & 31);
    up = w >= 32;
  } else {
    col = nt * BN + j;
    up = false;
  }
  return min(col, N - 1);
}

// ---- LDS-staged epilogues ------------------------------------------------
// After the K loop the LDS ring is free; each wavefront stages its part of
// the output in a region of its own.  Plain GEMM outputs are staged in bf16
// and leave as 16-byte row pieces.  The SwiGLU epilogues stage fp32 values:
// the MX codes they write are encoded from the fp32 results themselves
// (the quantisation fused into the kernel of the MXFP8 section), never from
// a rounded copy.
//
// fp32 region layout, W columns (W = 64 or 128) per row: column c of row r
// lives at r * W + fphys<W>(r, c).  32-column blocks swap by bit 2 of the
// row (rows r and r + 4, written together by the two wavefront halves in the
// MFMA layout, then hit different banks), and the eight 16-byte chunks of a
// block rotate by r mod 8 (so sixteen rows read at one logical chunk hit
// sixteen different chunk positions).  A block stays within one 128-byte
// span of its row.
template <int W>
__device__ __forceinline__ int fphys(int r, int c) {
  const int blk = (c >> 5) ^ ((r >> 2) & 1);
  const int ch = ((c >> 2) & 7) ^ (r & 7);
  return (blk << 5) | (ch << 2) | (c & 3);
}

// The 32 fp32 values of block b (columns 32b .. 32b+31) of region row r.
template <int W>
__device__ __forceinline__ void f32_block(const float *l, int r, int b,
                                          float (&v)[32]) {
  const float *row = l + r * W + ((b ^ ((r >> 2) & 1)) << 5);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 t = *(const float4 *)(row + ((k ^ (r & 7)) << 2));
    v[4 * k] = t.x; v[4 * k + 1] = t.y; v[4 * k + 2] = t.z; v[4 * k + 3] = t.w;
  }
}

// Row-wise MX encoding of a staged fp32 [NROWS][W] region: block b of region
// row r goes to codes q[(grow0 + r) * ldq + col0 + 32 b] and scale
// qs[(grow0 + r) * ldqs + col0 / 32 + b], for tile rows arow0 + r < rows.
// Lanes take consecutive rows of one block column (conflict-free reads).
template <int W, int NROWS, int F>
__device__ __forceinline__ void mx_quant_rows_f32(const float *l, uint8_t *q,
                                                  int64_t ldq, uint8_t *qs,
                                                  int64_t ldqs, int64_t col0,
                                                  int64_t grow0, int arow0,
                                                  int rows, int lane) {
  constexpr int BPR = W / 32;
  static_assert((NROWS * BPR) % 64 == 0, "region");
  // uniform bases (scalar registers) and 32-bit lane offsets: no 64-bit
  // per-lane address has to stay live across the loop
  uint8_t *qb = mx_uniform(q + grow0 * ldq + col0);
  uint8_t *sbb = mx_uniform(qs + grow0 * ldqs + col0 / 32);
#pragma unroll 1
  for (int it = 0; it < NROWS * BPR / 64; ++it) {
    const int item = it * 64 + lane;
    const int r = item % NROWS, b = item / NROWS;
    float v[32];
    f32_block<W>(l, r, b, v);
    uint32_t c[8];
    const uint32_t sb = mx_encode32_f32_t<F>(v, c);
    if (arow0 + r < rows) {
      uint4 *dst = (uint4 *)(qb + ((uint32_t)r * (uint32_t)ldq + 32u * b));
      dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
      dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
      sbb[(uint32_t)r * (uint32_t)ldqs + b] = (uint8_t)sb;
    }
  }
}

// A staged fp32 [NROWS][W] region rounded to bf16 (nearest even) and written
// to dst[(grow0 + r) * ld + col0 + c] as 16-byte row pieces, for tile rows
// arow0 + r < rows and columns col0 + c < N (N % 8 == 0).
template <int W, int NROWS>
__device__ __forceinline__ void store_f32_as_bf16(const float *l, uint16_t *dst,
                                                  int64_t ld, int64_t col0,
                                                  int N, int64_t grow0,
                                                  int arow0, int rows,
                                                  int lane) {
  constexpr int LPR = W / 8;                 // lanes per row
  constexpr int RPI = 64 / LPR;              // rows per instruction
  uint16_t *db = mx_uniform(dst + grow0 * ld + col0);
#pragma unroll 4
  for (int it = 0; it < NROWS / RPI; ++it) {
    const int r = it * RPI + lane / LPR;
    const int c8 = (lane % LPR) * 8;
    const float4 lo = *(const float4 *)(l + r * W + fphys<W>(r, c8));
    const float4 hi = *(const float4 *)(l + r * W + fphys<W>(r, c8 + 4));
    if (arow0 + r < rows && col0 + c8 < N)
      *(uint4 *)(db + ((uint32_t)r * (uint32_t)ld + (uint32_t)c8)) =
          make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                     pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w));
  }
}

// Column-wise MX encoding straight from the MFMA accumulator layout.  v holds
// this lane's 16 values of column c = c0 + (lane & 31) of a 32 x 32 block
// (rows 8 (i / 4) + 4 h + i % 4, h = lane / 32); lane ^ 32 holds the other
// 16, and the column's 32 values form one MX block.  Its codes go to
// qt[c * ldt + pos0 .. + 32) (the first 16 bytes written by half 0, the rest
// by half 1) and its scale byte to qts[c * ldts + pos0 / 32].  The launcher
// keeps 32 * ldt below 2^32.
template <int F>
__device__ __forceinline__ void mx_quant_col_block(const float (&v)[16],
                                                   int lane, uint8_t *qt,
                                                   uint8_t *qts, int64_t ldt,
                                                   int64_t ldts, int64_t c0,
                                                   int64_t pos0) {
  float mag = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) mag = fmaxf(mag, fabsf(v[i]));
  mag = fmaxf(mag, __shfl_xor(mag, 32, 64));
  const int X = mx_shared_exp_t<F>(mag);
  uint32_t d[4];                 // rows 8q + 4h .. 8q + 4h + 3
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d[q] = pack4_t<F>(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], -X);
  const int h = lane >> 5;
  // half 0 writes rows 0-15 (its d0, d1 and the partner's), half 1 rows 16-31
  const uint32_t x0 = h ? d[0] : d[2], x1 = h ? d[1] : d[3];
  const uint32_t y0 = (uint32_t)__shfl_xor((int)x0, 32, 64);
  const uint32_t y1 = (uint32_t)__shfl_xor((int)x1, 32, 64);
  const uint4 o = h ? make_uint4(y0, d[2], y1, d[3]) : make_uint4(d[0], y0, d[1], y1);
  // uniform base of the block's first column, 32-bit lane offsets
  uint8_t *cb = mx_uniform(qt + c0 * ldt + pos0);
  uint8_t *sb = mx_uniform(qts + c0 * ldts + pos0 / 32);
  const uint32_t c = (uint32_t)(lane & 31);
  *(uint4 *)(cb + (c * (uint32_t)ldt + 16u * h)) = o;
  if (h) sb[c * (uint32_t)ldts] = (uint8_t)(X + 127);
}

// fp32 g and u of 32 tile rows [ar0, ar0 + 32) x 128 columns (g_base and
// u_base point at tile row 0 of the wavefront's first column, both uniform;
// row pitch ld floats) into staged [32][128] fp32 regions at LDS byte
// addresses lg, lu (fphys<128> layout), by direct global -> LDS loads: one
// instruction fills two 512-byte region rows, lane i the physical 16-byte
// chunk i % 32 of row 2 it + i / 32, reading the logical chunk that fphys
// maps there (the map is its own inverse on chunks).  Rows past the tile
// (`rows`) read the tile's last row.  The launcher keeps 256 * ld * 4 below
// 2^32.  The caller waits on vmcnt before reading the regions.
__device__ __forceinline__ void mx_load_gu32(uint32_t lg, uint32_t lu,
                                             const float *g_base,
                                             const float *u_base, int64_t ld,
                                             int ar0, int rows, int lane) {
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int r = 2 * it + (lane >> 5);
    const int pc = lane & 31;
    const int lc = ((((pc >> 3) ^ ((r >> 2) & 1))) << 3) | ((pc & 7) ^ (r & 7));
    const int trow = min(ar0 + r, rows - 1);
    const uint32_t voff = (uint32_t)(trow * (uint32_t)ld + (uint32_t)(lc * 4)) * 4u;
    mx_load_lds16_so(lg + (uint32_t)(it * 1024), g_base, voff);
    mx_load_lds16_so(lu + (uint32_t)(it * 1024), u_base, voff);
  }
}

// SwiGLU forward of one 32-row block (region rows mloc ..): block 2q holds g
// and block 2q+1 the matching u in every lane.  a = s SiLU(g) u goes to the
// fp32 region la ([128][64], fphys<64>); g and u go to HBM in fp32 (gp: the
// wavefront's first row and column of [g | u], null: not written), 32 lanes
// writing 128 contiguous bytes of one row, from a per-row uniform base and a
// 32-bit lane offset.  s_reg: lane l holds the routing scale of region row
// (mloc & 64) + l.
template <int NB>
__device__ __forceinline__ void mx_swiglu_block(const f32x16 (&am)[NB],
                                                int mloc, int lane,
                                                float s_reg, float *la,
                                                float *gp, int64_t ldgu, int N,
                                                int arow0, int rows) {
  const int h = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = mloc + 8 * (r >> 2) + 4 * h + (r & 3);
    const float s = __shfl(s_reg, row & 63, 64);
#pragma unroll
    for (int q = 0; q < NB / 2; ++q) {
      const int col = q * 32 + (lane & 31);
      la[row * 64 + fphys<64>(row, col)] = s * silu_f32(am[2 * q][r]) * am[2 * q + 1][r];
    }
  }
  if (gp == nullptr) return;
  const uint32_t loff = (uint32_t)(4 * h * ldgu) + (uint32_t)(lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int urow = mloc + 8 * (r >> 2) + (r & 3);      // row of half 0
    float *base = mx_uniform(gp + (int64_t)urow * ldgu);
    if (arow0 + urow + 4 * h < rows) {
#pragma unroll
      for (int q = 0; q < NB / 2; ++q) {
        base[loff + q * 32] = am[2 * q][r];
        base[loff + N + q * 32] = am[2 * q + 1][r];
      }
    }
  }
}

// Plain bf16 output of one 32-row block into a staged [128][128] region.
template <int NB>
__device__ __forceinline__ void mx_plain_stage(const f32x16 (&am)[NB], int mloc,
                                               int lane, uint16_t *l) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = mloc + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
#pragma unroll
    for (int n = 0; n < NB; ++n)
      l[row * 128 + st_col<128>(row, n * 32 + (lane & 31))] =
          (uint16_t)f32_to_bf16_bits(am[n][r]);
  }
}

// Lane-xor exchanges inside 32-lane groups: ds_swizzle in bit mode
// (and-mask 31, xor-mask m) for 16, 8, 4; DPP quad permutations for 2, 1.
template <int M>
__device__ __forceinline__ float mx_xor32(float v) {
  const int x = __builtin_bit_cast(int, v);
  int y;
  if constexpr (M == 1) y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  else if constexpr (M == 2) y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  else y = __builtin_amdgcn_ds_swizzle(x, (M << 10) | 0x1F);
  return __builtin_bit_cast(float, y);
}

// Sums v[0..15] over the 32 lanes of each wavefront half by reduce-scatter:
// each exchange step halves the values a lane keeps (the half picked by its
// lane bit) and adds its partner's other half, 8 + 4 + 2 + 1 + 1 exchanges in
// all.  Returns in lane l the total of v[((l & 31) >> 1)].
__device__ __forceinline__ float mx_sum16_over32(const float (&v)[16], int lane) {
  const bool b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  float w[8], x[4], y[2];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j] = (b4 ? v[j + 8] : v[j]) + mx_xor32<16>(b4 ? v[j] : v[j + 8]);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x[j] = (b3 ? w[j + 4] : w[j]) + mx_xor32<8>(b3 ? w[j] : w[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    y[j] = (b2 ? x[j + 2] : x[j]) + mx_xor32<4>(b2 ? x[j] : x[j + 2]);
  const float z = (b1 ? y[1] : y[0]) + mx_xor32<2>(b1 ? y[0] : y[1]);
  return z + mx_xor32<1>(z);
}

// SwiGLU backward of one 32-row block m of a wavefront (tile rows mrow0 =
// arow0 + 32 m ..) against the staged fp32 g, u of its rows (lg, lu, [32][128]
// fphys<128>).  In fp32: a = s SiLU(g) u, dg = da s u SiLU'(g),
// du = da s SiLU(g), ds partial = sum over the wavefront's 128 columns of
// da SiLU(g) u.  dg and du replace g and u in the regions (for the row-wise
// outputs that follow); the column-wise MX codes of dg, du (t0, t1) and of a
// (t2) are written from the registers (dg, du in the gradient format FG, a in
// E4M3), rows past the segment (tile row >=
// rows) counting as zeros, i.e. as the segment's padding.  pos0: padded
// position of the block's first row.  s_reg: lane l holds the routing scale
// of wavefront row (32 m & 64) + l.
template <int BN, int WN, int NB, int FG>
__device__ __forceinline__ void mx_swiglu_bwd_block(
    const MxArgs &p, const f32x16 (&am)[NB], int m, int lane, int arow0,
    int rows, int row0, int nt, int wn, float s_reg, float *lg, float *lu,
    int64_t col0, int64_t pos0) {
  const int mrow0 = arow0 + 32 * m;
  const int h = lane >> 5;
  float part[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) part[r] = 0.f;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * h + (r & 3);
      const int o = row * 128 + fphys<128>(row, n * 32 + (lane & 31));
      const float s = __shfl(s_reg, (32 * m + row) & 63, 64);
      const float da = am[n][r];
      const float g = lg[o], u = lu[o];
      const float sg = sigmoid_f32(g);
      const float sl = g * sg;
      const float dsl = sg * (1.f + g * (1.f - sg));
      part[r] += da * sl * u;
      lg[o] = da * s * u * dsl;                       // dg
      lu[o] = da * s * sl;                            // du
      v[r] = mrow0 + row < rows ? s * sl * u : 0.f;   // a (padding rows: 0)
    }
    const int64_t c = col0 + n * 32;
    if (p.t2) mx_quant_col_block<kMxE4M3>(v, lane, p.t2, p.t2s, p.ldt, p.ldts, c, pos0);
    if (p.t0) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float *src = t ? lu : lg;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * h + (r & 3);
          const float x = src[row * 128 + fphys<128>(row, n * 32 + (lane & 31))];
          v[r] = mrow0 + row < rows ? x : 0.f;
        }
        if (t) mx_quant_col_block<FG>(v, lane, p.t1, p.t1s, p.ldt, p.ldts, c, pos0);
        else mx_quant_col_block<FG>(v, lane, p.t0, p.t0s, p.ldt, p.ldts, c, pos0);
      }
    }
    // keep the column blocks in sequence: interleaving them only raises the
    // number of live values (the accumulators already fill the registers)
    __builtin_amdgcn_sched_barrier(0);
  }
  const float tot = mx_sum16_over32(part, lane);
  const int r = (lane & 31) >> 1;
  const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
  const int ntw = p.NT * WN;
  float *dp = mx_uniform(p.ds_part + (int64_t)(row0 + mrow0) * ntw + nt * WN + wn);
  if ((lane & 1) == 0 && mrow0 + rr < rows) dp[(uint32_t)rr * (uint32_t)ntw] = tot;
}

template <int MODE, int EPI, int FA, int BM, int BN, int WM, int WN, int STAGES, int BKB>
__global__ __launch_bounds__(256) void mx_gemm_kernel(MxArgs p) {
  // BKB: K values (code bytes) per stage; a stage carries, for every A and B
  // row, its 128 codes and the scale dword of their four 32-value blocks.
  // The K loop below is pipelined for two such stages.
  static_assert(BKB == 128 && STAGES == 2, "two stages of 128 K values");
  constexpr int CPR = BKB / 16;                        // 16-byte chunks per row
  constexpr int WTM = BM / WM, WTN = BN / WN, MB = WTM / 32, NB = WTN / 32;
  constexpr int CODE_CHUNKS = (BM + BN) * CPR;
  constexpr int LC = CODE_CHUNKS / 256;                // code loads per thread
  constexpr int LS = (BM + BN) / 256;                  // scale loads per thread
  constexpr int L = LC + LS;
  constexpr int SCALE_OFF = CODE_CHUNKS * 16;          // bytes
  constexpr int STAGE_BYTES = SCALE_OFF + (BM + BN) * 4;
  static_assert(WM * WN == 4 && MB >= 1 && MB <= 4 && NB >= 1, "tile");
  static_assert(CODE_CHUNKS % 256 == 0 && (BM + BN) % 256 == 0, "load split");
  static_assert(L <= 63, "vmcnt range");
  static_assert(STAGE_BYTES % 16 == 0, "stage alignment");
  static_assert(STAGES * STAGE_BYTES >= WM * WN * WTM * WTN * 2,
                "the ring must hold every wavefront's epilogue region");
  __shared__ uint4 smem[STAGES * STAGE_BYTES / 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  int total;
  if (MODE == MX_ROWSEG) total = p.tile_prefix[p.G];
  else total = p.G * p.MT * p.NT;
  const int t = xcd_tile(blockIdx.x, total);
  if (t < 0) return;

  int e, row0, rows, nt, mt, k0, KT;
  int r_begin = 0;                // ROWSEG: first row of the tile's segment
  if (MODE == MX_ROWSEG) {
    e = upper_bound_minus1(p.tile_prefix, p.G, t);
    int r_end;
    seg_rows(p.offsets, e, p.r_cap, r_begin, r_end);
    const int local = t - p.tile_prefix[e];
    const int mtiles = (r_end - r_begin + BM - 1) / BM;
    banded_mn(local, mtiles, p.NT, 8, mt, nt);
    row0 = r_begin + mt * BM;
    rows = min(BM, r_end - row0);
    k0 = 0;
    KT = p.K / BKB;
  } else {
    const int per_g = p.MT * p.NT;
    e = t / per_g;
    banded_mn(t - e * per_g, p.MT, p.NT, 8, mt, nt);
    row0 = mt * BM;
    rows = min(BM, p.M - row0);
    k0 = p.kseg[e];
    KT = (p.kseg[e + 1] - k0) / BKB;
  }
  // The tile's coordinates come from memory the kernel cannot prove
  // unchanged; say that they are uniform, so that the addressing below
  // stays in scalar registers.
  e = __builtin_amdgcn_readfirstlane(e);
  r_begin = __builtin_amdgcn_readfirstlane(r_begin);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  nt = __builtin_amdgcn_readfirstlane(nt);
  k0 = __builtin_amdgcn_readfirstlane(k0);
  KT = __builtin_amdgcn_readfirstlane(KT);

  // ---- load sources ------------------------------------------------------
  // Code load i moves chunks q = (wid*LC + i)*64 + lane of a stage: stage row
  // q / CPR (eight 128-byte rows per instruction), chunk q % CPR.  Rows < BM
  // are A rows (tile rows), the rest B rows (output columns).  The eight rows
  // of one instruction are all A or all B rows, and for SwiGLU all gate or
  // all up rows, so the instruction reads from one uniform base plus a 32-bit
  // per-lane offset below 256 row pitches (the stage's K offset is added to
  // it).  Past the K split (KSPLIT) B rows read B1 at K - ksplit.
  // Scale load j moves the dword of row (wid*LS + j)*64 + lane through a
  // per-lane pointer; past the K split a uniform delta moves B rows to B1.
  const int colstep = EPI == MX_EPI_SWIGLU ? BN / 2 : BN;
  const int64_t bcol0 = (int64_t)nt * colstep;
  const char *baseA = (const char *)p.A + (int64_t)row0 * p.lda + k0;
  const int64_t gB = (int64_t)e * p.b_stride + bcol0 * p.ldb + k0;
  const char *baseB0 = (const char *)p.B0 + gB;
  const char *baseB1 = (const char *)p.B1 + gB;
  const char *baseBk = p.ksplit ? (const char *)p.B1 + gB - p.ksplit : baseB0;
  uint32_t voff[LC];
  const char *blo[LC], *bhi[LC];      // bases below / past the K split
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const int row8 = (wid * LC + i) * (64 / CPR);            // first stage row
    const bool up = EPI == MX_EPI_SWIGLU && ((row8 - BM) & 63) >= 32;
    blo[i] = mx_uniform(row8 < BM ? baseA : up ? baseB1 : baseB0);
    bhi[i] = mx_uniform(row8 < BM ? baseA : baseBk);
    const int q = (wid * LC + i) * 64 + lane;
    const int row = q / CPR, c = q % CPR;
    if (row < BM) {
      voff[i] = (uint32_t)(min(row, rows - 1) * p.lda) + (uint32_t)(mx_swz<CPR>(row, c) * 16);
    } else {
      bool up;
      const int col = mx_brow<EPI, BN>(nt, row - BM, p.N, up);
      voff[i] = (uint32_t)((col - bcol0) * p.ldb) + (uint32_t)(mx_swz<CPR>(row, c) * 16);
    }
  }
  const char *sptr[LS];
  const int64_t sdelta = p.ksplit ? ((const char *)p.B1s - (const char *)p.B0s) - p.ksplit / 32 : 0;
#pragma unroll
  for (int j = 0; j < LS; ++j) {
    const int row = (wid * LS + j) * 64 + lane;
    if (row < BM) {
      sptr[j] = (const char *)p.As + (int64_t)(row0 + min(row, rows - 1)) * p.ldas + k0 / 32;
    } else {
      bool up;
      const int col = mx_brow<EPI, BN>(nt, row - BM, p.N, up);
      sptr[j] = (const char *)(up ? p.B1s : p.B0s) + (int64_t)e * p.bs_stride +
                (int64_t)col * p.ldbs + k0 / 32;
    }
  }

  // Load i of stage ks into ring buffer b (i a compile-time index once
  // unrolled; ks and b uniform).
  auto issue = [&](int i, int b, int ks) {
    const uint32_t sb = lds0 + (uint32_t)(b * STAGE_BYTES);
    const bool hi = p.ksplit && ks * BKB >= p.ksplit;
    if (i < LC) {
      mx_load_lds16_so(sb + (uint32_t)((wid * LC + i) * 1024), hi ? bhi[i] : blo[i],
                       voff[i] + (uint32_t)(ks * BKB));
    } else {
      const int j = i - LC;
      const bool isB = (wid * LS + j) * 64 >= BM;
      mx_load_lds4(sb + (uint32_t)(SCALE_OFF + (wid * LS + j) * 256),
                   sptr[j] + (int64_t)(ks * BKB / 128) * 4 + (hi && isB ? sdelta : 0));
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

  const int arow0 = wm * WTM, brow0 = wn * WTN;
  const int h = lane >> 5;

  // Fragments of one 64-value step: A block m and B block n.  Operand layout
  // of the 32x32x64 f8 instruction: lane half h holds K [16h, 16h+16) in its
  // first four registers and [32+16h, 48+16h) in the last four; block b (K
  // [32b, 32b+32)) takes its scale from lane half b.  In 16-byte chunks of
  // the 64-value step: h and 2 + h.
  auto read_a = [&](int b, int kk, i32x8 &dst, int m) {
    const uint4 *As = (const uint4 *)((const char *)smem + b * STAGE_BYTES);
    const int row = arow0 + m * 32 + (lane & 31);
    const uint4 v0 = As[row * CPR + mx_swz<CPR>(row, 4 * kk + h)];
    const uint4 v1 = As[row * CPR + mx_swz<CPR>(row, 4 * kk + 2 + h)];
    dst = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
  };
  auto read_b = [&](int b, int kk, i32x8 &dst, int n) {
    const uint4 *Bs = (const uint4 *)((const char *)smem + b * STAGE_BYTES) + BM * CPR;
    const int row = brow0 + n * 32 + (lane & 31);
    const uint4 v0 = Bs[row * CPR + mx_swz<CPR>(row, 4 * kk + h)];
    const uint4 v1 = Bs[row * CPR + mx_swz<CPR>(row, 4 * kk + 2 + h)];
    dst = i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
  };
  // Scale dwords of a stage (four E8M0 bytes: the 32-value blocks of its 128
  // values) for this lane's A rows and B rows.
  auto read_s = [&](int b, uint32_t (&sa)[MB], uint32_t (&sbv)[NB]) {
    const uint32_t *Ssc = (const uint32_t *)((const char *)smem + b * STAGE_BYTES + SCALE_OFF);
#pragma unroll
    for (int m = 0; m < MB; ++m) sa[m] = Ssc[arow0 + m * 32 + (lane & 31)];
#pragma unroll
    for (int n = 0; n < NB; ++n) sbv[n] = Ssc[BM + brow0 + n * 32 + (lane & 31)];
  };
  // Order in which a step consumes fragments (m-major MFMAs): A0, B0..B(NB-1),
  // A1..A(MB-1).  read_next(k) reads the k-th of them into (af, bf).
  auto read_next = [&](int k, int b, int kk, i32x8 (&af)[MB], i32x8 (&bf)[NB]) {
    if (k == 0) read_a(b, kk, af[0], 0);
    else if (k <= NB) read_b(b, kk, bf[k - 1], k - 1);
    else read_a(b, kk, af[k - NB], k - NB);
  };
  constexpr int NFR = MB + NB;                          // fragments per step

  // Prologue: stages 0 and 1 (clamped) in flight, stage 0 landed, its scales
  // and first step's fragments read.  An expert without rows (KSEG, KT == 0)
  // loads nothing and stores zeros.
  i32x8 af0[MB], bf0[NB], af1[MB], bf1[NB];
  uint32_t sa[MB], sbv[NB], sa_n[MB], sbv_n[NB];
  if (KT > 0) {
#pragma unroll
    for (int i = 0; i < L; ++i) issue(i, 0, 0);
#pragma unroll
    for (int i = 0; i < L; ++i) issue(i, 1, min(1, KT - 1));
    mx_wait_barrier<L>();
    read_s(0, sa, sbv);
#pragma unroll
    for (int k = 0; k < NFR; ++k) read_next(k, 0, 0, af0, bf0);

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1, nb = cur ^ 1;
      const int ks = min(kt + 2, KT - 1);
      // Step 0 on (af0, bf0); the fragments of step 1 are read meanwhile.
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int f = m * NB + n;
          acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af0[m], bf0[n], acc[m][n], FA, kMxE4M3, 0, (int)((sa[m] >> (8 * h)) & 0xffu),
              0, (int)((sbv[n] >> (8 * h)) & 0xffu));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int k = 0; k < NFR; ++k)
            if (f == k + k / 2) read_next(k, cur, 1, af1, bf1);
          __builtin_amdgcn_sched_barrier(0);
        }
      // Step 1 on (af1, bf1).  After its first two MFMAs: stage kt+1 has landed
      // (own loads, then the barrier for everyone's) and nobody reads buffer
      // `cur` any more; so the loads of stage kt+2 go into it, and the scales
      // and first fragments of stage kt+1 are read from buffer nb.
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int g = m * NB + n;
          acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              af1[m], bf1[n], acc[m][n], FA, kMxE4M3, 0, (int)((sa[m] >> (8 * (2 + h))) & 0xffu),
              0, (int)((sbv[n] >> (8 * (2 + h))) & 0xffu));
          __builtin_amdgcn_sched_barrier(0);
          if (g == 1) {
            mx_wait_barrier<0>();
            read_s(nb, sa_n, sbv_n);
          }
          if (g >= 2) {
            constexpr int SL = MB * NB - 2;                 // slots for the rest
#pragma unroll
            for (int i = 0; i < L; ++i)
              if (i * SL / L == g - 2) issue(i, cur, ks);
#pragma unroll
            for (int k = 0; k < NFR; ++k)
              if (g - 2 == k) read_next(k, nb, 0, af0, bf0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int m = 0; m < MB; ++m) sa[m] = sa_n[m];
#pragma unroll
      for (int n = 0; n < NB; ++n) sbv[n] = sbv_n[n];
    }
  }
  mx_wait_barrier<0>();

  // Epilogues, one 32-row block at a time with constant block indices (the
  // accumulators stay in registers).
  uint16_t *lw = (uint16_t *)smem + (size_t)wid * (WTM * WTN);   // per-wavefront region
  // Routing scales of the wavefront's 128 rows, lane l: rows l and 64 + l.
  // Loaded once here: read inside the epilogue loops, each load would wait
  // behind the previous row's ds_part store (the pointers may alias).
  float s_lo = 1.f, s_hi = 1.f;
  if constexpr (EPI != MX_EPI_BF16) {
    if (p.row_scale) {
      if (arow0 + lane < rows) s_lo = p.row_scale[row0 + arow0 + lane];
      if (arow0 + 64 + lane < rows) s_hi = p.row_scale[row0 + arow0 + 64 + lane];
    }
  }
  if constexpr (EPI == MX_EPI_SWIGLU) {
    static_assert(WTM == 128 && WTN == 128, "SwiGLU staging expects 128x128 wavefront tiles");
    // region: a in fp32, [128][64]; g and u go to HBM from the registers
    float *la = (float *)lw;
    const int64_t col0 = (int64_t)nt * (BN / 2) + brow0 / 2;
    const int64_t grow0 = row0 + arow0;
    float *gp = p.gu ? p.gu + grow0 * p.ldgu + col0 : nullptr;
    // One 32-row block per pass (rolled; see the backward epilogue below).
    const int lane_id = lane;
#pragma unroll 1
    for (int m = 0; m < MB; ++m) {
      int ln = lane_id;
      asm volatile("" : "+v"(ln));
      f32x16 cur[NB];
      switch (m) {
#define MX_FWD_COPY(mm) \
        case mm: \
          _Pragma("unroll") for (int n = 0; n < NB; ++n) cur[n] = acc[mm][n]; \
          break;
        MX_FWD_COPY(0) MX_FWD_COPY(1) MX_FWD_COPY(2) MX_FWD_COPY(3)
#undef MX_FWD_COPY
      }
      mx_swiglu_block<NB>(cur, m * 32, ln, m < 2 ? s_lo : s_hi, la, gp, p.ldgu, p.N, arow0, rows);
    }
    __syncthreads();
    store_f32_as_bf16<64, 128>(la, (uint16_t *)p.C, p.ldc, col0, p.N, grow0, arow0, rows, lane);
    if (p.q) mx_quant_rows_f32<64, 128, kMxE4M3>(la, p.q, p.ldq, p.qs, p.ldqs, col0, grow0, arow0, rows, lane);
  } else if constexpr (EPI == MX_EPI_SWIGLU_BWD) {
    static_assert(WTM == 128 && WTN == 128 && MB == 4, "staging expects 128x128 wavefront tiles");
    // region: fp32 g and u of one 32-row block x 128 columns ([32][128] each)
    float *lg = (float *)lw, *lu = lg + 32 * 128;
    const uint32_t lgb = lds0 + (uint32_t)(wid * WTM * WTN * 2);
    const uint32_t lub = lgb + 32 * 128 * 4;
    const int64_t col0 = (int64_t)nt * BN + brow0;
    const float *gb = mx_uniform(p.gu + (int64_t)row0 * p.ldgu + col0);
    const float *ub = mx_uniform(gb + p.N);
    // padded position of tile row 0 in the column-wise copies: tile rows start
    // at the segment's first row + mt * BM, padded at tpad[e] + mt * BM
    const int64_t pbase = p.tpad ? (int64_t)p.tpad[e] + (row0 - r_begin) : 0;
    const int lane_id = lane;
    // One 32-row block per pass, not unrolled: the pass copies its block's
    // accumulators (constant indices in each case of the switch) and the
    // rest of the body exists once, which keeps the live values in bounds.
#pragma unroll 1
    for (int m = 0; m < MB; ++m) {
      const int ar0 = arow0 + 32 * m;
      const int64_t grow0 = row0 + ar0;
      // An opaque copy of the lane index: the LDS and global offsets derived
      // from it are recomputed in each pass instead of being hoisted out of
      // the loop and kept live (which spills them).
      int lane = lane_id;
      asm volatile("" : "+v"(lane));
      f32x16 cur[NB];
      switch (m) {
#define MX_BWD_COPY(mm) \
        case mm: \
          _Pragma("unroll") for (int n = 0; n < NB; ++n) cur[n] = acc[mm][n]; \
          break;
        MX_BWD_COPY(0) MX_BWD_COPY(1) MX_BWD_COPY(2) MX_BWD_COPY(3)
#undef MX_BWD_COPY
      }
      mx_load_gu32(lgb, lub, gb, ub, p.ldgu, ar0, rows, lane);
      mx_wait_barrier<0>();
      mx_swiglu_bwd_block<BN, WN, NB, FA>(p, cur, m, lane, arow0, rows, row0, nt, wn,
                                      m < 2 ? s_lo : s_hi, lg, lu, col0, pbase + ar0);
      __syncthreads();
      if (p.dgu) {
        store_f32_as_bf16<128, 32>(lg, p.dgu, p.ldgu, col0, p.N, grow0, ar0, rows, lane);
        store_f32_as_bf16<128, 32>(lu, p.dgu + p.N, p.ldgu, col0, p.N, grow0, ar0, rows, lane);
      }
      if (p.q) {
        mx_quant_rows_f32<128, 32, FA>(lg, p.q, p.ldq, p.qs, p.ldqs, col0, grow0, ar0, rows, lane);
        mx_quant_rows_f32<128, 32, FA>(lu, p.q, p.ldq, p.qs, p.ldqs, p.N + col0, grow0, ar0, rows, lane);
      }
      __syncthreads();
    }
  } else {
    static_assert(WTM == 128 && WTN == 128, "staging expects 128x128 wavefront tiles");
    const int64_t base = (MODE == MX_KSEG) ? (int64_t)e * p.c_stride : 0;
#define MX_PL_BLOCK(m) \
    if constexpr (MB > (m)) mx_plain_stage<NB>(acc[m], (m) * 32, lane, lw);
    MX_PL_BLOCK(0) MX_PL_BLOCK(1) MX_PL_BLOCK(2) MX_PL_BLOCK(3)
#undef MX_PL_BLOCK
    __syncthreads();
    store_staged<128, 128>(lw, (uint16_t *)p.C + base, p.ldc,
                              (int64_t)nt * BN + brow0, p.N, row0 + arow0,
                              arow0, rows, lane);
  }
}

// ds[r] = sum_j ds_part[r, j] in ascending j (fixed order: deterministic).
__global__ void mx_ds_reduce_kernel(const float *__restrict__ part, int nparts,
                                    const int32_t *__restrict__ R_ptr,
                                    float *__restrict__ ds) {
  const int R = *R_ptr;
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < R;
       r += gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int j = 0; j < nparts; ++j) s += part[(int64_t)r * nparts + j];
    ds[r] = s;
  }
}

namespace {

// Tile shape: 256 x 256 on 2 x 2 wavefronts of 128 x 128; STAGES stages of
// BKB K values: (256 + 256) x BKB code bytes + 2 KB of scales each.
#ifndef MOE_MX_CFG
#define MOE_MX_CFG 256, 256, 2, 2, 2, 128
#endif
constexpr int kMxCfg[6] = {MOE_MX_CFG};
constexpr int kMxBM = kMxCfg[0], kMxBN = kMxCfg[1], kMxWN = kMxCfg[3];

template <int MODE, int EPI, int FA>
hipError_t mx_launch(const MxArgs &p, int64_t max_tiles, hipStream_t s) {
  mx_gemm_kernel<MODE, EPI, FA, MOE_MX_CFG>
      <<<(unsigned)tile_grid(max_tiles), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

size_t mx_ds_parts(int64_t N) {
  return (size_t)((N + kMxBN - 1) / kMxBN) * kMxWN;
}

hipError_t launch_mx_rowseg(const MxGemmDesc &d, int epi, int num_cus,
                            hipStream_t s) {
  MxArgs p{};
  p.A = d.A; p.As = d.As; p.lda = d.lda; p.ldas = d.ldas;
  p.B0 = d.B0; p.B0s = d.B0s; p.B1 = d.B1; p.B1s = d.B1s;
  p.ldb = d.ldb; p.ldbs = d.ldbs; p.b_stride = d.b_stride; p.bs_stride = d.bs_stride;
  p.offsets = d.offsets; p.G = d.G; p.N = d.N; p.K = d.K;
  p.C = d.C; p.ldc = d.ldc; p.row_scale = d.row_scale;
  p.gu = d.gu; p.ldgu = d.ldgu; p.dgu = d.dgu; p.ds_part = d.ds_part;
  p.q = d.q; p.qs = d.qs; p.ldq = d.ldq; p.ldqs = d.ldqs;
  p.t0 = d.t0; p.t0s = d.t0s; p.t1 = d.t1; p.t1s = d.t1s;
  p.t2 = d.t2; p.t2s = d.t2s;
  p.ldt = d.ldt; p.ldts = d.ldts; p.tpad = d.tpad;
  p.ksplit = d.ksplit;
  const int cols = epi == MX_EPI_SWIGLU ? kMxBN / 2 : kMxBN;
  p.NT = (d.N + cols - 1) / cols;
  p.tile_prefix = d.tile_ws;
  p.r_cap = (int)d.R_cap;
  mx_plan_kernel<<<1, 1024, 0, s>>>(d.offsets, d.G, p.r_cap, kMxBM, p.NT,
                                    d.tile_ws, d.err);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // 32-bit lane offsets of the epilogues' stores (row pitches of the
  // column-wise copies, of the row-wise codes and of the outputs).
  if ((int64_t)32 * d.ldt >= (1ll << 32) || (int64_t)256 * d.ldq >= (1ll << 32) ||
      (int64_t)256 * d.ldc * 2 >= (1ll << 32) || (int64_t)256 * d.ldgu * 4 >= (1ll << 32))
    return hipErrorInvalidValue;
  // SwiGLU backward: 32-bit byte offsets within a tile's rows of fp32 g|u.
  if (epi == MX_EPI_SWIGLU_BWD && (int64_t)kMxBM * d.ldgu * 4 >= (1ll << 32))
    return hipErrorInvalidValue;
  const int64_t max_tiles = ((d.R_cap + kMxBM - 1) / kMxBM + d.G) * (int64_t)p.NT;
  // A in E5M2 only where A is a gradient: the SwiGLU backward and dX
  if (d.fa == kMxE5M2 && epi == MX_EPI_SWIGLU) return hipErrorInvalidValue;
  if (epi == MX_EPI_SWIGLU)
    err = mx_launch<MX_ROWSEG, MX_EPI_SWIGLU, kMxE4M3>(p, max_tiles, s);
  else if (epi == MX_EPI_SWIGLU_BWD)
    err = d.fa == kMxE5M2
              ? mx_launch<MX_ROWSEG, MX_EPI_SWIGLU_BWD, kMxE5M2>(p, max_tiles, s)
              : mx_launch<MX_ROWSEG, MX_EPI_SWIGLU_BWD, kMxE4M3>(p, max_tiles, s);
  else
    err = d.fa == kMxE5M2 ? mx_launch<MX_ROWSEG, MX_EPI_BF16, kMxE5M2>(p, max_tiles, s)
                          : mx_launch<MX_ROWSEG, MX_EPI_BF16, kMxE4M3>(p, max_tiles, s);
  if (err != hipSuccess || epi != MX_EPI_SWIGLU_BWD) return err;
  mx_ds_reduce_kernel<<<(unsigned)num_cus, 256, 0, s>>>(
      d.ds_part, p.NT * kMxWN, d.offsets + d.G, d.ds);
  return hipGetLastError();
}

hipError_t launch_mx_kseg(const MxGemmDesc &d, int num_cus, hipStream_t s) {
  (void)num_cus;
  MxArgs p{};
  p.A = d.A; p.As = d.As; p.lda = d.lda; p.ldas = d.ldas;
  p.B0 = d.B0; p.B0s = d.B0s; p.ldb = d.ldb; p.ldbs = d.ldbs;
  p.b_stride = 0; p.bs_stride = 0;
  p.kseg = d.kseg; p.G = d.G; p.M = d.M; p.N = d.N;
  p.MT = (d.M + kMxBM - 1) / kMxBM;
  p.NT = (d.N + kMxBN - 1) / kMxBN;
  p.C = d.C; p.ldc = d.ldc; p.c_stride = d.c_stride;
  const int64_t tiles = (int64_t)d.G * p.MT * p.NT;
  return d.fa == kMxE5M2 ? mx_launch<MX_KSEG, MX_EPI_BF16, kMxE5M2>(p, tiles, s)
                         : mx_launch<MX_KSEG, MX_EPI_BF16, kMxE4M3>(p, tiles, s);
}

}  // namespace moe
