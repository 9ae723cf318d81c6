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
  void *C;
  int64_t ldc, c_stride;
  const float *row_scale;       // SWIGLU, SWIGLU_BWD: s per row (or null)
  uint16_t *gu;                 // SWIGLU: g,u out; SWIGLU_BWD: g,u in
  int64_t ldgu;                 // u at column offset N of gu
  uint16_t *dgu;                // SWIGLU_BWD: dg, du out [rows, ldgu]
  float *ds_part;               // SWIGLU_BWD: [rows, NT * WN]
  int ksplit;                   // KSPLIT: K of the B0 part (0 = none)
  uint8_t *q, *qs;              // SWIGLU(_BWD): row-wise MX copy of the
  int64_t ldq, ldqs;            //   bf16 output (null: none)
  // SWIGLU_BWD: column-wise MX copies of dg (t0) and du (t1) for the weight
  // gradients: codes [N, ldt], scales [N, ldts]; row r of expert e lands at
  // position tpad[e] + (r - offsets[e]) (segments padded to BM rows).
  uint8_t *t0, *t0s, *t1, *t1s;
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

// tile_prefix[e+1] = tile_prefix[e] + ceil(rows_e / BM) * NT.  One block.
__global__ __launch_bounds__(1024) void mx_plan_kernel(
    const int32_t *__restrict__ offsets, int G, int BM, int NT,
    int32_t *__restrict__ prefix) {
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
    prefix[e] = run;
    run += (offsets[e + 1] - offsets[e] + BM - 1) / BM * NT;
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
// After the K loop the LDS ring is free.  Each wavefront stages its part of
// the output in a region of its own and writes it back to HBM as 16-byte
// row pieces (8 lanes per 128-byte row), instead of 2-byte stores per lane.
// Region rows are 128 bytes (64 bf16) for SwiGLU outputs, 256 bytes (128
// bf16) for the SwiGLU-backward g, u, dg, du tiles.

// Row-wise MX encoding of a staged [NROWS][W] bf16 region (st_col<W>
// layout: the XOR by 32 columns moves whole 32-column blocks, so every block
// is 64 contiguous bytes).  Block b of region row r goes to codes
// q[(grow0 + r) * ldq + col0 + 32 b] and scale qs[(grow0 + r) * ldqs +
// col0 / 32 + b], for tile rows arow0 + r < rows.  The values are the bf16
// values staged for the output, so the codes equal a row quantisation of
// that output.
template <int W, int NROWS>
__device__ __forceinline__ void mx_quant_staged(const uint16_t *l, uint8_t *q,
                                                int64_t ldq, uint8_t *qs,
                                                int64_t ldqs, int64_t col0,
                                                int64_t grow0, int arow0,
                                                int rows, int lane) {
  static_assert(W % 32 == 0 && (NROWS * W / 32) % 64 == 0, "region");
  constexpr int BPR = W / 32;                  // blocks per row
#pragma unroll 1
  for (int it = 0; it < NROWS * BPR / 64; ++it) {
    const int item = it * 64 + lane;
    const int r = item / BPR, b = item % BPR;
    const int pb = st_col<W>(r, b * 32) / 32;  // physical block
    const uint4 *src = (const uint4 *)(l + r * W + pb * 32);
    uint4 in[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) in[k] = src[k];
    uint32_t c[8];
    const uint32_t sb = mx_encode32(in, c);
    if (arow0 + r < rows) {
      uint4 *dst = (uint4 *)(q + (grow0 + r) * ldq + col0 + 32 * b);
      dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
      dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
      qs[(grow0 + r) * ldqs + col0 / 32 + b] = (uint8_t)sb;
    }
  }
}

// Column-wise MX encoding of a staged [NROWS][W] bf16 region: blocks of 32
// region rows down each column.  Block b of column c goes to codes
// qt[(col0 + c) * ldt + pos0 + 32 b] and scale qts[(col0 + c) * ldts +
// (pos0 + 32 b) / 32]; region rows at or past `valid` count as zeros (the
// segment's padding).  Pass it handles block b of 64 neighbouring columns,
// one per lane, so each of its 32 LDS reads covers 128 contiguous bytes of
// one region row; every read is issued unconditionally (rows past `valid`
// are read and then replaced by zero), so the reads are all in flight
// together instead of each behind its own branch and wait.
template <int W, int NROWS>
__device__ __forceinline__ void mx_quant_staged_cols(const uint16_t *l,
                                                     uint8_t *qt, uint8_t *qts,
                                                     int64_t ldt, int64_t ldts,
                                                     int64_t col0, int64_t pos0,
                                                     int valid, int lane) {
  constexpr int BPC = NROWS / 32;              // blocks per column
  static_assert(NROWS % 32 == 0 && W % 64 == 0, "region");
#pragma unroll 1
  for (int it = 0; it < (W / 64) * BPC; ++it) {
    const int b = it % BPC, c = (it / BPC) * 64 + lane;
    uint32_t v[32];                            // bf16 bit patterns
    uint32_t mag = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int r = b * 32 + j;
      const uint32_t x = l[r * W + st_col<W>(r, c)];
      v[j] = r < valid ? x : 0u;
      mag = max(mag, v[j] & 0x7fffu);
    }
    const int X = mx_shared_exp_bf16(mag);
    uint32_t pk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pk[j] = e4m3_pack4(bf16_bits_to_f32(v[4 * j]), bf16_bits_to_f32(v[4 * j + 1]),
                         bf16_bits_to_f32(v[4 * j + 2]), bf16_bits_to_f32(v[4 * j + 3]), -X);
    uint4 *dst = (uint4 *)(qt + (col0 + c) * ldt + pos0 + 32 * b);
    dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    qts[(col0 + c) * ldts + (pos0 + 32 * b) / 32] = (uint8_t)(X + 127);
  }
}

// g and u rows [arow0, arow0 + NROWS) of a tile (tile-relative; g_base and
// u_base point at the tile's row 0 and first column, both uniform) into a
// wavefront's staged [NROWS][128] regions at LDS byte addresses lg, lu
// (st_col<128> layout) by direct global -> LDS loads, four 256-byte rows per
// instruction: lane i fills region row 4*it + i/16 at column position
// 8*(i%16), so it reads the column that st_col maps there.  Rows past the
// tile (`rows`) read the tile's last row (their outputs are never stored):
// no branches, and one 32-bit offset per row serves both loads, so every
// load is in flight at once.  The launcher keeps 256 * ld * 2 below 2^32.
// The caller waits on vmcnt before reading the regions.
template <int NROWS>
__device__ __forceinline__ void mx_load_gu_staged(uint32_t lg, uint32_t lu,
                                                  const uint16_t *g_base,
                                                  const uint16_t *u_base,
                                                  int64_t ld, int arow0,
                                                  int rows, int lane) {
#pragma unroll
  for (int it = 0; it < NROWS / 4; ++it) {
    const int r = it * 4 + (lane >> 4);
    const int c = ((lane & 15) * 8) ^ ((it & 1) * 32);   // st_col<128>(r, .)
    const int trow = min(arow0 + r, rows - 1);
    const uint32_t voff = (uint32_t)(trow * (uint32_t)ld + (uint32_t)c) * 2u;
    mx_load_lds16_so(lg + (uint32_t)(it * 1024), g_base, voff);
    mx_load_lds16_so(lu + (uint32_t)(it * 1024), u_base, voff);
  }
}

// SwiGLU forward, one 32-row block: block 2q holds g and block 2q+1 the
// matching u in every lane.  s_reg: lane l holds the routing scale of
// region row (mloc & 64) + l.
template <int NB>
__device__ __forceinline__ void mx_swiglu_stage(
    const f32x16 (&am)[NB], int mloc, int lane, float s_reg, uint16_t *l0,
    uint16_t *l1, int phase) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = mloc + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const float s = phase == 0 ? __shfl(s_reg, row & 63, 64) : 1.f;
#pragma unroll
    for (int q = 0; q < NB / 2; ++q) {
      const float g = am[2 * q][r], u = am[2 * q + 1][r];
      const int col = q * 32 + (lane & 31);
      const int o = row * 64 + st_col<64>(row, col);
      if (phase == 0) {
        l0[o] = (uint16_t)f32_to_bf16_bits(s * silu_f32(g) * u);
        l1[o] = (uint16_t)f32_to_bf16_bits(g);
      } else {
        l0[o] = (uint16_t)f32_to_bf16_bits(u);
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

// SwiGLU backward of one 32-row block against the staged g, u of its rows
// (region rows `mloc` relative): dg, du replace g, u in place; the partial
// ds of each row (over this wavefront's 128 columns) goes to ds_part.
// s_reg: lane l holds the routing scale of wavefront row (mrow & 64) + l.
template <int BN, int WN, int NB>
__device__ __forceinline__ void mx_swiglu_bwd_stage(
    const MxArgs &p, const f32x16 (&am)[NB], int mloc, int mrow, int lane,
    int arow0, int rows, int row0, int nt, int wn, float s_reg, uint16_t *lg,
    uint16_t *lu) {
  float part[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    const int row = mloc + rr;                 // region row
    const float s = __shfl(s_reg, (mrow + rr) & 63, 64);
    part[r] = 0.f;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int o = row * 128 + st_col<128>(row, n * 32 + (lane & 31));
      const float da = am[n][r];
      const float g = bf16_bits_to_f32(lg[o]);
      const float u = bf16_bits_to_f32(lu[o]);
      const float sg = sigmoid_f32(g);
      const float sl = g * sg;
      const float dsl = sg * (1.f + g * (1.f - sg));
      lg[o] = (uint16_t)f32_to_bf16_bits(da * s * u * dsl);
      lu[o] = (uint16_t)f32_to_bf16_bits(da * s * sl);
      part[r] += da * sl * u;
    }
  }
  const float tot = mx_sum16_over32(part, lane);
  const int r = (lane & 31) >> 1;
  const int rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
  if ((lane & 1) == 0 && arow0 + mrow + rr < rows)
    p.ds_part[(int64_t)(row0 + arow0 + mrow + rr) * (p.NT * WN) + nt * WN + wn] = tot;
}

template <int MODE, int EPI, int BM, int BN, int WM, int WN, int STAGES, int BKB>
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
  if (MODE == MX_ROWSEG) {
    e = upper_bound_minus1(p.tile_prefix, p.G, t);
    const int r_begin = p.offsets[e], r_end = p.offsets[e + 1];
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
              af0[m], bf0[n], acc[m][n], 0, 0, 0, (int)((sa[m] >> (8 * h)) & 0xffu),
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
              af1[m], bf1[n], acc[m][n], 0, 0, 0, (int)((sa[m] >> (8 * (2 + h))) & 0xffu),
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
    // region: two [128][64] arrays (a | g, then u)
    uint16_t *l0 = lw, *l1 = lw + 128 * 64;
    const int64_t col0 = (int64_t)nt * (BN / 2) + brow0 / 2;
    const int64_t grow0 = row0 + arow0;
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
#define MX_SW_BLOCK(m) \
      if constexpr (MB > (m)) mx_swiglu_stage<NB>(acc[m], (m) * 32, lane, (m) < 2 ? s_lo : s_hi, l0, l1, phase);
      MX_SW_BLOCK(0) MX_SW_BLOCK(1) MX_SW_BLOCK(2) MX_SW_BLOCK(3)
#undef MX_SW_BLOCK
      __syncthreads();
      if (phase == 0) {
        store_staged<64, 128>(l0, (uint16_t *)p.C, p.ldc, col0, p.N, grow0, arow0, rows, lane);
        if (p.q) mx_quant_staged<64, 128>(l0, p.q, p.ldq, p.qs, p.ldqs, col0, grow0, arow0, rows, lane);
        if (p.gu) store_staged<64, 128>(l1, p.gu, p.ldgu, col0, p.N, grow0, arow0, rows, lane);
      } else if (p.gu) {
        store_staged<64, 128>(l0, p.gu, p.ldgu, p.N + col0, 2 * p.N, grow0, arow0, rows, lane);
      }
      __syncthreads();
    }
  } else if constexpr (EPI == MX_EPI_SWIGLU_BWD) {
    static_assert(WTM == 128 && WTN == 128 && MB == 4, "staging expects 128x128 wavefront tiles");
    // region: g and u of 64 rows x 128 columns, two halves of the 128 rows
    uint16_t *lg = lw, *lu = lw + 64 * 128;
    const uint32_t lgb = lds0 + (uint32_t)(wid * WTM * WTN * 2);
    const uint32_t lub = lgb + 64 * 128 * 2;
    const int64_t col0 = (int64_t)nt * BN + brow0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t grow0 = row0 + arow0 + half * 64;
      const int ar0 = arow0 + half * 64;
      const uint16_t *gb = mx_uniform(p.gu + (int64_t)row0 * p.ldgu + col0);
      mx_load_gu_staged<64>(lgb, lub, gb, mx_uniform(gb + p.N), p.ldgu, ar0, rows, lane);
      mx_wait_barrier<0>();
      if (half == 0) {
        mx_swiglu_bwd_stage<BN, WN, NB>(p, acc[0], 0, 0, lane, arow0, rows, row0, nt, wn, s_lo, lg, lu);
        mx_swiglu_bwd_stage<BN, WN, NB>(p, acc[1], 32, 32, lane, arow0, rows, row0, nt, wn, s_lo, lg, lu);
      } else {
        mx_swiglu_bwd_stage<BN, WN, NB>(p, acc[2], 0, 64, lane, arow0, rows, row0, nt, wn, s_hi, lg, lu);
        mx_swiglu_bwd_stage<BN, WN, NB>(p, acc[3], 32, 96, lane, arow0, rows, row0, nt, wn, s_hi, lg, lu);
      }
      __syncthreads();
      if (p.dgu) {
        store_staged<128, 64>(lg, p.dgu, p.ldgu, col0, p.N, grow0, ar0, rows, lane);
        store_staged<128, 64>(lu, p.dgu + p.N, p.ldgu, col0, p.N, grow0, ar0, rows, lane);
      }
      if (p.t0) {
        // tile rows start at offsets[e] + mt * BM, padded position tpad[e] + mt * BM
        const int64_t pos0 = (int64_t)p.tpad[e] + (row0 - p.offsets[e]) + ar0;
        const int valid = min(max(rows - ar0, 0), 64);
        mx_quant_staged_cols<128, 64>(lg, p.t0, p.t0s, p.ldt, p.ldts, col0, pos0, valid, lane);
        mx_quant_staged_cols<128, 64>(lu, p.t1, p.t1s, p.ldt, p.ldts, col0, pos0, valid, lane);
      }
      if (p.q) {
        mx_quant_staged<128, 64>(lg, p.q, p.ldq, p.qs, p.ldqs, col0, grow0, ar0, rows, lane);
        mx_quant_staged<128, 64>(lu, p.q, p.ldq, p.qs, p.ldqs, p.N + col0, grow0, ar0, rows, lane);
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

template <int MODE, int EPI>
hipError_t mx_launch(const MxArgs &p, int64_t max_tiles, hipStream_t s) {
  mx_gemm_kernel<MODE, EPI, MOE_MX_CFG>
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
  p.ldt = d.ldt; p.ldts = d.ldts; p.tpad = d.tpad;
  p.ksplit = d.ksplit;
  const int cols = epi == MX_EPI_SWIGLU ? kMxBN / 2 : kMxBN;
  p.NT = (d.N + cols - 1) / cols;
  p.tile_prefix = d.tile_ws;
  mx_plan_kernel<<<1, 1024, 0, s>>>(d.offsets, d.G, kMxBM, p.NT, d.tile_ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // SwiGLU backward: 32-bit byte offsets within a tile's rows of g|u.
  if (epi == MX_EPI_SWIGLU_BWD && (int64_t)kMxBM * d.ldgu * 2 >= (1ll << 32))
    return hipErrorInvalidValue;
  const int64_t max_tiles = ((d.R_cap + kMxBM - 1) / kMxBM + d.G) * (int64_t)p.NT;
  if (epi == MX_EPI_SWIGLU) err = mx_launch<MX_ROWSEG, MX_EPI_SWIGLU>(p, max_tiles, s);
  else if (epi == MX_EPI_SWIGLU_BWD) err = mx_launch<MX_ROWSEG, MX_EPI_SWIGLU_BWD>(p, max_tiles, s);
  else err = mx_launch<MX_ROWSEG, MX_EPI_BF16>(p, max_tiles, s);
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
  return mx_launch<MX_KSEG, MX_EPI_BF16>(p, (int64_t)d.G * p.MT * p.NT, s);
}

}  // namespace moe
