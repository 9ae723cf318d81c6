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
//           K runs over an expert's rows, zero-padded to 512).
// KSPLIT (data gradient through gate and up): B rows are [B0 row | B1 row]
// along K, the switch at K/2.
//
// Pipeline as in the bf16 grouped GEMM: 128 x 128 tiles (4 wavefronts of
// 64 x 64), K advances 128 values per stage, 4-stage LDS ring filled by
// direct global->LDS loads from inline assembly (explicit vmcnt waits).  A
// stage holds A and B code rows (128 B each, chunks swizzled against bank
// conflicts) plus, per row, the 16-byte scale chunk covering the 512 K
// values around the stage (so K must be a multiple of 512).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

struct MxArgs {
  const uint8_t *A, *As;
  int64_t lda, ldas;
  const uint8_t *B0, *B0s, *B1, *B1s;
  int64_t ldb, ldbs, b_stride, bs_stride;
  const int32_t *offsets;       // ROWSEG: [G + 1]
  const int32_t *tile_prefix;   // ROWSEG: [G + 1]
  const int32_t *kseg;          // KSEG: [G + 1] K ranges (multiples of 512)
  int G, M, N, K, NT, MT;
  void *C;
  int64_t ldc, c_stride;
  const float *row_scale;       // SWIGLU, SWIGLU_BWD: s per row (or null)
  uint16_t *gu;                 // SWIGLU: g,u out; SWIGLU_BWD: g,u in
  int64_t ldgu;                 // u at column offset N of gu
  uint16_t *dgu;                // SWIGLU_BWD: dg, du out [rows, ldgu]
  float *ds_part;               // SWIGLU_BWD: [rows, NT * 2]
  int ksplit;                   // KSPLIT: K of the B0 part (0 = none)
};

enum MxMode { MX_ROWSEG = 0, MX_KSEG = 1 };
enum MxEpi { MX_EPI_BF16 = 0, MX_EPI_SWIGLU = 1, MX_EPI_SWIGLU_BWD = 2 };

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

__device__ __forceinline__ void mx_load_lds16(uint32_t lds_base, const void *g) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory");
}

template <int N>
__device__ __forceinline__ void mx_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
               :: "i"(N) : "memory");
}

// 128-byte rows, 16 consecutive rows at one logical chunk hit 16 bank groups.
__device__ __forceinline__ int mx_swz(int row, int c) {
  return c ^ ((row >> 1) & 7);
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

template <int MODE, int EPI>
__global__ __launch_bounds__(256) void mx_gemm_kernel(MxArgs p) {
  constexpr int BM = 128, BN = 128, WM = 2, WN = 2, STAGES = 4;
  constexpr int WTM = BM / WM, WTN = BN / WN, MB = WTM / 32, NB = WTN / 32;
  constexpr int CODE_CHUNKS = (BM + BN) * 8;
  constexpr int STAGE_CHUNKS = CODE_CHUNKS + BM + BN;   // + scale chunks
  constexpr int L = STAGE_CHUNKS / 256;                 // loads per thread
  static_assert(STAGE_CHUNKS % 256 == 0, "load split");
  static_assert((STAGES - 2) * L <= 63, "vmcnt range");
  __shared__ uint4 smem[STAGES * STAGE_CHUNKS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  const uint32_t wave_off = (uint32_t)(wid * L * 64 * 16);

  int total;
  if (MODE == MX_ROWSEG) total = p.tile_prefix[p.G];
  else total = p.G * p.MT * p.NT;
  const int t = xcd_tile(blockIdx.x, total);
  if (t < 0) return;
  {
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
      KT = p.K / 128;
    } else {
      const int per_g = p.MT * p.NT;
      e = t / per_g;
      banded_mn(t - e * per_g, p.MT, p.NT, 8, mt, nt);
      row0 = mt * BM;
      rows = min(BM, p.M - row0);
      k0 = p.kseg[e];
      KT = (p.kseg[e + 1] - k0) / 128;
    }

    // sources of this thread's loads: chunk q = (wid*L + i)*64 + lane
    const char *gsrc[L];
    const char *gsrc1[L];   // KSPLIT: B rows taken from B1 past the split
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = (wid * L + i) * 64 + lane;
      gsrc1[i] = nullptr;
      if (q < CODE_CHUNKS) {
        const int row = q / 8;
        const int kc = mx_swz(row, q % 8);
        if (row < BM) {
          gsrc[i] = (const char *)p.A + (int64_t)(row0 + min(row, rows - 1)) * p.lda + k0 + kc * 16;
        } else {
          const int j = row - BM;
          int col;
          const uint8_t *base;
          if (EPI == MX_EPI_SWIGLU) {
            const int w = j & 31;
            col = nt * (BN / 2) + (j >> 5) * 16 + (w & 15);
            base = w < 16 ? p.B0 : p.B1;
          } else {
            col = nt * BN + j;
            base = p.B0;
          }
          col = min(col, p.N - 1);
          const int64_t ro = (int64_t)e * p.b_stride + (int64_t)col * p.ldb + k0 + kc * 16;
          gsrc[i] = (const char *)base + ro;
          if (p.ksplit) gsrc1[i] = (const char *)p.B1 + ro - p.ksplit;
        }
      } else {
        const int row = q - CODE_CHUNKS;  // scale chunk of A row or B row
        if (row < BM) {
          gsrc[i] = (const char *)p.As + (int64_t)(row0 + min(row, rows - 1)) * p.ldas + k0 / 32;
        } else {
          const int j = row - BM;
          int col;
          const uint8_t *base;
          if (EPI == MX_EPI_SWIGLU) {
            const int w = j & 31;
            col = nt * (BN / 2) + (j >> 5) * 16 + (w & 15);
            base = w < 16 ? p.B0s : p.B1s;
          } else {
            col = nt * BN + j;
            base = p.B0s;
          }
          col = min(col, p.N - 1);
          const int64_t ro = (int64_t)e * p.bs_stride + (int64_t)col * p.ldbs + k0 / 32;
          gsrc[i] = (const char *)base + ro;
          if (p.ksplit) gsrc1[i] = (const char *)p.B1s + ro - p.ksplit / 32;
        }
      }
    }

    f32x16 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

    // Stage kt's load i: codes advance 128 bytes per stage, scale chunks
    // (16 blocks = 512 K values) every 4 stages.
#define MX_ISSUE(stage_, kt_)                                                   \
  {                                                                             \
    const uint32_t sb = lds0 + (uint32_t)((stage_) * STAGE_CHUNKS * 16) + wave_off; \
    const int kk_ = (kt_);                                                      \
    const bool hi = p.ksplit && kk_ * 128 >= p.ksplit;                          \
    _Pragma("unroll") for (int i = 0; i < L; ++i) {                             \
      const int q = (wid * L + i) * 64 + lane;                                  \
      const int64_t off = q < CODE_CHUNKS ? (int64_t)kk_ * 128 : (int64_t)(kk_ >> 2) * 16; \
      const char *src = (hi && gsrc1[i]) ? gsrc1[i] : gsrc[i];                  \
      mx_load_lds16(sb + (uint32_t)(i * 64 * 16), src + off);                   \
    }                                                                           \
  }

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
      if (st < KT) MX_ISSUE(st, st);

    const int arow0 = wm * WTM, brow0 = wn * WTN;
    for (int kt = 0; kt < KT; ++kt) {
      const int after = min(STAGES - 2, KT - 1 - kt);
      if (after >= 2) mx_wait_barrier<2 * L>();
      else if (after == 1) mx_wait_barrier<L>();
      else mx_wait_barrier<0>();
      if (kt + STAGES - 1 < KT) MX_ISSUE((kt + STAGES - 1) % STAGES, kt + STAGES - 1);

      const uint4 *S = smem + (kt % STAGES) * STAGE_CHUNKS;
      const uint4 *As = S, *Bs = S + BM * 8;
      const uint8_t *Ssc = (const uint8_t *)(S + CODE_CHUNKS);  // scale chunks
      const int h = lane >> 5;
      // scale dwords (4 blocks of this stage) for this lane's rows
      uint32_t sa[MB], sbv[NB];
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int row = arow0 + m * 32 + (lane & 31);
        sa[m] = *(const uint32_t *)(Ssc + row * 16 + (kt & 3) * 4);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int row = BM + brow0 + n * 32 + (lane & 31);
        sbv[n] = *(const uint32_t *)(Ssc + row * 16 + (kt & 3) * 4);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // Operand layout of the 32x32x64 f8 instruction: lane half h holds
        // K [16h, 16h+16) in its first four registers and [32+16h, 48+16h)
        // in the last four; block b (K [32b, 32b+32)) takes its scale from
        // lane half b.  In 16-byte chunks of the 64-value step: h and 2 + h.
        const int c0 = 4 * kk + h, c1 = 4 * kk + 2 + h;
        i32x8_t af[MB], bfr[NB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const int row = arow0 + m * 32 + (lane & 31);
          const uint4 v0 = As[row * 8 + mx_swz(row, c0)];
          const uint4 v1 = As[row * 8 + mx_swz(row, c1)];
          af[m] = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                          (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int row = brow0 + n * 32 + (lane & 31);
          const uint4 v0 = Bs[row * 8 + mx_swz(row, c0)];
          const uint4 v1 = Bs[row * 8 + mx_swz(row, c1)];
          bfr[n] = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                           (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        }
        const int sh = 8 * (2 * kk + h);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int n = 0; n < NB; ++n)
            acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[m], bfr[n], acc[m][n], 0, 0, 0, (int)((sa[m] >> sh) & 0xffu),
                0, (int)((sbv[n] >> sh) & 0xffu));
      }
    }
#undef MX_ISSUE
    mx_wait_barrier<0>();

    // Epilogue: lane holds column (lane & 31) of each 32x32 block and rows
    // 8*(r/4) + 4*(lane/32) + (r%4).
    if (EPI == MX_EPI_SWIGLU_BWD) {
      // per row: partial ds over this wavefront's columns
#pragma unroll
      for (int m = 0; m < MB; ++m) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = arow0 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const bool row_ok = i < rows;
          const int64_t grow = row0 + (row_ok ? i : 0);
          const float s = p.row_scale ? p.row_scale[grow] : 1.f;
          float part = 0.f;
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const int col = nt * BN + brow0 + n * 32 + (lane & 31);
            const bool ok = row_ok && col < p.N;
            const float da = acc[m][n][r];
            float g = 0.f, u = 0.f;
            if (ok) {
              g = bf16_bits_to_f32(p.gu[grow * p.ldgu + col]);
              u = bf16_bits_to_f32(p.gu[grow * p.ldgu + p.N + col]);
            }
            const float sg = 1.f / (1.f + __expf(-g));
            const float sl = g * sg;
            const float dsl = sg * (1.f + g * (1.f - sg));
            if (ok) {
              p.dgu[grow * p.ldgu + col] = (uint16_t)f32_to_bf16_bits(da * s * u * dsl);
              p.dgu[grow * p.ldgu + p.N + col] = (uint16_t)f32_to_bf16_bits(da * s * sl);
              part += da * sl * u;
            }
          }
          // sum over the 32 columns held by this half-wavefront
#pragma unroll
          for (int off = 16; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
          if ((lane & 31) == 0 && row_ok)
            p.ds_part[grow * (p.NT * WN) + nt * WN + wn] = part;
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
#pragma unroll
        for (int n = 0; n < NB; ++n) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = arow0 + m * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const float v = acc[m][n][r];
            if (EPI == MX_EPI_SWIGLU) {
              const float other = __shfl_xor(v, 16, 64);
              if ((lane & 31) < 16 && i < rows) {
                const int col = nt * (BN / 2) + (brow0 + n * 32) / 2 + (lane & 15);
                if (col < p.N) {
                  const int64_t grow = row0 + i;
                  const float s = p.row_scale ? p.row_scale[grow] : 1.f;
                  ((uint16_t *)p.C)[grow * p.ldc + col] =
                      (uint16_t)f32_to_bf16_bits(s * silu_f32(v) * other);
                  if (p.gu) {
                    p.gu[grow * p.ldgu + col] = (uint16_t)f32_to_bf16_bits(v);
                    p.gu[grow * p.ldgu + p.N + col] = (uint16_t)f32_to_bf16_bits(other);
                  }
                }
              }
            } else {
              const int col = nt * BN + brow0 + n * 32 + (lane & 31);
              if (i < rows && col < p.N) {
                const int64_t base = (MODE == MX_KSEG) ? (int64_t)e * p.c_stride : 0;
                ((uint16_t *)p.C)[base + (int64_t)(row0 + i) * p.ldc + col] =
                    (uint16_t)f32_to_bf16_bits(v);
              }
            }
          }
        }
      }
    }
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

template <int MODE, int EPI>
hipError_t mx_launch(const MxArgs &p, int num_cus, int64_t max_tiles,
                     hipStream_t s) {
  (void)num_cus;
  mx_gemm_kernel<MODE, EPI><<<(unsigned)tile_grid(max_tiles), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_rowseg(const MxGemmDesc &d, int epi, int num_cus,
                            hipStream_t s) {
  MxArgs p{};
  p.A = d.A; p.As = d.As; p.lda = d.lda; p.ldas = d.ldas;
  p.B0 = d.B0; p.B0s = d.B0s; p.B1 = d.B1; p.B1s = d.B1s;
  p.ldb = d.ldb; p.ldbs = d.ldbs; p.b_stride = d.b_stride; p.bs_stride = d.bs_stride;
  p.offsets = d.offsets; p.G = d.G; p.N = d.N; p.K = d.K;
  p.C = d.C; p.ldc = d.ldc; p.row_scale = d.row_scale;
  p.gu = d.gu; p.ldgu = d.ldgu; p.dgu = d.dgu; p.ds_part = d.ds_part;
  p.ksplit = d.ksplit;
  const int cols = epi == MX_EPI_SWIGLU ? 64 : 128;
  p.NT = (d.N + cols - 1) / cols;
  p.tile_prefix = d.tile_ws;
  mx_plan_kernel<<<1, 1024, 0, s>>>(d.offsets, d.G, 128, p.NT, d.tile_ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t max_tiles = ((d.R_cap + 127) / 128 + d.G) * (int64_t)p.NT;
  if (epi == MX_EPI_SWIGLU) err = mx_launch<MX_ROWSEG, MX_EPI_SWIGLU>(p, num_cus, max_tiles, s);
  else if (epi == MX_EPI_SWIGLU_BWD) err = mx_launch<MX_ROWSEG, MX_EPI_SWIGLU_BWD>(p, num_cus, max_tiles, s);
  else err = mx_launch<MX_ROWSEG, MX_EPI_BF16>(p, num_cus, max_tiles, s);
  if (err != hipSuccess || epi != MX_EPI_SWIGLU_BWD) return err;
  mx_ds_reduce_kernel<<<(unsigned)num_cus, 256, 0, s>>>(
      d.ds_part, p.NT * 2, d.offsets + d.G, d.ds);
  return hipGetLastError();
}

hipError_t launch_mx_kseg(const MxGemmDesc &d, int num_cus, hipStream_t s) {
  MxArgs p{};
  p.A = d.A; p.As = d.As; p.lda = d.lda; p.ldas = d.ldas;
  p.B0 = d.B0; p.B0s = d.B0s; p.ldb = d.ldb; p.ldbs = d.ldbs;
  p.b_stride = 0; p.bs_stride = 0;
  p.kseg = d.kseg; p.G = d.G; p.M = d.M; p.N = d.N;
  p.MT = (d.M + 127) / 128;
  p.NT = (d.N + 127) / 128;
  p.C = d.C; p.ldc = d.ldc; p.c_stride = d.c_stride;
  return mx_launch<MX_KSEG, MX_EPI_BF16>(p, num_cus,
                                         (int64_t)d.G * p.MT * p.NT, s);
}

}  // namespace moe
