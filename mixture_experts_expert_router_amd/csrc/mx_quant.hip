// MXFP8 quantisation: FP8 E4M3 element codes with one E8M0 scale per block
// of 32 values.  BioNeMo MoE article, "MXFP8 Precision Reduces Memory
// Footprint for Biological Models": 8-bit values, a scaling factor for each
// block of 32 consecutive values.  The pages fix no rounding rule; the one
// used is the OCP Microscaling (MX) v1.0 conversion: shared exponent
// X = floor(log2(max |v|)) - 8 (8 = largest E4M3 exponent), scale byte
// X + 127 (clamped to [0, 254]), elements v * 2^-X rounded to the nearest
// E4M3 value (ties to even), saturating at +-448; an all-zero block gets
// scale byte 0.  The sign of a value that rounds to zero is kept (0x80).
//
// Element conversion: v * 2^-X by v_ldexp_f32 (exact for every result that
// can round to a non-zero code), a clamp to +-448 (the saturation), then
// gfx950's v_cvt_pk_fp8_f32, which rounds to nearest, ties to even, in the
// default rounding mode.  Four values cost about five VALU instructions.
// The GPU tests run every finite bf16 value under every shared exponent
// through both kernels and compare the codes with the oracle bit for bit.
//
// F = kMxE5M2 (the gradient option) quantises to E5M2 elements instead:
// X = floor(log2(max |v|)) - 15, a clamp to +-57344 and gfx950's
// v_cvt_pk_bf8_f32 (nearest, ties to even); tested the same way.
#include "common.hpp"
#include "kernels.hpp"
#include "mx_codec.hpp"

namespace moe {

// axis 0: one thread per block of 32 values along a row.
//   in [rows, cols] bf16 (row pitch ld_in), codes [rows, ld_codes] (first
//   cols used), scales [rows, ld_scales].  rows_dev (may be null): a device
//   row count below `rows`; rows past it are left alone.
template <int F>
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(
    const uint16_t *__restrict__ in, int64_t rows, int64_t cols,
    int64_t ld_in, uint8_t *__restrict__ codes, int64_t ld_codes,
    uint8_t *__restrict__ scales, int64_t ld_scales,
    const int32_t *__restrict__ rows_dev) {
  const int64_t nb = cols / 32;
  if (rows_dev) rows = min(rows, (int64_t)*rows_dev);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * nb) return;
  const int64_t r = t / nb, b = t % nb;
  const uint4 *src = (const uint4 *)(in + r * ld_in + b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = src[q];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[q * 8 + 2 * j] = bf16_bits_to_f32(u[j] & 0xffffu);
      v[q * 8 + 2 * j + 1] = bf16_bits_to_f32(u[j] >> 16);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int X = mx_shared_exp_t<F>(amax);
  uint32_t packed[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    packed[j] = pack4_t<F>(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], -X);
  uint4 *dst = (uint4 *)(codes + r * ld_codes + b * 32);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  scales[r * ld_scales + b] = (uint8_t)(X + 127);
}

// axis 1: blocks of 32 rows down each column, inside segments of rows
// [seg[s], seg[s+1]) zero-padded to a multiple of `align` (32 or 512); output
// transposed: codesT[c, pad[s] + j] for row seg[s] + j, scalesT[c, blk].
// seg == null: one segment of all `rows`.
// A workgroup walks tiles of 128 padded rows x 64 columns, one tile ahead:
// the next tile's 16-byte loads are in flight while the current one is
// quantised.  The tile goes through LDS (8 lanes per 128-byte row piece);
// wavefront b quantises block b (32 rows) of the 64 columns, a lane per
// column, and stages the codes transposed in LDS, so that the write-back
// stores whole 128-byte lines of codesT (8 lanes per line) and each
// column's four scale bytes as one dword.
// Requires ld_in % 8 == 0, ld_codes % 16 == 0, cols % 32 == 0 and 16-byte
// aligned input and codes.
template <int F>
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(
    const uint16_t *__restrict__ in, int64_t rows, int64_t cols,
    int64_t ld_in, const int32_t *__restrict__ seg,
    const int32_t *__restrict__ pad, int nseg, int align,
    uint8_t *__restrict__ codes, int64_t ld_codes,
    uint8_t *__restrict__ scales, int64_t ld_scales) {
  constexpr int TR = 128, TC = 64, LDT = TC + 2;   // +2: row pitch 132 B
  constexpr int LDO = TR + 16;                     // staged code row pitch
  __shared__ uint16_t tile[TR * LDT];
  __shared__ __align__(16) uint8_t ostage[TC * LDO];
  __shared__ uint32_t sstage[TC];
  __shared__ int32_t src[2][TR];
  const int tid = threadIdx.x;
  const int padded = seg ? pad[nseg] : (int)((rows + align - 1) / align * align);
  const int ngrp = (padded + TR - 1) / TR;
  const int ncg = (int)((cols + TC - 1) / TC);
  const int64_t ntiles = (int64_t)ngrp * ncg;
  const bool dword_scales =
      ld_scales % 4 == 0 && ((uintptr_t)scales & 3) == 0;

  // Source row of each padded row of tile g (-1: padding).
  auto lookup = [&](int64_t g, int buf) {
    if (tid < TR) {
      const int prow = (int)(g / ncg) * TR + tid;
      int sr = -1;
      if (prow < padded) {
        if (seg) {
          const int s = upper_bound_minus1(pad, nseg, prow);
          int b, e;
          seg_rows(seg, s, (int)rows, b, e);
          const int r = b + (prow - pad[s]);
          if (r < e) sr = r;
        } else if (prow < rows) {
          sr = prow;
        }
      }
      src[buf][tid] = sr;
    }
  };
  auto load = [&](int64_t g, int buf, uint4 (&v)[TR / 32]) {
    const int64_t c0 = (g % ncg) * TC;
    const int cc = (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < TR / 32; ++p) {
      const int sr = src[buf][p * 32 + (tid >> 3)];
      v[p] = make_uint4(0u, 0u, 0u, 0u);
      if (sr >= 0 && c0 + cc < cols)
        v[p] = *(const uint4 *)(in + (int64_t)sr * ld_in + c0 + cc);
    }
  };

  int64_t g = blockIdx.x;
  if (g >= ntiles) return;
  int buf = 0;
  lookup(g, 0);
  __syncthreads();
  uint4 v[TR / 32];
  load(g, 0, v);
  for (; g < ntiles; g += gridDim.x, buf ^= 1) {
    const int prow0 = (int)(g / ncg) * TR;
    const int64_t c0 = (g % ncg) * TC;
#pragma unroll
    for (int p = 0; p < TR / 32; ++p) {
      uint32_t *d = (uint32_t *)(tile + (p * 32 + (tid >> 3)) * LDT + (tid & 7) * 8);
      d[0] = v[p].x; d[1] = v[p].y; d[2] = v[p].z; d[3] = v[p].w;
    }
    const int64_t gn = g + gridDim.x;
    if (gn < ntiles) lookup(gn, buf ^ 1);
    __syncthreads();
    if (gn < ntiles) load(gn, buf ^ 1, v);

    const int b = tid >> 6, c = tid & 63;
    {
      float x[32];
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        x[j] = bf16_bits_to_f32(tile[(b * 32 + j) * LDT + c]);
        amax = fmaxf(amax, fabsf(x[j]));
      }
      const int X = mx_shared_exp_t<F>(amax);
      uint32_t pk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pk[j] = pack4_t<F>(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3], -X);
      uint4 *o = (uint4 *)(ostage + c * LDO + b * 32);
      o[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      o[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      ((uint8_t *)sstage)[c * 4 + b] = (uint8_t)(X + 127);
    }
    __syncthreads();

    // Write-back: piece q = (column q/8, 16 bytes q%8) of the staged codes.
#pragma unroll
    for (int i = 0; i < (TC * TR / 16) / 256; ++i) {
      const int q = tid + 256 * i;
      const int cq = q >> 3, j = q & 7;
      if (c0 + cq < cols && prow0 + j * 16 < padded)
        *(uint4 *)(codes + (c0 + cq) * ld_codes + prow0 + j * 16) =
            *(const uint4 *)(ostage + cq * LDO + j * 16);
    }
    if (tid < TC && c0 + tid < cols) {
      const uint32_t w = sstage[tid];
      uint8_t *sd = scales + (c0 + tid) * ld_scales + prow0 / 32;
      if (dword_scales && prow0 + TR <= padded) {
        *(uint32_t *)sd = w;
      } else {
        for (int k = 0; k < TR / 32; ++k)
          if (prow0 + 32 * k < padded) sd[k] = (uint8_t)(w >> (8 * k));
      }
    }
  }
}

// pad[s+1] = pad[s] + ceil(len_s / align) * align, pad[0] = 0, len_s the
// length of segment s cut at `rows`.  One block.
__global__ __launch_bounds__(1024) void mx_pad_offsets_kernel(
    const int32_t *__restrict__ seg, int nseg, int rows, int align,
    int32_t *__restrict__ pad) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (nseg + 1023) / 1024;
  const int s0 = min(nseg, tid * per), s1 = min(nseg, s0 + per);
  auto padded = [&](int s) {
    int b, e;
    seg_rows(seg, s, rows, b, e);
    return (e - b + align - 1) / align * align;
  };
  int32_t sum = 0;
  for (int s = s0; s < s1; ++s) sum += padded(s);
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - sum;
  for (int s = s0; s < s1; ++s) {
    pad[s] = run;
    run += padded(s);
  }
  if (tid == 1023) pad[nseg] = part[1023];
}

hipError_t launch_mx_quant_rows(const uint16_t *in, int64_t rows, int64_t cols,
                                int64_t ld_in, uint8_t *codes,
                                int64_t ld_codes, uint8_t *scales,
                                int64_t ld_scales, const int32_t *rows_dev,
                                hipStream_t s, int fmt) {
  const int64_t n = rows * (cols / 32);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (fmt == kMxE5M2)
    mx_quant_rows_kernel<kMxE5M2><<<grid, 256, 0, s>>>(
        in, rows, cols, ld_in, codes, ld_codes, scales, ld_scales, rows_dev);
  else
    mx_quant_rows_kernel<kMxE4M3><<<grid, 256, 0, s>>>(
        in, rows, cols, ld_in, codes, ld_codes, scales, ld_scales, rows_dev);
  return hipGetLastError();
}

hipError_t launch_mx_pad_offsets(const int32_t *seg, int nseg, int64_t rows,
                                 int align, int32_t *pad, hipStream_t s) {
  mx_pad_offsets_kernel<<<1, 1024, 0, s>>>(seg, nseg, (int)rows, align, pad);
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(const uint16_t *in, int64_t rows,
                                int64_t cols, int64_t ld_in,
                                const int32_t *seg, int nseg, int align,
                                int32_t *pad, uint8_t *codes,
                                int64_t ld_codes, uint8_t *scales,
                                int64_t ld_scales, int num_cus,
                                hipStream_t s, int fmt) {
  if (seg) {
    mx_pad_offsets_kernel<<<1, 1024, 0, s>>>(seg, nseg, (int)rows, align, pad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // As many workgroups as fit on the chip at once (LDS bounds them; both
  // element formats use the same resources).
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, mx_quant_cols_kernel<kMxE4M3>, 256, 0) != hipSuccess ||
        n < 1)
      n = 4;
    per_cu = n;
  }
  const unsigned grid = (unsigned)((int64_t)num_cus * per_cu);
  if (fmt == kMxE5M2)
    mx_quant_cols_kernel<kMxE5M2><<<grid, 256, 0, s>>>(
        in, rows, cols, ld_in, seg, pad, nseg, align, codes, ld_codes, scales,
        ld_scales);
  else
    mx_quant_cols_kernel<kMxE4M3><<<grid, 256, 0, s>>>(
        in, rows, cols, ld_in, seg, pad, nseg, align, codes, ld_codes, scales,
        ld_scales);
  return hipGetLastError();
}

}  // namespace moe
