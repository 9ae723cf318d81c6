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
// The E4M3 rounding is done with exact fp32 arithmetic (scaling by a power
// of two is exact; rintf rounds half to even), so the codes do not depend on
// any conversion instruction's rounding mode.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// floor(log2(a)) for a finite a > 0.
__device__ __forceinline__ int ilog2f(float a) {
  int e;
  frexpf(a, &e);  // a = m * 2^e, m in [0.5, 1)
  return e - 1;
}

__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  if (!(amax > 0.f)) return 0u;
  int X = ilog2f(amax) - 8;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  return (uint32_t)(X + 127);
}

// E4M3 code of v * 2^-(scale_byte - 127).
__device__ __forceinline__ uint32_t e4m3_code(float v, uint32_t scale_byte) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float f = ldexpf(fabsf(v), 127 - (int)scale_byte);
  uint32_t code;
  if (f >= 464.f) {
    code = 0x7E;                                   // saturate to 448
  } else if (f < 0.015625f) {                      // below 2^-6: subnormal
    code = (uint32_t)rintf(f * 512.f);             // m * 2^-9, m = 0..8
  } else {
    int e = ilog2f(f);
    const float m = ldexpf(f, -e) - 1.f;           // [0, 1), exact
    uint32_t q = (uint32_t)rintf(m * 8.f);         // 0..8
    if (q == 8) { q = 0; ++e; }
    code = ((uint32_t)(e + 7) << 3) | q;
    if (code > 0x7E) code = 0x7E;
  }
  return sign | code;
}

// axis 0: one thread per block of 32 values along a row.
//   in [rows, cols] bf16 (row pitch ld_in), codes [rows, ld_codes] (first
//   cols used), scales [rows, ld_scales].  rows_dev (may be null): a device
//   row count below `rows`; rows past it are left alone.
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
  const uint32_t sb = mx_scale_byte(amax);
  uint32_t packed[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    packed[j] = e4m3_code(v[4 * j], sb) | (e4m3_code(v[4 * j + 1], sb) << 8) |
                (e4m3_code(v[4 * j + 2], sb) << 16) |
                (e4m3_code(v[4 * j + 3], sb) << 24);
  uint4 *dst = (uint4 *)(codes + r * ld_codes + b * 32);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  scales[r * ld_scales + b] = (uint8_t)sb;
}

// axis 1: blocks of 32 rows down each column, inside segments of rows
// [seg[s], seg[s+1]) zero-padded to a multiple of `align` (32 or 512); output
// transposed: codesT[c, pad[s] + j] for row seg[s] + j, scalesT[c, blk].
// seg == null: one segment of all `rows`.
// One workgroup per tile of 128 padded rows x 64 columns: the tile is read
// with coalesced 16-byte loads (8 threads per 128-byte row piece) into LDS,
// then wavefront b quantises block b (32 rows) of all 64 columns, a lane per
// column, and writes that column's 32 codes; the four wavefronts together
// write each column's 128 codes as one 128-byte line.
// Requires ld_in % 8 == 0, cols % 32 == 0 and a 16-byte aligned input.
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(
    const uint16_t *__restrict__ in, int64_t rows, int64_t cols,
    int64_t ld_in, const int32_t *__restrict__ seg,
    const int32_t *__restrict__ pad, int nseg, int align,
    uint8_t *__restrict__ codes, int64_t ld_codes,
    uint8_t *__restrict__ scales, int64_t ld_scales) {
  constexpr int TR = 128, TC = 64, LDT = TC + 2;   // +2: row pitch 132 B
  __shared__ uint16_t tile[TR * LDT];
  __shared__ int32_t src[TR];
  const int tid = threadIdx.x;
  const int padded = seg ? pad[nseg] : (int)((rows + align - 1) / align * align);
  const int ngrp = (padded + TR - 1) / TR;
  const int ncg = (int)((cols + TC - 1) / TC);
  const int64_t ntiles = (int64_t)ngrp * ncg;
  for (int64_t g = blockIdx.x; g < ntiles; g += gridDim.x) {
    const int rg = (int)(g / ncg), cg = (int)(g % ncg);
    const int prow0 = rg * TR;
    const int64_t c0 = (int64_t)cg * TC;
    if (tid < TR) {
      const int prow = prow0 + tid;
      int sr = -1;
      if (prow < padded) {
        if (seg) {
          const int s = upper_bound_minus1(pad, nseg, prow);
          const int r = seg[s] + (prow - pad[s]);
          if (r < seg[s + 1]) sr = r;
        } else if (prow < rows) {
          sr = prow;
        }
      }
      src[tid] = sr;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < TR / 32; ++p) {
      const int r = p * 32 + (tid >> 3);
      const int cc = (tid & 7) * 8;
      const int sr = src[r];
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (sr >= 0 && c0 + cc < cols)
        v = *(const uint4 *)(in + (int64_t)sr * ld_in + c0 + cc);
      uint32_t *d = (uint32_t *)(tile + r * LDT + cc);
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    __syncthreads();
    const int b = tid >> 6, c = tid & 63;
    const int prow = prow0 + b * 32;
    if (prow < padded && c0 + c < cols) {
      float v[32];
      float amax = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        v[j] = bf16_bits_to_f32(tile[(b * 32 + j) * LDT + c]);
        amax = fmaxf(amax, fabsf(v[j]));
      }
      const uint32_t sb = mx_scale_byte(amax);
      uint32_t packed[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        packed[j] = e4m3_code(v[4 * j], sb) | (e4m3_code(v[4 * j + 1], sb) << 8) |
                    (e4m3_code(v[4 * j + 2], sb) << 16) |
                    (e4m3_code(v[4 * j + 3], sb) << 24);
      uint4 *dst = (uint4 *)(codes + (c0 + c) * ld_codes + prow);
      dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      scales[(c0 + c) * ld_scales + prow / 32] = (uint8_t)sb;
    }
    __syncthreads();
  }
}

// pad[s+1] = pad[s] + ceil(len_s / align) * align, pad[0] = 0.  One block.
__global__ __launch_bounds__(1024) void mx_pad_offsets_kernel(
    const int32_t *__restrict__ seg, int nseg, int align,
    int32_t *__restrict__ pad) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (nseg + 1023) / 1024;
  const int s0 = min(nseg, tid * per), s1 = min(nseg, s0 + per);
  int32_t sum = 0;
  for (int s = s0; s < s1; ++s) sum += (seg[s + 1] - seg[s] + align - 1) / align * align;
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
    run += (seg[s + 1] - seg[s] + align - 1) / align * align;
  }
  if (tid == 1023) pad[nseg] = part[1023];
}

hipError_t launch_mx_quant_rows(const uint16_t *in, int64_t rows, int64_t cols,
                                int64_t ld_in, uint8_t *codes,
                                int64_t ld_codes, uint8_t *scales,
                                int64_t ld_scales, const int32_t *rows_dev,
                                hipStream_t s) {
  const int64_t n = rows * (cols / 32);
  if (n == 0) return hipSuccess;
  mx_quant_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
      in, rows, cols, ld_in, codes, ld_codes, scales, ld_scales, rows_dev);
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(const uint16_t *in, int64_t rows,
                                int64_t cols, int64_t ld_in,
                                const int32_t *seg, int nseg, int align,
                                int32_t *pad, uint8_t *codes,
                                int64_t ld_codes, uint8_t *scales,
                                int64_t ld_scales, int num_cus,
                                hipStream_t s) {
  if (seg) {
    mx_pad_offsets_kernel<<<1, 1024, 0, s>>>(seg, nseg, align, pad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int64_t grid = (int64_t)num_cus * 8;
  mx_quant_cols_kernel<<<(unsigned)grid, 256, 0, s>>>(
      in, rows, cols, ld_in, seg, pad, nseg, align, codes, ld_codes, scales,
      ld_scales);
  return hipGetLastError();
}

}  // namespace moe
