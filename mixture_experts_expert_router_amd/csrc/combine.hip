// Unpermute / combine: expert outputs return to token order and are summed
// (Wide-EP explainer, 前提:MoEとは - the chosen experts' results are added;
// 前提条件:GPU間の高速通信 - combine).  Each token's output row is owned by
// one workgroup, which reads its (at most k) expert rows in slot order and
// accumulates in fp32 registers: no atomics, bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"

// 16-byte vectors of a row each combine thread loads at once
#ifndef MOE_COMBINE_CV
#define MOE_COMBINE_CV 4
#endif

namespace moe {

// bf16 rows as 16-byte vectors of 8 values.  Lane j < k of every wavefront
// loads the token's slot j (row and weight) with one load each; a ballot
// then names the local slots, and the row loop visits only those, four rows
// at a time, summing in slot order.  Each thread owns CV vectors of the row
// (c, c + 256, ...), and the loads of all of them for the current rows are
// issued before any is used, so a row costs one memory round trip, not one
// per vector.  The slot list is the same in every wavefront, so the loops
// are uniform.
template <int CV>
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint4 *__restrict__ y, const int32_t *__restrict__ inv,
    const float *__restrict__ w, int64_t T, int k, int64_t vecs,
    uint4 *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    int32_t rj = -1;
    float wj = 1.f;
    if (lane < k) {
      rj = inv[t * k + lane];
      if (w) wj = w[t * k + lane];
    }
    const uint64_t local = __ballot(rj >= 0);
    if (local == 0) {  // no local slot: a zero row
      for (int64_t c = threadIdx.x; c < vecs; c += blockDim.x)
        out[t * vecs + c] = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    for (int64_t c0 = threadIdx.x; c0 < vecs; c0 += CV * blockDim.x) {
      // vectors c0 + i*256 (i < CV); past the row end they read vector c0
      // again and are not stored
      int64_t cv[CV];
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int64_t c = c0 + (int64_t)i * blockDim.x;
        cv[i] = c < vecs ? c : c0;
      }
      float acc[CV][8];
#pragma unroll
      for (int i = 0; i < CV; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
      uint64_t rest = local;
      while (rest) {
        // the next (up to) four local slots, in slot order; missing ones
        // repeat the first row and are left out of the sum
        int32_t r[4];
        float cw[4];
        const int n = min(4, __popcll(rest));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < n) {
            const int j = __builtin_ctzll(rest);
            rest &= rest - 1;
            r[q] = __builtin_amdgcn_readlane(rj, j);
            cw[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j));
          } else {
            r[q] = r[0];
            cw[q] = 0.f;
          }
        }
        uint4 v[4][CV];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < CV; ++i)
            v[q][i] = (q < n) ? y[(int64_t)r[q] * vecs + cv[i]] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < n) {
#pragma unroll
            for (int i = 0; i < CV; ++i) {
              const uint32_t u[4] = {v[q][i].x, v[q][i].y, v[q][i].z, v[q][i].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                acc[i][2 * e] = fmaf(cw[q], bf16_bits_to_f32(u[e] & 0xffffu), acc[i][2 * e]);
                acc[i][2 * e + 1] = fmaf(cw[q], bf16_bits_to_f32(u[e] >> 16), acc[i][2 * e + 1]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < CV; ++i) {
        const int64_t c = c0 + (int64_t)i * blockDim.x;
        if (c >= vecs) continue;
        uint4 o;
        o.x = pack_bf16x2(acc[i][0], acc[i][1]);
        o.y = pack_bf16x2(acc[i][2], acc[i][3]);
        o.z = pack_bf16x2(acc[i][4], acc[i][5]);
        o.w = pack_bf16x2(acc[i][6], acc[i][7]);
        // Non-temporal: the output is not read again by this kernel, and
        // keeping it out of the caches leaves them to the gathered rows
        // (4% faster at 8192 tokens x 8 slots x 7168).
        uint32_t *const dst = (uint32_t *)&out[t * vecs + c];
        __builtin_nontemporal_store(o.x, dst);
        __builtin_nontemporal_store(o.y, dst + 1);
        __builtin_nontemporal_store(o.z, dst + 2);
        __builtin_nontemporal_store(o.w, dst + 3);
      }
    }
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(
    const float4 *__restrict__ y, const int32_t *__restrict__ inv,
    const float *__restrict__ w, int64_t T, int k, int64_t vecs,
    float4 *__restrict__ out) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    for (int64_t c = threadIdx.x; c < vecs; c += blockDim.x) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j = 0; j < k; ++j) {
        const int r = inv[t * k + j];
        if (r < 0) continue;
        const float cj = w ? w[t * k + j] : 1.f;
        const float4 v = y[(int64_t)r * vecs + c];
        acc.x = fmaf(cj, v.x, acc.x);
        acc.y = fmaf(cj, v.y, acc.y);
        acc.z = fmaf(cj, v.z, acc.z);
        acc.w = fmaf(cj, v.w, acc.w);
      }
      out[t * vecs + c] = acc;
    }
  }
}

hipError_t launch_combine(const void *y, const int32_t *inv,
                          const float *topk_w, int64_t T, int k, int64_t H,
                          int dtype, void *out, int num_cus, hipStream_t s) {
  int64_t grid = T < (int64_t)num_cus * 16 ? T : (int64_t)num_cus * 16;
  if (grid < 1) return hipSuccess;
  if (dtype == 1)
    combine_bf16_kernel<MOE_COMBINE_CV><<<(unsigned)grid, 256, 0, s>>>(
        (const uint4 *)y, inv, topk_w, T, k, H / 8, (uint4 *)out);
  else
    combine_f32_kernel<<<(unsigned)grid, 256, 0, s>>>(
        (const float4 *)y, inv, topk_w, T, k, H / 4, (float4 *)out);
  return hipGetLastError();
}

}  // namespace moe
