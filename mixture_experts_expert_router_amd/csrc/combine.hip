// Unpermute / combine: expert outputs return to token order and are summed
// (Wide-EP explainer, 前提:MoEとは - the chosen experts' results are added;
// 前提条件:GPU間の高速通信 - combine).  Each token's output row is owned by
// one workgroup, which reads its (at most k) expert rows in slot order and
// accumulates in fp32 registers: no atomics, bitwise reproducible.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// bf16 rows as 16-byte vectors of 8 values.
__global__ __launch_bounds__(256) void combine_bf16_kernel(
    const uint4 *__restrict__ y, const int32_t *__restrict__ inv,
    const float *__restrict__ w, int64_t T, int k, int64_t vecs,
    uint4 *__restrict__ out) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    for (int64_t c = threadIdx.x; c < vecs; c += blockDim.x) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < k; ++j) {
        const int r = inv[t * k + j];
        if (r < 0) continue;
        const float cj = w ? w[t * k + j] : 1.f;
        const uint4 v = y[(int64_t)r * vecs + c];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(cj, bf16_bits_to_f32(u[q] & 0xffffu), acc[2 * q]);
          acc[2 * q + 1] = fmaf(cj, bf16_bits_to_f32(u[q] >> 16), acc[2 * q + 1]);
        }
      }
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      out[t * vecs + c] = o;
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
    combine_bf16_kernel<<<(unsigned)grid, 256, 0, s>>>(
        (const uint4 *)y, inv, topk_w, T, k, H / 8, (uint4 *)out);
  else
    combine_f32_kernel<<<(unsigned)grid, 256, 0, s>>>(
        (const float4 *)y, inv, topk_w, T, k, H / 4, (float4 *)out);
  return hipGetLastError();
}

}  // namespace moe
