// Device helpers shared by the gfx950 kernels of the MoE expert-layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// SiLU(z) = z * sigmoid(z)
__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + __expf(-z));
}

// Index of the last entry of the non-decreasing array p[0..n] that is <= v,
// for p[0] <= v < p[n].
__device__ __forceinline__ int upper_bound_minus1(const int32_t *p, int n,
                                                  int v) {
  int lo = 0, hi = n;  // invariant: p[lo] <= v < p[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (p[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace moe
