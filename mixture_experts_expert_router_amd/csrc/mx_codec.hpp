// E8M0 / E4M3 encoding of one MX block on the device, shared by the
// quantisation kernels and the GEMM epilogues that quantise their output.
// The rule (OCP Microscaling v1.0, the reading of the BioNeMo MoE article's
// MXFP8 section): X = floor(log2(max |v|)) - 8, scale byte X + 127, codes
// RNE(v * 2^-X) in E4M3 saturating at +-448, sign kept on zero.
// The gradient option uses E5M2 elements instead (OCP FP8 E5M2: largest
// normal exponent 15, largest finite 57344): X = floor(log2(max |v|)) - 15,
// codes RNE(v * 2^-X) saturating at +-57344.  The *_t<F> forms take the
// element format F (kMxE4M3 or kMxE5M2); the plain forms are E4M3.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kMxE4M3 = 0;
constexpr int kMxE5M2 = 1;

// Shared exponent X of a block whose largest magnitude is amax (finite).
// Blocks with amax < 2^-118 (all-zero ones included) get the floor -127;
// a finite fp32 amax gives X <= 119, so the scale byte X + 127 <= 246.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax >= 0x1p-118f)) return -127;
  int e;
  frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
  return e - 9;
}

// E4M3 codes of a * 2^nX .. d * 2^nX (nX = -X), packed low byte first.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c,
                                               float d, int nX) {
  a = __builtin_amdgcn_fmed3f(ldexpf(a, nX), -448.f, 448.f);
  b = __builtin_amdgcn_fmed3f(ldexpf(b, nX), -448.f, 448.f);
  c = __builtin_amdgcn_fmed3f(ldexpf(c, nX), -448.f, 448.f);
  d = __builtin_amdgcn_fmed3f(ldexpf(d, nX), -448.f, 448.f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// Shared exponent X from the bf16 bit pattern of a block's largest
// magnitude (sign bit clear, finite).  With exponent field E >= 1 the value
// lies in [2^(E-127), 2^(E-126)), so X = E - 127 - 8; below 2^-118 (E < 9,
// zero and subnormals included) X takes the floor -127.  For a bf16 amax
// this equals mx_shared_exp of its fp32 value.
__device__ __forceinline__ int mx_shared_exp_bf16(uint32_t mag) {
  const int E = (int)(mag >> 7);
  return E >= 9 ? E - 135 : -127;
}

// Codes and scale byte of 32 bf16 values (bit patterns, two per word, low
// half first): codes[0..7] get the packed bytes, the return value the scale
// byte.  The largest magnitude is found on the bit patterns (for values of
// one sign, integer order is float order), and each value is widened to
// fp32 only where it is encoded, so no 32-value fp32 copy is held.
__device__ __forceinline__ uint32_t mx_encode32(const uint4 (&in)[4], uint32_t (&codes)[8]) {
  uint32_t mag = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t u[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mag = max(mag, max(u[j] & 0x7fffu, (u[j] >> 16) & 0x7fffu));
  }
  const int X = mx_shared_exp_bf16(mag);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t u[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
#pragma unroll
    for (int j = 0; j < 2; ++j)
      codes[2 * q + j] = e4m3_pack4(
          bf16_bits_to_f32(u[2 * j] & 0xffffu), bf16_bits_to_f32(u[2 * j] >> 16),
          bf16_bits_to_f32(u[2 * j + 1] & 0xffffu), bf16_bits_to_f32(u[2 * j + 1] >> 16), -X);
  }
  return (uint32_t)(X + 127);
}

// Shared exponent for elements of format F (E4M3: mx_shared_exp).  For
// E5M2, X = e - 16 with amax = m * 2^e, m in [0.5, 1); blocks with
// amax < 2^-111 (X below -127, all-zero ones included) get -127.
template <int F>
__device__ __forceinline__ int mx_shared_exp_t(float amax) {
  if (F == kMxE4M3) return mx_shared_exp(amax);
  if (!(amax >= 0x1p-111f)) return -127;
  int e;
  frexpf(amax, &e);
  return e - 16;
}

// Shared exponent from the bf16 bit pattern of a block's largest magnitude,
// for elements of format F.  The value lies in [2^(E-127), 2^(E-126)) for
// exponent field E >= 1, so X = E - 127 - emax, floored at -127.
template <int F>
__device__ __forceinline__ int mx_shared_exp_bf16_t(uint32_t mag) {
  if (F == kMxE4M3) return mx_shared_exp_bf16(mag);
  const int E = (int)(mag >> 7);
  return E >= 15 ? E - 142 : -127;
}

// Codes of a * 2^nX .. d * 2^nX in format F, packed low byte first.
template <int F>
__device__ __forceinline__ uint32_t pack4_t(float a, float b, float c, float d,
                                            int nX) {
  if (F == kMxE4M3) return e4m3_pack4(a, b, c, d, nX);
  a = __builtin_amdgcn_fmed3f(ldexpf(a, nX), -57344.f, 57344.f);
  b = __builtin_amdgcn_fmed3f(ldexpf(b, nX), -57344.f, 57344.f);
  c = __builtin_amdgcn_fmed3f(ldexpf(c, nX), -57344.f, 57344.f);
  d = __builtin_amdgcn_fmed3f(ldexpf(d, nX), -57344.f, 57344.f);
  int r = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, r, true);
  return (uint32_t)r;
}

// mx_encode32 (bf16 bit patterns in) for elements of format F.
template <int F>
__device__ __forceinline__ uint32_t mx_encode32_t(const uint4 (&in)[4],
                                                  uint32_t (&codes)[8]) {
  uint32_t mag = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t u[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mag = max(mag, max(u[j] & 0x7fffu, (u[j] >> 16) & 0x7fffu));
  }
  const int X = mx_shared_exp_bf16_t<F>(mag);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t u[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
#pragma unroll
    for (int j = 0; j < 2; ++j)
      codes[2 * q + j] = pack4_t<F>(
          bf16_bits_to_f32(u[2 * j] & 0xffffu), bf16_bits_to_f32(u[2 * j] >> 16),
          bf16_bits_to_f32(u[2 * j + 1] & 0xffffu), bf16_bits_to_f32(u[2 * j + 1] >> 16), -X);
  }
  return (uint32_t)(X + 127);
}

// Codes and scale byte of 32 fp32 values (finite) in format F: codes[j]
// packs values 4j .. 4j+3, low byte first; the return value is the scale
// byte.
template <int F>
__device__ __forceinline__ uint32_t mx_encode32_f32_t(const float (&v)[32],
                                                      uint32_t (&codes)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int X = mx_shared_exp_t<F>(amax);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    codes[j] = pack4_t<F>(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], -X);
  return (uint32_t)(X + 127);
}

__device__ __forceinline__ uint32_t mx_encode32_f32(const float (&v)[32],
                                                    uint32_t (&codes)[8]) {
  return mx_encode32_f32_t<kMxE4M3>(v, codes);
}

}  // namespace moe
