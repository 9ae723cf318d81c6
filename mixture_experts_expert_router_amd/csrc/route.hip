// Router: fp32 router GEMM (the bf16 router GEMM runs on the MFMA grouped
// GEMM with a single group) and the per-token softmax / top-k / renormalise.
// Wide-EP explainer, section 前提:MoE(Mixture of Experts)とは: per token the
// router chooses a few of the layer's experts.
#include <float.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// logits[t, e] = sum_h x[t,h] * w[e,h] (+ bias[e]); fp32.  One thread per
// output; used for the fp32 path, whose shapes are small.
__global__ void router_gemm_f32_kernel(const float *__restrict__ x,
                                       const float *__restrict__ w,
                                       const float *__restrict__ bias,
                                       float *__restrict__ logits, int64_t T,
                                       int64_t H, int64_t E) {
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= T * E) return;
  const int64_t t = o / E, e = o % E;
  const float *xr = x + t * H, *wr = w + e * H;
  float acc = 0.f;
  for (int64_t h = 0; h < H; ++h) acc = fmaf(xr[h], wr[h], acc);
  logits[o] = acc + (bias ? bias[e] : 0.f);
}

// Order-preserving integer key of a logit: larger logit -> larger key, so the
// arg-max runs on integers.  -0 and +0 share a key (equal logits); NaN ranks
// below every number, -inf included; kTopkGone marks removed or absent
// entries and ranks below NaN.  Because k <= E, the k winners are always
// real, distinct expert indices, whatever the logits hold.
constexpr int32_t kTopkGone = INT32_MIN;
constexpr int32_t kTopkNaN = INT32_MIN + 1;

__device__ __forceinline__ int32_t topk_key(float f) {
  if (f != f) return kTopkNaN;
  const int32_t b = __float_as_int(f == 0.f ? 0.f : f);
  return b >= 0 ? b : b ^ 0x7fffffff;
}

__device__ __forceinline__ float topk_value(int32_t key) {
  return __int_as_float(key >= 0 ? key : key ^ 0x7fffffff);
}

// One wavefront per token.  Lane l holds the keys of experts e = l + 64*i,
// i < EPL.  k rounds of a wave-wide arg-max; ties go to the lower expert
// index.  Weights: p_j = exp(l_j - l_max) over the k kept logits (l_max the
// first winner), normalised to sum 1.  Non-finite logits: a NaN or -inf
// logit gets p = 0 when l_max is finite; when l_max is +inf, each +inf
// logit gets p = 1 and the rest 0; when l_max is -inf or NaN (no kept logit
// is a number above -inf), every kept expert gets p = 1.
template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ logits, int64_t T, int E, int k,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float *l = logits + t * E;
  int32_t v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? topk_key(l[e]) : kTopkGone;
  }
  int32_t kmax = 0;
  float denom = 0.f;
  float my_p = 0.f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    // local best of this lane (ascending index order, strict > keeps lowest)
    int32_t bv = kTopkGone;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      if (v[i] > bv) { bv = v[i]; bi = e; }
    }
    // wave reduce: larger key wins, equal keys -> lower index
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const int32_t ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    // remove the winner
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i == bi) v[i] = kTopkGone;
    if (j == 0) kmax = bv;
    const float lmax = topk_value(kmax), lj = topk_value(bv);
    float p;
    if (kmax == kTopkNaN || lmax == -INFINITY) p = 1.f;
    else if (lmax == INFINITY) p = lj == INFINITY ? 1.f : 0.f;
    else p = bv == kTopkNaN ? 0.f : expf(lj - lmax);
    denom += p;
    if (lane == j) { my_idx = bi; my_p = p; }
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_idx;
    topk_w[t * k + lane] = my_p / denom;
  }
}

hipError_t launch_router_gemm_f32(const float *x, const float *w,
                                  const float *bias, float *logits, int64_t T,
                                  int64_t H, int64_t E, hipStream_t s) {
  const int64_t n = T * E;
  const int bs = 256;
  const int64_t grid = (n + bs - 1) / bs;
  router_gemm_f32_kernel<<<dim3((unsigned)grid), dim3(bs), 0, s>>>(
      x, w, bias, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int64_t T, int E, int k,
                       int32_t *idx, float *w, hipStream_t s) {
  const int wpb = 4;  // wavefronts (tokens) per block
  const int64_t grid = (T + wpb - 1) / wpb;
  dim3 g((unsigned)grid), b(64 * wpb);
  if (E <= 64) topk_kernel<1><<<g, b, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 128) topk_kernel<2><<<g, b, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 256) topk_kernel<4><<<g, b, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 512) topk_kernel<8><<<g, b, 0, s>>>(logits, T, E, k, idx, w);
  else topk_kernel<16><<<g, b, 0, s>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
