// fp32 expert FFN (tiny shapes: the fp32 workload exists to check the
// arithmetic, not to be fast).  Same contract as the bf16 grouped GEMMs:
// rows of expert e are [offsets[e], offsets[e+1]); the routing scale goes
// into the gate/up epilogue (BioNeMo MoE article, GroupedLinear section,
// ScaledSwiGLU).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// a[r, i] = s[r] * SiLU(x[r] . Wg[e, i]) * (x[r] . Wu[e, i]), one thread per
// output.  Rows at or past R_cap are never touched.
__global__ void gate_up_f32_kernel(const float *__restrict__ x,
                                   const int32_t *__restrict__ offsets,
                                   const float *__restrict__ s, int n_local,
                                   int64_t R_cap, int64_t H, int64_t I,
                                   const float *__restrict__ wg,
                                   const float *__restrict__ wu,
                                   float *__restrict__ a) {
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int R = min(max(offsets[n_local], 0), (int)R_cap);
  if (o >= (int64_t)R * I) return;
  const int r = (int)(o / I);
  const int64_t i = o % I;
  const int e = upper_bound_minus1(offsets, n_local, r);
  const float *xr = x + (int64_t)r * H;
  const float *g_row = wg + ((int64_t)e * I + i) * H;
  const float *u_row = wu + ((int64_t)e * I + i) * H;
  float g = 0.f, u = 0.f;
  for (int64_t h = 0; h < H; ++h) {
    g = fmaf(xr[h], g_row[h], g);
    u = fmaf(xr[h], u_row[h], u);
  }
  a[o] = (s ? s[r] : 1.f) * (g / (1.f + expf(-g))) * u;
}

// y[r, h] = a[r] . Wd[e, h], one thread per output.
__global__ void down_f32_kernel(const float *__restrict__ a,
                                const int32_t *__restrict__ offsets,
                                int n_local, int64_t R_cap, int64_t H,
                                int64_t I, const float *__restrict__ wd,
                                float *__restrict__ y) {
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int R = min(max(offsets[n_local], 0), (int)R_cap);
  if (o >= (int64_t)R * H) return;
  const int r = (int)(o / H);
  const int64_t h = o % H;
  const int e = upper_bound_minus1(offsets, n_local, r);
  const float *ar = a + (int64_t)r * I;
  const float *w = wd + ((int64_t)e * H + h) * I;
  float acc = 0.f;
  for (int64_t i = 0; i < I; ++i) acc = fmaf(ar[i], w[i], acc);
  y[o] = acc;
}

hipError_t launch_gate_up_f32(const float *x_perm, const int32_t *offsets,
                              const float *s_perm, int n_local, int64_t R_cap,
                              int64_t H, int64_t I, const float *w_gate,
                              const float *w_up, float *a, hipStream_t s) {
  const int64_t n = R_cap * I;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0)
    gate_up_f32_kernel<<<(unsigned)grid, 256, 0, s>>>(
        x_perm, offsets, s_perm, n_local, R_cap, H, I, w_gate, w_up, a);
  return hipGetLastError();
}

hipError_t launch_down_f32(const float *a, const int32_t *offsets,
                           int n_local, int64_t R_cap, int64_t H, int64_t I,
                           const float *w_down, float *y, hipStream_t s) {
  const int64_t n = R_cap * H;
  const int64_t grid = (n + 255) / 256;
  if (grid > 0)
    down_f32_kernel<<<(unsigned)grid, 256, 0, s>>>(a, offsets, n_local, R_cap,
                                                   H, I, w_down, y);
  return hipGetLastError();
}

// *err = kDevErrRows when the offsets decrease or run past R_cap, else 0.
__global__ __launch_bounds__(256) void check_offsets_kernel(
    const int32_t *__restrict__ offsets, int n_local, int R_cap,
    int32_t *__restrict__ err) {
  int bad = 0;
  for (int e = threadIdx.x; e < n_local; e += 256)
    bad |= seg_bad(offsets, e, R_cap);
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) *err = bad ? kDevErrRows : 0;
}

hipError_t launch_check_offsets(const int32_t *offsets, int n_local,
                                int64_t R_cap, int32_t *err, hipStream_t s) {
  check_offsets_kernel<<<1, 256, 0, s>>>(offsets, n_local, (int)R_cap, err);
  return hipGetLastError();
}

}  // namespace moe
