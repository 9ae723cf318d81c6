// Decode-sized expert FFN (gate/up, ScaledSwiGLU, down) as one persistent
// gfx950 kernel.
//
// BioNeMo MoE article, "GroupedLinear Optimizes Expert Computation in MoE
// Models": the fused MLP does not materialise intermediate results, and all
// experts run as one operation.  With a few rows per expert (decode, or an
// EP8 share of a small batch: C3 holds 7-34 rows per expert) every weight
// byte is used by so few rows that the layer is a pure weight stream; the
// grouped path then pays for two launches, their ramp-up and drain, and the
// plan kernels between them.  Here one launch does both projections:
//
//   * Work units.  A gate/up unit is (expert e, group of <= 32 of its rows,
//     64 columns of a): it reads the 64 gate and the 64 matching up rows of
//     W_gate[e] / W_up[e] once and writes a = s * SiLU(g) * u (bf16) for its
//     rows.  A down unit is (expert e, row group, 128 columns of y): it reads
//     128 rows of W_down[e] once and writes y (bf16).  A plan kernel turns
//     the device offsets into unit prefixes (gate/up units of every expert
//     first, then down units) and clears the flags.
//   * Workers.  Two workgroups per CU claim units.  Inside a unit the four
//     wavefronts split K into quarters, so the unit's rows of x (or of a)
//     are read once per unit for 128 weight rows.
//   * Scheduling.  Units are claimed in order through one atomic counter:
//     the gate/up units of every expert, then the down units.  A down unit
//     of expert e waits until every gate/up unit of e has published its part
//     of a; those precede it and gate/up units never wait, so every unit a
//     waiting workgroup depends on has already been claimed by a running
//     workgroup and finishes: the wait always ends, however many workgroups
//     are resident.  (A wall-clock bound on the wait sets MOE_DEVERR_WAIT
//     and gives up instead of hanging.)
//   * Hand-over of a, across the XCDs' separate L2 caches, without
//     device-scope fences (on gfx950 those write back or invalidate a whole
//     L2; in a polling loop run by many workgroups they would stall every
//     XCD).  Everything one workgroup writes for another goes through
//     relaxed device-scope atomic stores and loads, which the hardware
//     serves at the device's coherence point rather than from a CU's or an
//     XCD's cache: the gate/up unit stores its part of a that way (64 bits
//     at a time), waits for the stores to complete (s_waitcnt vmcnt(0), an
//     ordering-only fence), then sets its flag; the down unit polls its
//     expert's flags and then reads a the same way.  a is small (rows x I
//     bf16) and is the one intermediate, as in the grouped path.
//   * Inside a unit.  Each wavefront streams its quarter of K straight into
//     registers in the v_mfma_f32_16x16x32_bf16 operand layout (lane l: row
//     l % 16 of every 16-row block, 16 contiguous K values of every 64),
//     kDepth k-steps ahead; the four partial accumulators are summed in a
//     fixed order through LDS (deterministic results) and the epilogue
//     writes whole row pieces.
//   * Control flow branches only on workgroup-uniform values: with a
//     per-lane condition around the claim or the loop exit, the compiler's
//     structurizer may split the loop so that most lanes iterate without
//     passing the claim.  So wavefront 0 claims with all its lanes (lane 0
//     adds 1, the others 0; lane 0's result is the unit) and the unit index
//     is made uniform with readfirstlane.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kRG = 32;          // rows per row group (two 16-row blocks)
constexpr int kCI = 64;          // a-columns per gate/up unit
constexpr int kCH = 128;         // y-columns per down unit
constexpr int kNB = 8;           // 16-row weight blocks per unit
#ifndef MOE_FUSED_DEPTH
#define MOE_FUSED_DEPTH 3
#endif
constexpr int kDepth = MOE_FUSED_DEPTH;  // k-steps of 32 in flight per wavefront
constexpr int kStride = 132;     // floats per staged row (128 + 4 pad)
// Bound on one wait, in ticks of the 100 MHz constant clock (0.2 s).
constexpr uint64_t kWaitTicks = 20000000;

// Workspace (int32 words): the error header; the claim counter; the gate/up
// and down unit totals; then p1, p2 (exclusive prefixes of the gate/up and
// of the down units over the experts, G + 1 entries each), ng (row groups
// per expert) and one flag per gate/up unit (numbered by p1).
constexpr int kCtl = (int)(kErrHeaderBytes / 4);
constexpr int kArr = kCtl + 64;

struct FusedArgs {
  const uint16_t *x;        // [T, H] with row_src, else [R_cap, H]
  const int32_t *row_src;   // permuted row r reads x[min(row_src[r] / kdiv, x_last)]
  int kdiv, x_last;
  const int32_t *offsets;   // [G + 1]
  const float *s_perm;      // [R_cap] or null
  const uint16_t *wg, *wu;  // [G, I, H]
  const uint16_t *wd;       // [G, H, I]
  uint16_t *a;              // [R_cap, I]
  uint16_t *y;              // [R_cap, H]
  int32_t *ws;
  int G, H, I, r_cap;
};

// Per expert: ng = row groups, gate/up units ng * I/kCI, down units
// ng * ceil(H/kCH); exclusive prefixes p1, p2 of the unit counts (G + 1
// entries each); the counter and the flags of all gate/up units cleared;
// error word set.  One block.
__global__ __launch_bounds__(1024) void ffn_fused_plan_kernel(
    const int32_t *__restrict__ offsets, int G, int r_cap, int nci, int nch,
    int32_t *__restrict__ ws) {
  __shared__ int32_t wsum[2][16];
  __shared__ int32_t bad_or;
  int32_t *ctl = ws + kCtl;
  int32_t *p1 = ws + kArr, *p2 = p1 + G + 1, *ng = p2 + G + 1, *flags = ng + G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) bad_or = 0;
  const int per = (G + 1023) / 1024;
  const int e0 = min(G, tid * per), e1 = min(G, e0 + per);
  int32_t s[2] = {0, 0};
  int bad = 0;
  for (int e = e0; e < e1; ++e) {
    int b, en;
    seg_rows(offsets, e, r_cap, b, en);
    const int g = (en - b + kRG - 1) / kRG;
    s[0] += g * nci;
    s[1] += g * nch;
    bad |= seg_bad(offsets, e, r_cap) ? kDevErrRows : 0;
  }
  int32_t x[2] = {s[0], s[1]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int32_t v = __shfl_up(x[c], off, 64);
      if (lane >= off) x[c] += v;
    }
  }
  if (lane == 63) { wsum[0][wv] = x[0]; wsum[1][wv] = x[1]; }
  __syncthreads();
  int32_t run[2], total[2];
  for (int c = 0; c < 2; ++c) {
    int32_t before = 0, all = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int32_t v = wsum[c][q];
      before += q < wv ? v : 0;
      all += v;
    }
    run[c] = before + x[c] - s[c];
    total[c] = all;
  }
  for (int e = e0; e < e1; ++e) {
    int b, en;
    seg_rows(offsets, e, r_cap, b, en);
    const int g = (en - b + kRG - 1) / kRG;
    p1[e] = run[0];
    p2[e] = run[1];
    ng[e] = g;
    run[0] += g * nci;
    run[1] += g * nch;
  }
  if (tid == 0) {
    p1[G] = total[0];
    p2[G] = total[1];
    ctl[0] = 0;
    ctl[1] = total[0];
    ctl[2] = total[1];
  }
  for (int u = tid; u < total[0]; u += 1024) flags[u] = 0;
  if (bad) atomicOr(&bad_or, bad);
  __syncthreads();
  if (tid == 0) ws[0] = bad_or;
}

// acc[m][j] += sum over k-steps s in [s0, s1) of A_m(s) . B_j(s)^T.  ap[m]
// points at the lane's first A element (row l % 16 of the block); B block
// j's rows start at the workgroup-uniform bb[j] and the lane's element is
// boff further (a 32-bit offset, so the loads take the scalar-base +
// vector-offset form).  K order: the MFMA sums its 32 K values in any order
// as long as A and B agree, so a pair of steps (64 K values, 128 bytes of a
// row) is split so that lane l takes the 16 contiguous values 16*(l/16) ..
// +16, the first 8 in the pair's first step and the last 8 in its second:
// the two loads of a pair then touch each 128-byte line of a row once per
// instruction (one L2 request per row, not two 64-byte halves).  ap[m] and
// boff include the lane's 16*(l/16).
// kCoherentA: A is another workgroup's output, read through coherent loads.
// kDepth steps are in flight: each step's registers are refilled with the
// step kDepth ahead right after its MFMAs (past the end: the last step
// again, a harmless re-read that keeps the loop free of branches), and the
// last ns % kDepth steps run from registers after the loop.
template <int MB, bool kCoherentA>
__device__ __forceinline__ void stream_mma(const uint16_t *const (&ap)[MB],
                                           const uint16_t *const (&bb)[kNB],
                                           uint32_t boff, int s0, int s1,
                                           f32x4 (&acc)[MB][kNB]) {
  if (s1 <= s0) return;
  bf16x8 aq[kDepth][MB], bq[kDepth][kNB];
  const int last = s1 - 1;
  auto load = [&](int d, int step) {
    const int st = min(step, last);
    // element offset of step st: its pair's 64 values, then its half
    const int64_t off = (int64_t)(st >> 1) * 64 + (st & 1) * 8;
#pragma unroll
    for (int m = 0; m < MB; ++m)
      aq[d][m] = kCoherentA ? load_coherent16(ap[m] + off)
                            : *(const bf16x8 *)(ap[m] + off);
    const uint32_t bo = (boff + (uint32_t)off) * 2u;
#pragma unroll
    for (int j = 0; j < kNB; ++j)
      bq[d][j] = *(const bf16x8 *)((const char *)bb[j] + bo);
  };
  auto mma = [&](int d) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            aq[d][m], bq[d][j], acc[m][j], 0, 0, 0);
  };
  // Scheduling barriers keep each step's loads where they are written: the
  // loop's first step then always waits for the oldest loads in flight, on
  // entry as on every later iteration (reordered, the wait on entry can
  // degrade to waiting for every load).
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    load(d, s0 + d);
    __builtin_amdgcn_sched_barrier(0);
  }
  int s = s0;
  for (; s + kDepth <= s1; s += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      mma(d);
      __builtin_amdgcn_sched_barrier(0);
      load(d, s + d + kDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (s + d < s1) mma(d);
}

// One unit: operand pointers, the K loop of this wavefront's quarter, the
// partial sums staged in LDS (red[w][row][col], col < 128), one barrier.
template <int MB>
__device__ __forceinline__ void unit_mma(const FusedArgs &p, bool gate_up,
                                         int e, int r0, int nr, int chunk,
                                         int wid, int lane, float *red) {
  const int K = gate_up ? p.H : p.I;
  // K (a multiple of 64) in pairs of 32-value steps, a quarter per wavefront
  const int kp = K / 64;
  const int s0 = 2 * (wid * kp / 4), s1 = 2 * ((wid + 1) * kp / 4);
  const int koff = 16 * (lane >> 4), l16 = lane & 15;
  const uint16_t *ap[MB];
  const uint16_t *bb[kNB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int r = r0 + min(m * 16 + l16, nr - 1);
    if (gate_up) {
      const int64_t xr = p.row_src ? min(p.row_src[r] / p.kdiv, p.x_last) : r;
      ap[m] = p.x + xr * p.H + koff;
    } else {
      ap[m] = p.a + (int64_t)r * p.I + koff;
    }
  }
  const int64_t wstride = (int64_t)p.I * p.H;
  // lane offset inside a block of 16 weight rows (row stride K)
  const uint32_t boff = (uint32_t)(l16 * K + koff);
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    if (gate_up) {
      // blocks 0-3: gate rows of the chunk's 64 columns, 4-7: the up rows
      const int c = chunk * kCI + (j & 3) * 16;
      bb[j] = (j < 4 ? p.wg : p.wu) + e * wstride + (int64_t)c * p.H;
    } else {
      // blocks past the last row of W_down re-read the last full block
      // (H is a multiple of 64); their columns are not stored
      const int h = min(chunk * kCH + j * 16, p.H - 16);
      bb[j] = p.wd + e * wstride + (int64_t)h * p.I;
    }
  }
  f32x4 acc[MB][kNB];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][j][r] = 0.f;
  if (gate_up) stream_mma<MB, false>(ap, bb, boff, s0, s1, acc);
  else stream_mma<MB, true>(ap, bb, boff, s0, s1, acc);
  // lane holds column l % 16 and rows 4*(l/16) .. +4 of each 16x16 block
  float *mine = red + wid * (kRG * kStride);
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mine[(m * 16 + 4 * (lane >> 4) + r) * kStride + j * 16 + l16] = acc[m][j][r];
  __syncthreads();
}

// Sum of the four wavefronts' partials of element (row, col), in order.
__device__ __forceinline__ float red_sum(const float *red, int row, int col) {
  const int o = row * kStride + col;
  constexpr int W = kRG * kStride;
  return ((red[o] + red[W + o]) + red[2 * W + o]) + red[3 * W + o];
}

__global__ __launch_bounds__(256, 2) void ffn_fused_kernel(FusedArgs p) {
  __shared__ float red[4 * kRG * kStride];
  __shared__ int s_unit;
  int32_t *ctl = p.ws + kCtl;
  const int32_t *p1 = p.ws + kArr, *p2 = p1 + p.G + 1, *ngs = p2 + p.G + 1;
  int32_t *flags = p.ws + kArr + 3 * p.G + 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int N1 = ctl[1], N = N1 + ctl[2];
  for (;;) {
    if (wid == 0) {
      const int v = atomicAdd(&ctl[0], lane == 0 ? 1 : 0);
      s_unit = __builtin_amdgcn_readfirstlane(v);
    }
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(s_unit);
    __syncthreads();
    if (u >= N) break;
    const bool gate_up = u < N1;
    const int v = gate_up ? u : u - N1;
    const int32_t *pre = gate_up ? p1 : p2;
    const int e = upper_bound_minus1(pre, p.G, v);
    const int local = v - pre[e];
    const int ng = ngs[e];
    const int grp = local % ng, chunk = local / ng;
    int b, en;
    seg_rows(p.offsets, e, p.r_cap, b, en);
    const int r0 = b + grp * kRG, nr = min(kRG, en - r0);
    if (!gate_up) {
      // wait for the flags of every gate/up unit of expert e (wavefront 0
      // polls 64 flags per load; the others wait at the barrier)
      if (wid == 0) {
        const int f0 = p1[e], nf = p1[e + 1] - f0;
        const uint64_t t0 = wall_clock64();
        bool late = false;
        for (int base = 0; base < nf && !late; base += 64) {
          // lanes past the expert's last flag read its first one (set or
          // not, it is one of the flags waited for)
          const int f = f0 + (base + lane < nf ? base + lane : 0);
          for (;;) {
            const bool ok = __hip_atomic_load(&flags[f], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) != 0;
            if (__all(ok)) break;
            if (wall_clock64() - t0 > kWaitTicks) {
              late = true;
              break;
            }
            __builtin_amdgcn_s_sleep(16);
          }
        }
        if (late) atomicOr(&p.ws[0], lane == 0 ? kDevErrWait : 0);
      }
      wait_vmem();
      __syncthreads();
    }
    if (nr <= 16) unit_mma<1>(p, gate_up, e, r0, nr, chunk, wid, lane, red);
    else unit_mma<2>(p, gate_up, e, r0, nr, chunk, wid, lane, red);
    if (gate_up) {
      // a[r0 + row][c0 + c] = s * SiLU(g) * u, 8 columns per piece
      const int c0 = chunk * kCI;
      for (int q0 = 0; q0 < nr * (kCI / 8); q0 += 256) {
        const int q = q0 + tid;
        if (q >= nr * (kCI / 8)) continue;
        const int row = q / (kCI / 8), c8 = (q % (kCI / 8)) * 8;
        const float sc = p.s_perm ? p.s_perm[r0 + row] : 1.f;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int c = c8 + 2 * i + h;
            const float g = red_sum(red, row, c), uu = red_sum(red, row, kCI + c);
            v2[h] = sc * silu_f32(g) * uu;
          }
          w[i] = pack_bf16x2(v2[0], v2[1]);
        }
        store_coherent16(p.a + (int64_t)(r0 + row) * p.I + c0 + c8, w[0],
                         w[1], w[2], w[3]);
      }
      // publish: the coherent stores complete, then the unit's flag
      wait_vmem();
      __syncthreads();
      if (wid == 0)  // every lane stores the same flag
        __hip_atomic_store(&flags[u], 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const int h0 = chunk * kCH;
      const int ncol = min(kCH, p.H - h0);
      for (int q0 = 0; q0 < nr * (ncol / 8); q0 += 256) {
        const int q = q0 + tid;
        if (q >= nr * (ncol / 8)) continue;
        const int row = q / (ncol / 8), c8 = (q % (ncol / 8)) * 8;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = pack_bf16x2(red_sum(red, row, c8 + 2 * i),
                             red_sum(red, row, c8 + 2 * i + 1));
        *(uint4 *)(p.y + (int64_t)(r0 + row) * p.H + h0 + c8) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
      __syncthreads();
    }
  }
}

}  // namespace

size_t ffn_fused_workspace_bytes(int64_t n_local, int64_t R_cap, int64_t I) {
  // at most sum_e ceil(rows_e / kRG) <= R_cap / kRG + n_local row groups
  const size_t units1 = (size_t)(R_cap / kRG + n_local) * (size_t)(I / kCI);
  const size_t words = (size_t)kArr + 3 * (size_t)n_local + 2 + units1;
  return (words * 4 + 255) / 256 * 256;
}

hipError_t launch_ffn_fused_bf16(const uint16_t *x, const int32_t *row_src,
                                 int k, int64_t T, const int32_t *offsets,
                                 const float *s_perm, int n_local,
                                 int64_t R_cap, int H, int I,
                                 const uint16_t *w_gate, const uint16_t *w_up,
                                 const uint16_t *w_down, uint16_t *a,
                                 uint16_t *y, int32_t *ws, int num_cus,
                                 hipStream_t s) {
  const int nci = I / kCI, nch = (H + kCH - 1) / kCH;
  ffn_fused_plan_kernel<<<1, 1024, 0, s>>>(offsets, n_local, (int)R_cap, nci,
                                           nch, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  FusedArgs p{};
  p.x = x; p.row_src = row_src; p.kdiv = row_src ? k : 1;
  p.x_last = row_src ? (int)(T - 1) : (int)R_cap - 1;
  p.offsets = offsets; p.s_perm = s_perm;
  p.wg = w_gate; p.wu = w_up; p.wd = w_down; p.a = a; p.y = y; p.ws = ws;
  p.G = n_local; p.H = H; p.I = I; p.r_cap = (int)R_cap;
  // two workgroups per CU, so that one's claim, pipeline ramp and epilogue
  // overlap the other's weight stream; a grid larger than the work only
  // adds workgroups that claim nothing
  const int64_t upper = (R_cap / kRG + n_local) * (int64_t)(nci + nch);
  const int grid =
      (int)std::max<int64_t>(1, std::min<int64_t>(2 * (int64_t)num_cus, upper));
  ffn_fused_kernel<<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
