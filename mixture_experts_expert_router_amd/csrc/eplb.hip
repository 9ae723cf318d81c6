// Expert-parallel load balancing on the device: the plan (copies per
// expert and their placement on ranks) from the device histogram of earlier
// routing, and the dispatch of the current routing to one rank's slots.
// "Wide-EPとは?" explainer, section 負荷の偏り:EPLB: skewed expert loads
// make the GPU holding the hot experts the bottleneck; between forward
// passes the balancer looks at the loads, rearranges the placement and gives
// the heaviest experts copies on several GPUs.
//
// Plan (one workgroup; integer arithmetic only, so it equals a host
// computation of the same rule bit for bit):
//   1. every expert gets one copy; each spare slot goes to the expert with
//      the largest load per copy, n_e / r_e (compared exactly as n_a r_b >
//      n_b r_a; ties to the lower expert): a workgroup arg-max per spare
//      slot;
//   2. copy i of r takes rows [floor(i n / r), floor((i+1) n / r)) of its
//      expert's n rows; the copies are sorted by decreasing rows (ties:
//      lower expert, lower copy) with a bitonic sort of 64-bit keys in LDS;
//   3. one wavefront places them in that order, each on the rank with the
//      smallest load among those with a free slot that do not yet hold the
//      expert (if none: among those with a free slot; ties: lower rank);
//      every lane keeps the loads of its ranks in registers and the pick is
//      a wavefront arg-min;
//   4. rank g owns slots [g S/G, (g+1) S/G), in increasing (expert, copy)
//      order.
//
// Dispatch to slots [s_begin, s_begin + n_slots): the full permute over all
// E experts orders every expert's entries stably (counts, offsets, row of
// each entry); copy i of expert e then owns the contiguous rows [off_e + lo,
// off_e + hi) of that layout, with lo, hi from the current count of e, so a
// slot's rows are a copy of one contiguous range.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxE = 1024;
constexpr int kPlanMaxS = 4096;
constexpr int kPlanMaxG = 1024;

__device__ __forceinline__ int64_t copy_lo(int64_t n, int64_t r, int64_t i) {
  return i * n / r;
}

__global__ __launch_bounds__(kPlanThreads) void eplb_plan_kernel(
    const int32_t *__restrict__ counts, int E, int S, int G,
    int32_t *__restrict__ rep_out, int32_t *__restrict__ rep_first_out,
    int32_t *__restrict__ rep_slot, int32_t *__restrict__ slot_expert,
    int32_t *__restrict__ slot_copy) {
  __shared__ int32_t cnt[kPlanMaxE];
  __shared__ int32_t rep[kPlanMaxE];
  __shared__ int32_t first[kPlanMaxE + 1];
  __shared__ uint64_t keys[kPlanMaxS];
  __shared__ int32_t rank_of[kPlanMaxS];
  __shared__ int32_t wbest[kPlanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += kPlanThreads) {
    cnt[e] = max(counts[e], 0);
    rep[e] = 1;
  }
  __syncthreads();

  // 1. replication: (n_a, r_a) beats (n_b, r_b) when n_a r_b > n_b r_a, or
  // equal and a < b.  E <= 1024: one expert per thread.
  auto better = [&](int a, int b) {
    if (b < 0) return a >= 0;
    if (a < 0) return false;
    const int64_t x = (int64_t)cnt[a] * rep[b], y = (int64_t)cnt[b] * rep[a];
    return x > y || (x == y && a < b);
  };
  for (int extra = 0; extra < S - E; ++extra) {
    int b = tid < E ? tid : -1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const int o = __shfl_xor(b, off, 64);
      if (better(o, b)) b = o;
    }
    if (lane == 0) wbest[wv] = b;
    __syncthreads();
    if (tid == 0) {
      int best = -1;
      for (int w = 0; w < kPlanThreads / 64; ++w)
        if (better(wbest[w], best)) best = wbest[w];
      ++rep[best];
    }
    __syncthreads();
  }

  // prefix of the copy counts (one thread: E <= 1024 additions)
  if (tid == 0) {
    int32_t run = 0;
    for (int e = 0; e < E; ++e) {
      first[e] = run;
      run += rep[e];
    }
    first[E] = run;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kPlanThreads) {
    rep_first_out[e] = first[e];
    if (e < E) rep_out[e] = rep[e];
  }

  // 2. sort keys: decreasing rows, then increasing copy index q
  int P = 1;
  while (P < S) P <<= 1;
  for (int q = tid; q < P; q += kPlanThreads) {
    uint64_t key = ~0ull;
    if (q < S) {
      const int e = upper_bound_minus1(first, E, q);
      const int64_t n = cnt[e], r = rep[e], i = q - first[e];
      const uint32_t rows = (uint32_t)(copy_lo(n, r, i + 1) - copy_lo(n, r, i));
      key = ((uint64_t)(0xffffffffu - rows) << 32) | (uint32_t)q;
    }
    keys[q] = key;
    if (q < S) rank_of[q] = -1;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kPlanThreads) {
        const int l = i ^ j;
        if (l > i) {
          const bool up = (i & k) == 0;
          const uint64_t a = keys[i], b = keys[l];
          if ((a > b) == up) { keys[i] = b; keys[l] = a; }
        }
      }
      __syncthreads();
    }

  // 3. placement by wavefront 0; lane l owns ranks l, l + 64, ...
  if (wv == 0) {
    constexpr int RPL = kPlanMaxG / 64;
    const int per = S / G;
    int64_t load[RPL];
    int32_t used[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) { load[m] = 0; used[m] = 0; }
    for (int j = 0; j < S; ++j) {
      const int q = (int)(keys[j] & 0xffffffffu);
      const int e = upper_bound_minus1(first, E, q);
      const int64_t n = cnt[e], r = rep[e], i = q - first[e];
      const int64_t rows = copy_lo(n, r, i + 1) - copy_lo(n, r, i);
      int pick = -1;
      for (int pass = 0; pass < 2 && pick < 0; ++pass) {
        int64_t bl = INT64_MAX;
        int bg = 0x7fffffff;
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
          const int g = lane + 64 * m;
          if (g >= G || used[m] == per) continue;
          bool holds = false;
          if (pass == 0)
            for (int c = first[e]; c < first[e + 1]; ++c) holds |= rank_of[c] == g;
          if (holds) continue;
          if (load[m] < bl) { bl = load[m]; bg = g; }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const int64_t ol = __shfl_xor(bl, off, 64);
          const int og = __shfl_xor(bg, off, 64);
          if (ol < bl || (ol == bl && og < bg)) { bl = ol; bg = og; }
        }
        if (bg != 0x7fffffff) pick = bg;
      }
#pragma unroll
      for (int m = 0; m < RPL; ++m)
        if (lane + 64 * m == pick) { load[m] += rows; ++used[m]; }
      // capacity S = number of copies, so some rank always has a free slot
      if (lane == 0) rank_of[q] = max(pick, 0);
      // every lane reads rank_of[] in the next step's holds test
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  }
  __syncthreads();

  // 4. slot numbers: copies of rank g in increasing q
  const int per = S / G;
  for (int q = tid; q < S; q += kPlanThreads) {
    const int g = rank_of[q];
    int before = 0;
    for (int p = 0; p < q; ++p) before += rank_of[p] == g;
    const int s = min(g * per + before, S - 1);
    const int e = upper_bound_minus1(first, E, q);
    rep_slot[q] = s;
    slot_expert[s] = e;
    slot_copy[s] = q - first[e];
  }
}

// Local slot counts under the current routing, their exclusive scan, and
// the first row of each slot in the full (all-expert) layout.  One block.
__global__ __launch_bounds__(1024) void eplb_slot_rows_kernel(
    const int32_t *__restrict__ rep_first, const int32_t *__restrict__ slot_expert,
    const int32_t *__restrict__ slot_copy, int s_begin, int n_slots,
    const int32_t *__restrict__ full_offsets, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ full_start) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (n_slots + 1023) / 1024;
  const int s0 = min(n_slots, tid * per), s1 = min(n_slots, s0 + per);
  int32_t sum = 0;
  for (int s = s0; s < s1; ++s) {
    const int e = slot_expert[s_begin + s], i = slot_copy[s_begin + s];
    const int64_t r = rep_first[e + 1] - rep_first[e];
    const int64_t n = full_offsets[e + 1] - full_offsets[e];
    const int64_t lo = copy_lo(n, r, i), hi = copy_lo(n, r, i + 1);
    counts[s] = (int32_t)(hi - lo);
    full_start[s] = full_offsets[e] + (int32_t)lo;
    sum += (int32_t)(hi - lo);
  }
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
    offsets[s] = run;
    run += counts[s];
  }
  if (tid == 1023) offsets[n_slots] = part[1023];
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t *p, int64_t n,
                                                       int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    p[i] = v;
}

// Local row rho -> its entry f in the full layout; row_src, inv, s_perm.
__global__ __launch_bounds__(256) void eplb_remap_kernel(
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ full_start,
    int n_slots, const int32_t *__restrict__ full_row_src,
    const float *__restrict__ w, int32_t *__restrict__ row_src,
    int32_t *__restrict__ inv, float *__restrict__ s_perm) {
  const int R = offsets[n_slots];
  for (int rho = blockIdx.x * 256 + threadIdx.x; rho < R; rho += gridDim.x * 256) {
    const int s = upper_bound_minus1(offsets, n_slots, rho);
    const int32_t f = full_row_src[full_start[s] + (rho - offsets[s])];
    row_src[rho] = f;
    inv[f] = rho;
    if (s_perm) s_perm[rho] = w[f];
  }
}

hipError_t launch_eplb_plan(const int32_t *counts, int E, int S, int G,
                            int32_t *rep, int32_t *rep_first,
                            int32_t *rep_slot, int32_t *slot_expert,
                            int32_t *slot_copy, hipStream_t s) {
  eplb_plan_kernel<<<1, kPlanThreads, 0, s>>>(counts, E, S, G, rep, rep_first,
                                              rep_slot, slot_expert, slot_copy);
  return hipGetLastError();
}

size_t permute_replicated_workspace_bytes(int64_t T, int64_t k, int64_t E,
                                          int64_t n_slots) {
  const int64_t F = T * k;
  auto r256 = [](int64_t b) { return (size_t)((b + 255) / 256 * 256); };
  return permute_workspace_bytes(T, k, E) + r256(F * 4) * 2 +
         r256((E + 1) * 4) * 2 + r256(n_slots * 4);
}

hipError_t launch_permute_replicated(
    const int32_t *idx, const float *w, const void *x, int64_t T, int64_t k,
    int64_t row_bytes, int64_t E, const int32_t *rep_first,
    const int32_t *rep_slot, const int32_t *slot_expert,
    const int32_t *slot_copy, int64_t s_begin, int64_t n_slots, void *x_perm,
    float *s_perm, int32_t *row_src, int32_t *inv, int32_t *counts,
    int32_t *offsets, void *ws, int num_cus, hipStream_t s) {
  (void)rep_slot;
  const int64_t F = T * k;
  auto r256 = [](int64_t b) { return (size_t)((b + 255) / 256 * 256); };
  char *p = (char *)ws;
  void *pws = p;                           // the full permute's workspace first:
  p += permute_workspace_bytes(T, k, E);   // its error word is ours
  int32_t *full_row_src = (int32_t *)p; p += r256(F * 4);
  int32_t *full_inv = (int32_t *)p; p += r256(F * 4);
  int32_t *full_counts = (int32_t *)p; p += r256((E + 1) * 4);
  int32_t *full_offsets = (int32_t *)p; p += r256((E + 1) * 4);
  int32_t *full_start = (int32_t *)p;
  hipError_t err = launch_permute(idx, nullptr, nullptr, T, k, 0, E, 0, E,
                                  nullptr, nullptr, full_row_src, full_inv,
                                  full_counts, full_offsets, pws, num_cus, s);
  if (err != hipSuccess) return err;
  eplb_slot_rows_kernel<<<1, 1024, 0, s>>>(rep_first, slot_expert, slot_copy,
                                           (int)s_begin, (int)n_slots,
                                           full_offsets, counts, offsets,
                                           full_start);
  const int64_t blocks = std::min<int64_t>((F + 255) / 256, 8LL * num_cus);
  fill_i32_kernel<<<(unsigned)std::max<int64_t>(blocks, 1), 256, 0, s>>>(inv, F, -1);
  eplb_remap_kernel<<<(unsigned)std::max<int64_t>(blocks, 1), 256, 0, s>>>(
      offsets, full_start, (int)n_slots, full_row_src, w, row_src, inv,
      w ? s_perm : nullptr);
  err = hipGetLastError();
  if (err != hipSuccess || !(x && x_perm)) return err;
  return launch_permute_gather(x, row_bytes, k, row_src, offsets + n_slots,
                               x_perm, F, num_cus, s);
}

}  // namespace moe
