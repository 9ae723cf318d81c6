// Local dispatch: per-expert counts and offsets, a stable placement of every
// (token, slot) pair routed to this GPU's experts, and the row copy.
// Wide-EP explainer, 前提条件:GPU間の高速通信 (dispatch to the expert) and
// MoEの課題 (counts are only known once the router has run).
//
// Four launches, all on the caller's stream, none needing the host to know a
// count:
//   1. hist:    each block counts its chunk of flat slots per local expert
//               (LDS histogram) -> hist[e][blk]
//   2. scan:    one block turns hist (expert-major) into exclusive prefixes:
//               base[e][blk] = offsets[e] + slots of e in earlier chunks;
//               writes counts and offsets
//   3. scatter: one wavefront per chunk walks its slots in order, 64 at a
//               time; a slot's rank among equal experts inside the 64 comes
//               from ballots over the expert id bits (a wave-level match),
//               plus a running per-expert count in LDS -> stable rows
//   4. gather:  copies x[row_src[r] / k] into x_perm[r] with 16-byte vectors
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void permute_hist_kernel(
    const int32_t *__restrict__ idx, int64_t F, int e_begin, int n_local,
    int chunk, int nblk, int32_t *__restrict__ hist) {
  extern __shared__ int32_t bins[];
  for (int e = threadIdx.x; e < n_local; e += blockDim.x) bins[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)blockIdx.x * chunk;
  const int64_t f1 = min(F, f0 + chunk);
  for (int64_t f = f0 + threadIdx.x; f < f1; f += blockDim.x) {
    const uint32_t e = (uint32_t)(idx[f] - e_begin);
    if (e < (uint32_t)n_local) atomicAdd(&bins[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_local; e += blockDim.x)
    hist[(int64_t)e * nblk + blockIdx.x] = bins[e];
}

// Exclusive scan of hist[n_local * nblk] (expert-major), in place, one block
// of 1024 threads.  Also writes offsets[0..n_local] and counts[0..n_local).
// The array is walked in tiles of 4096 entries, four consecutive entries per
// thread (so a wavefront's loads and stores cover contiguous 1 KB).  Per
// tile: an inclusive scan of the thread sums inside each wavefront (lane
// shuffles), the 16 wavefront totals through LDS, and a running carry, so a
// tile costs two barriers; the next tile's loads overlap the current scan.
__global__ __launch_bounds__(1024) void permute_scan_kernel(
    int32_t *__restrict__ hist, int n_local, int nblk,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
  constexpr int NWAVE = 1024 / 64;
  __shared__ int32_t wsum[NWAVE];
  __shared__ int32_t offs[4097];
  const int64_t total = (int64_t)n_local * nblk;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t carry = 0;
  int32_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = 4 * tid + j < total ? hist[4 * tid + j] : 0;
  for (int64_t base = 0; base < total; base += 4096) {
    const int64_t i0 = base + 4 * tid;
    // the next tile's entries are loaded while this one is scanned
    int32_t vn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      vn[j] = i0 + 4096 + j < total ? hist[i0 + 4096 + j] : 0;
    const int32_t s = v[0] + v[1] + v[2] + v[3];
    int32_t x = s;  // inclusive prefix of s over the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int32_t before = 0, tile = 0;  // sums of the wavefronts before this one, of all
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) {
      const int32_t t = wsum[q];
      before += q < wv ? t : 0;
      tile += t;
    }
    int32_t run = carry + before + x - s;  // exclusive prefix of entry i0
    // expert e and block r of entry i0 (one division per tile, not per entry)
    int e = (int)(i0 / nblk), r = (int)(i0 - (int64_t)e * nblk);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = i0 + j;
      if (i < total) {
        hist[i] = run;
        if (r == 0) offs[e] = run;
        run += v[j];
      }
      if (++r == nblk) { r = 0; ++e; }
    }
    carry += tile;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = vn[j];
    __syncthreads();  // wsum is rewritten by the next tile
  }
  if (tid == 0) offs[n_local] = carry;
  __syncthreads();
  for (int e = tid; e <= n_local; e += 1024) {
    offsets[e] = offs[e];
    if (e < n_local) counts[e] = offs[e + 1] - offs[e];
  }
}

// One wavefront per chunk of CHUNK flat slots.  The chunk's expert ids and
// weights, and the chunk's base row of every local expert, are loaded up
// front with independent loads; the ranking then runs on ballots and LDS
// alone, so the chunk costs a few memory round trips, not one per 64 slots.
template <int CHUNK>
__global__ __launch_bounds__(64) void permute_scatter_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ w, int64_t F,
    int e_begin, int n_local, int nbits, int nblk,
    const int32_t *__restrict__ base, int32_t *__restrict__ row_src,
    int32_t *__restrict__ inv, float *__restrict__ s_perm) {
  constexpr int STEPS = CHUNK / 64;
  extern __shared__ int32_t running[];  // next row of each local expert
  const int lane = threadIdx.x;
  const int64_t f0 = (int64_t)blockIdx.x * CHUNK;
  uint32_t ev[STEPS];
  float wv[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int64_t f = f0 + st * 64 + lane;
    ev[st] = f < F ? (uint32_t)(idx[f] - e_begin) : 0xffffffffu;
    wv[st] = (f < F && s_perm) ? w[f] : 0.f;
  }
  for (int e = lane; e < n_local; e += 64)
    running[e] = base[(int64_t)e * nblk + blockIdx.x];
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int64_t f = f0 + st * 64 + lane;
    const uint32_t e = ev[st];
    const bool local = e < (uint32_t)n_local;
    uint64_t match = __ballot(local);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1u;
      const uint64_t bb = __ballot(local && bit);
      match &= bit ? bb : ~bb;
    }
    int32_t r = -1;
    if (local) r = running[e] + __popcll(match & lt_mask);
    // every lane has read running[] above before any leader updates it
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (local && (match & lt_mask) == 0) running[e] += __popcll(match);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    if (f < F) inv[f] = r;
    if (local) {
      row_src[r] = (int32_t)f;
      if (s_perm) s_perm[r] = wv[st];
    }
  }
}

// x_perm[r] = x[row_src[r] / k] for r < offsets[n_local]; rows are `vecs`
// 16-byte vectors long.
__global__ __launch_bounds__(256) void permute_gather_kernel(
    const uint4 *__restrict__ x, int64_t vecs, int k,
    const int32_t *__restrict__ row_src, const int32_t *__restrict__ R_ptr,
    uint4 *__restrict__ x_perm) {
  const int R = *R_ptr;
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const int64_t t = row_src[r] / k;
    const uint4 *src = x + t * vecs;
    uint4 *dst = x_perm + (int64_t)r * vecs;
    for (int64_t c = threadIdx.x; c < vecs; c += blockDim.x) dst[c] = src[c];
  }
}

int permute_chunk(int64_t F, int64_t n_local) {
  (void)F;
  return n_local <= 64 ? 256 : 1024;
}

// counts[0, n) = 0 and offsets[0, n] = 0 (an empty batch).  A kernel rather
// than a memset, so that a caller may capture the call in a graph.
__global__ __launch_bounds__(256) void permute_zero_kernel(int32_t *counts,
                                                           int32_t *offsets,
                                                           int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i <= n; i += gridDim.x * 256) {
    if (i < n) counts[i] = 0;
    offsets[i] = 0;
  }
}

hipError_t launch_permute_empty(int32_t *counts, int32_t *offsets,
                                int64_t n_local, hipStream_t s) {
  const int64_t blocks = (n_local + 1 + 255) / 256;
  permute_zero_kernel<<<(unsigned)(blocks < 64 ? blocks : 64), 256, 0, s>>>(
      counts, offsets, (int)n_local);
  return hipGetLastError();
}

size_t permute_workspace_bytes(int64_t T, int64_t k, int64_t n_local) {
  const int64_t F = T * k;
  const int chunk = permute_chunk(F, n_local);
  const int64_t nblk = F > 0 ? (F + chunk - 1) / chunk : 1;
  return (size_t)(((nblk * n_local * 4) + 255) / 256 * 256);
}

hipError_t launch_permute(const int32_t *idx, const float *w, const void *x,
                          int64_t T, int64_t k, int64_t row_bytes,
                          int64_t e_begin, int64_t n_local, void *x_perm,
                          float *s_perm, int32_t *row_src, int32_t *inv,
                          int32_t *counts, int32_t *offsets, void *ws,
                          int num_cus, hipStream_t s) {
  const int64_t F = T * k;
  const int chunk = permute_chunk(F, n_local);
  const int nblk = (int)((F + chunk - 1) / chunk);
  int32_t *hist = (int32_t *)ws;
  int nbits = 0;
  while ((1ll << nbits) < n_local) ++nbits;
  const size_t lds = (size_t)n_local * 4;
  permute_hist_kernel<<<nblk, 256, lds, s>>>(idx, F, (int)e_begin,
                                              (int)n_local, chunk, nblk, hist);
  permute_scan_kernel<<<1, 1024, 0, s>>>(hist, (int)n_local, nblk, counts,
                                         offsets);
  if (chunk == 256)
    permute_scatter_kernel<256><<<nblk, 64, lds, s>>>(
        idx, w, F, (int)e_begin, (int)n_local, nbits, nblk, hist, row_src,
        inv, (w ? s_perm : nullptr));
  else
    permute_scatter_kernel<1024><<<nblk, 64, lds, s>>>(
        idx, w, F, (int)e_begin, (int)n_local, nbits, nblk, hist, row_src,
        inv, (w ? s_perm : nullptr));
  if (x && x_perm) {
    const int64_t vecs = row_bytes / 16;
    int64_t grid = F < (int64_t)num_cus * 8 ? F : (int64_t)num_cus * 8;
    if (grid < 1) grid = 1;
    permute_gather_kernel<<<(unsigned)grid, 256, 0, s>>>(
        (const uint4 *)x, vecs, (int)k, row_src, offsets + n_local,
        (uint4 *)x_perm);
  }
  return hipGetLastError();
}

}  // namespace moe
