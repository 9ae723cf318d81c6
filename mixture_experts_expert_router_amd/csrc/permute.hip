// Local dispatch: per-expert counts and offsets, a stable placement of every
// (token, slot) pair routed to this GPU's experts, and the row copy.
// Wide-EP explainer, 前提条件:GPU間の高速通信 (dispatch to the expert) and
// MoEの課題 (counts are only known once the router has run).
//
// Four launches, all on the caller's stream, none needing the host to know a
// count (small batches take one launch for steps 1-3, then step 4; see
// permute_small_kernel):
//   1. hist:    each block counts its chunk of flat slots per local expert
//               (LDS histogram) -> hist[e][blk], and flags the chunk when
//               one of its indices lies outside [0, E)
//   2. scan:    one block turns hist (expert-major) into exclusive prefixes:
//               base[e][blk] = offsets[e] + slots of e in earlier chunks;
//               writes counts and offsets, and the workspace's error word
//               (kDevErrExpertIndex when a chunk was flagged, else 0)
//   3. scatter: one wavefront per chunk walks its slots in order, 64 at a
//               time; a slot's rank among equal experts inside the 64 comes
//               from ballots over the expert id bits (a wave-level match),
//               plus a running per-expert count in LDS -> stable rows
//   4. gather:  copies x[row_src[r] / k] into x_perm[r] with 16-byte vectors
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Per-expert counts of one chunk of flat slots (LDS histogram), and a flag
// for the chunk: 1 when one of its indices lies outside [0, E) (such a slot
// is dropped like a non-local one; the scan reports it in the error word).
__global__ __launch_bounds__(256) void permute_hist_kernel(
    const int32_t *__restrict__ idx, int64_t F, int E, int e_begin,
    int n_local, int chunk, int nblk, int32_t *__restrict__ hist,
    int32_t *__restrict__ bad_blk) {
  extern __shared__ int32_t bins[];
  for (int e = threadIdx.x; e < n_local; e += blockDim.x) bins[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)blockIdx.x * chunk;
  const int64_t f1 = min(F, f0 + chunk);
  int bad = 0;
  for (int64_t f = f0 + threadIdx.x; f < f1; f += blockDim.x) {
    const int32_t g = idx[f];
    bad |= (uint32_t)g >= (uint32_t)E;
    const uint32_t e = (uint32_t)(g - e_begin);
    if (e < (uint32_t)n_local) atomicAdd(&bins[e], 1);
  }
  bad = __syncthreads_or(bad);
  for (int e = threadIdx.x; e < n_local; e += blockDim.x)
    hist[(int64_t)e * nblk + blockIdx.x] = bins[e];
  if (threadIdx.x == 0) bad_blk[blockIdx.x] = bad;
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
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    const int32_t *__restrict__ bad_blk, int32_t *__restrict__ err) {
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
  int bad = 0;
  for (int b = tid; b < nblk; b += 1024) bad |= bad_blk[b];
  bad = __syncthreads_or(bad);
  if (tid == 0) *err = bad ? kDevErrExpertIndex : 0;
  for (int e = tid; e <= n_local; e += 1024) {
    offsets[e] = offs[e];
    if (e < n_local) counts[e] = offs[e + 1] - offs[e];
  }
}

// Stable rows of one wavefront's 64 consecutive slots: a slot's rank among
// the equal local experts before it in the 64 comes from ballots over the
// expert id bits (a wave-level match); running[e] (LDS, this wavefront's
// alone) holds the next row of expert e and is advanced by the leader of
// each expert group.  Returns the slot's row, or -1 for a non-local slot.
__device__ __forceinline__ int32_t rank_step(uint32_t e, bool local,
                                             int n_local, int nbits,
                                             uint64_t lt_mask,
                                             int32_t *running) {
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
  return r;
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
    const int32_t r = rank_step(e, local, n_local, nbits, lt_mask, running);
    if (f < F) inv[f] = r;
    if (local) {
      row_src[r] = (int32_t)f;
      if (s_perm) s_perm[r] = wv[st];
    }
  }
}

// Steps 1-3 in one workgroup of 1024 threads, for F <= kSmallPermuteF and
// n_local <= kSmallPermuteExperts.  Wavefront w owns the flat slots
// [w*per, (w+1)*per) (per a multiple of 64), in groups of 8 x 64:
//   1. it counts them per local expert into its own LDS row bins[w][.] and
//      keeps their local expert ids in LDS (16 bits each);
//   2. thread e turns column e into prefixes: counts[e] is the column's sum,
//      offsets[e] an exclusive scan of the counts over the block (wavefront
//      shuffles, then the 16 wavefront totals), and bins[w][e] becomes
//      offsets[e] + the slots of e owned by wavefronts before w;
//   3. each wavefront ranks its slots in order against its own row.
// The rows are the same as the four-launch path's: both place every expert's
// slots in flat-slot order.
constexpr int64_t kSmallPermuteF = 8192;
constexpr int kSmallPermuteExperts = 1024;
constexpr int kSmallPermuteWaves = 16;

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ w, int64_t F,
    int E, int e_begin, int n_local, int nbits, int32_t *__restrict__ row_src,
    int32_t *__restrict__ inv, float *__restrict__ s_perm,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ err) {
  constexpr int NW = kSmallPermuteWaves, G = 8;
  constexpr uint16_t kNone = 0xffff;  // a slot of no local expert
  __shared__ int32_t bins[NW * kSmallPermuteExperts];
  __shared__ uint16_t ev[kSmallPermuteF];
  __shared__ int32_t wtot[NW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per = (int)((F + NW * 64 - 1) / (NW * 64)) * 64;
  const int ngroups = (per / 64 + G - 1) / G;
  const int64_t f0 = (int64_t)wid * per;
  for (int i = tid; i < NW * n_local; i += 1024) bins[i] = 0;
  __syncthreads();
  // 1. this wavefront's slots: local ids into LDS, counts into its row
  int32_t *const mine = bins + wid * n_local;
  int bad = 0;
  // A wavefront owns at most G * 64 slots (one group), so the routing
  // weights are loaded here with the expert ids and kept in registers for
  // step 3: one memory round trip instead of two.
  static_assert(kSmallPermuteF <= (int64_t)NW * 64 * G, "one group per wavefront");
  float wpre[G];
  for (int g = 0; g < ngroups; ++g) {
    int32_t gi[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t f = f0 + (g * G + i) * 64 + lane;
      const bool in = f < f0 + per && f < F;
      gi[i] = in ? idx[f] : 0;
      wpre[i] = (in && s_perm) ? w[f] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t f = f0 + (g * G + i) * 64 + lane;
      if (!(f < f0 + per && f < F)) continue;  // past this wavefront's slots
      bad |= (uint32_t)gi[i] >= (uint32_t)E;
      const uint32_t e = (uint32_t)(gi[i] - e_begin);
      const bool local = e < (uint32_t)n_local;
      ev[f] = local ? (uint16_t)e : kNone;
      if (local) atomicAdd(&mine[e], 1);
    }
  }
  bad = __syncthreads_or(bad);
  // 2. column sums, their exclusive scan over the experts, per-wave bases
  int32_t s = 0;
  if (tid < n_local)
    for (int q = 0; q < NW; ++q) s += bins[q * n_local + tid];
  int32_t x = s;  // inclusive prefix over the wavefront
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t yv = __shfl_up(x, off, 64);
    if (lane >= off) x += yv;
  }
  if (lane == 63) wtot[wid] = x;
  __syncthreads();
  int32_t before = 0, total = 0;
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    const int32_t tq = wtot[q];
    before += q < wid ? tq : 0;
    total += tq;
  }
  if (tid < n_local) {
    int32_t run = before + x - s;  // offsets[tid]
    offsets[tid] = run;
    counts[tid] = s;
    for (int q = 0; q < NW; ++q) {
      const int32_t c = bins[q * n_local + tid];
      bins[q * n_local + tid] = run;
      run += c;
    }
  }
  if (tid == 0) {
    offsets[n_local] = total;
    *err = bad ? kDevErrExpertIndex : 0;
  }
  __syncthreads();
  // 3. stable rows of this wavefront's slots, in order
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int g = 0; g < ngroups; ++g) {
    uint32_t e[G];
    float wv[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int64_t f = f0 + (g * G + i) * 64 + lane;
      const bool in = f < f0 + per && f < F;
      e[i] = in ? (uint32_t)ev[f] : 0xffffffffu;
      wv[i] = (s_perm && e[i] < (uint32_t)n_local) ? wpre[i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if ((g * G + i) * 64 >= per) break;  // uniform
      const int64_t f = f0 + (g * G + i) * 64 + lane;
      const bool local = e[i] < (uint32_t)n_local;
      const int32_t r = rank_step(e[i], local, n_local, nbits, lt_mask, mine);
      if (f < F) inv[f] = r;
      if (local) {
        row_src[r] = (int32_t)f;
        if (s_perm) s_perm[r] = wv[i];
      }
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

hipError_t launch_permute_gather(const void *x, int64_t row_bytes, int64_t k,
                                 const int32_t *row_src, const int32_t *R_ptr,
                                 void *x_perm, int64_t F, int num_cus,
                                 hipStream_t s) {
  int64_t grid = F < (int64_t)num_cus * 8 ? F : (int64_t)num_cus * 8;
  if (grid < 1) grid = 1;
  permute_gather_kernel<<<(unsigned)grid, 256, 0, s>>>(
      (const uint4 *)x, row_bytes / 16, (int)k, row_src, R_ptr,
      (uint4 *)x_perm);
  return hipGetLastError();
}

int permute_chunk(int64_t F, int64_t n_local) {
  (void)F;
  return n_local <= 64 ? 256 : 1024;
}

// counts[0, n) = 0 and offsets[0, n] = 0 (an empty batch).  A kernel rather
// than a memset, so that a caller may capture the call in a graph.
__global__ __launch_bounds__(256) void permute_zero_kernel(int32_t *counts,
                                                           int32_t *offsets,
                                                           int n,
                                                           int32_t *err) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i <= n; i += gridDim.x * 256) {
    if (i < n) counts[i] = 0;
    offsets[i] = 0;
  }
}

hipError_t launch_permute_empty(int32_t *counts, int32_t *offsets,
                                int64_t n_local, void *ws, hipStream_t s) {
  const int64_t blocks = (n_local + 1 + 255) / 256;
  permute_zero_kernel<<<(unsigned)(blocks < 64 ? blocks : 64), 256, 0, s>>>(
      counts, offsets, (int)n_local, (int32_t *)ws);
  return hipGetLastError();
}

// Workspace: the error header, then hist [n_local][nblk], then the chunk
// flags [nblk].
size_t permute_workspace_bytes(int64_t T, int64_t k, int64_t n_local) {
  const int64_t F = T * k;
  const int chunk = permute_chunk(F, n_local);
  const int64_t nblk = F > 0 ? (F + chunk - 1) / chunk : 1;
  return kErrHeaderBytes +
         (size_t)(((nblk * (n_local + 1) * 4) + 255) / 256 * 256);
}

hipError_t launch_permute(const int32_t *idx, const float *w, const void *x,
                          int64_t T, int64_t k, int64_t row_bytes, int64_t E,
                          int64_t e_begin, int64_t n_local, void *x_perm,
                          float *s_perm, int32_t *row_src, int32_t *inv,
                          int32_t *counts, int32_t *offsets, void *ws,
                          int num_cus, hipStream_t s) {
  const int64_t F = T * k;
  const int chunk = permute_chunk(F, n_local);
  const int nblk = (int)((F + chunk - 1) / chunk);
  int32_t *err = (int32_t *)ws;
  int32_t *hist = (int32_t *)((char *)ws + kErrHeaderBytes);
  int32_t *bad_blk = hist + (int64_t)n_local * nblk;
  int nbits = 0;
  while ((1ll << nbits) < n_local) ++nbits;
  if (F <= kSmallPermuteF && n_local <= kSmallPermuteExperts) {
    permute_small_kernel<<<1, 1024, 0, s>>>(
        idx, w, F, (int)E, (int)e_begin, (int)n_local, nbits, row_src, inv,
        (w ? s_perm : nullptr), counts, offsets, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !(x && x_perm)) return e;
    return launch_permute_gather(x, row_bytes, k, row_src, offsets + n_local,
                                 x_perm, F, num_cus, s);
  }
  const size_t lds = (size_t)n_local * 4;
  permute_hist_kernel<<<nblk, 256, lds, s>>>(idx, F, (int)E, (int)e_begin,
                                              (int)n_local, chunk, nblk, hist,
                                              bad_blk);
  permute_scan_kernel<<<1, 1024, 0, s>>>(hist, (int)n_local, nblk, counts,
                                         offsets, bad_blk, err);
  if (chunk == 256)
    permute_scatter_kernel<256><<<nblk, 64, lds, s>>>(
        idx, w, F, (int)e_begin, (int)n_local, nbits, nblk, hist, row_src,
        inv, (w ? s_perm : nullptr));
  else
    permute_scatter_kernel<1024><<<nblk, 64, lds, s>>>(
        idx, w, F, (int)e_begin, (int)n_local, nbits, nblk, hist, row_src,
        inv, (w ? s_perm : nullptr));
  if (x && x_perm)
    return launch_permute_gather(x, row_bytes, k, row_src, offsets + n_local,
                                 x_perm, F, num_cus, s);
  return hipGetLastError();
}

}  // namespace moe
