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
// fp32 -> bf16 bits, round to nearest even (the hardware conversion,
// v_cvt_pk_bf16_f32, in the default round-to-nearest-even mode).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 1 / (1 + e^-z) with the hardware reciprocal (1 ulp).
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// SiLU(z) = z * sigmoid(z)
__device__ __forceinline__ float silu_f32(float z) {
  return z * sigmoid_f32(z);
}

// Rows [b, e) of segment g of a device offsets array, clamped to [0, cap]:
// a segment running past the row capacity is cut there, a decreasing one is
// empty (the plan kernels report both in the error word).
__device__ __forceinline__ void seg_rows(const int32_t *offsets, int g,
                                         int cap, int &b, int &e) {
  b = min(max(offsets[g], 0), cap);
  e = min(max(offsets[g + 1], b), cap);
}

// Whether segment g of `offsets` breaks 0 <= offsets[g] <= offsets[g+1] <= cap.
__device__ __forceinline__ bool seg_bad(const int32_t *offsets, int g,
                                        int cap) {
  const int32_t b = offsets[g], e = offsets[g + 1];
  return b < 0 || e < b || e > cap;
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

// ---- hand-over between workgroups ----------------------------------------
// On gfx950 each XCD has its own L2, and device-scope fences write back or
// invalidate a whole L2.  Data one workgroup hands to another (possibly on
// another XCD) within a kernel goes instead through relaxed device-scope
// atomic stores and loads, which the hardware serves at the device's
// coherence point; s_waitcnt vmcnt(0) orders the stores before the signal
// (a flag or a counter) that publishes them.

__device__ __forceinline__ uint64_t load_coherent8(const void *p) {
  return __hip_atomic_load((uint64_t *)p, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent8(void *p, uint64_t v) {
  __hip_atomic_store((uint64_t *)p, v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes (8 bf16) through two coherent 8-byte loads.
__device__ __forceinline__ bf16x8 load_coherent16(const uint16_t *p) {
  uint64_t v[2] = {load_coherent8(p), load_coherent8(p + 4)};
  bf16x8 r;
  __builtin_memcpy(&r, v, 16);
  return r;
}

__device__ __forceinline__ void store_coherent16(uint16_t *p, uint32_t w0,
                                                 uint32_t w1, uint32_t w2,
                                                 uint32_t w3) {
  store_coherent8(p, (uint64_t)w0 | ((uint64_t)w1 << 32));
  store_coherent8(p + 4, (uint64_t)w2 | ((uint64_t)w3 << 32));
}

// Wait for this wavefront's vector-memory operations (stores included): the
// ordering point between coherent stores and the signal that publishes them.
__device__ __forceinline__ void wait_vmem() {
  // vmcnt 0; expcnt and lgkmcnt at their maxima (not waited for)
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
}

// ---- staged epilogues ----------------------------------------------------
// After a GEMM's K loop its LDS ring is free; each wavefront stages its part
// of the output in a region of its own ([NROWS][W] bf16) and writes it back
// to HBM as 16-byte row pieces instead of 2-byte stores per lane.
// Staged regions swizzle columns by bit 2 of the row: the two halves of a
// wavefront write rows i and i + 4 of one 32x32 block at once, which would
// otherwise fall on the same banks.  The XOR moves whole 8-column chunks,
// so 16-byte row pieces stay contiguous.
template <int W>
__device__ __forceinline__ int st_col(int row, int col) {
  constexpr int X = W >= 64 ? 32 : W / 2;   // a multiple of 8 below W
  return col ^ (((row >> 2) & 1) * X);
}

// Write rows [0, nrows) of a staged [nrows][W] bf16 region to
// dst[(grow0 + r) * ld + col0 + c] for tile rows arow0 + r < rows and
// columns col0 + c < N (N % 8 == 0).
template <int W, int NROWS>
__device__ __forceinline__ void store_staged(const uint16_t *l, uint16_t *dst,
                                                int64_t ld, int64_t col0, int N,
                                                int64_t grow0, int arow0,
                                                int rows, int lane) {
  constexpr int LPR = W / 8;                 // lanes per row
  constexpr int RPI = 64 / LPR;              // rows per instruction
#pragma unroll
  for (int it = 0; it < NROWS / RPI; ++it) {
    const int r = it * RPI + lane / LPR;
    const int c8 = (lane % LPR) * 8;
    if (arow0 + r < rows && col0 + c8 < N)
      *(uint4 *)(dst + (grow0 + r) * ld + col0 + c8) =
          *(const uint4 *)(l + r * W + st_col<W>(r, c8));
  }
}

// store_staged for data that other workgroups of the same launch read:
// every 16-byte piece leaves through device-coherent stores (see
// store_coherent16); the caller waits for them (wait_vmem) before it
// signals.
template <int W, int NROWS>
__device__ __forceinline__ void store_staged_coherent(const uint16_t *l,
                                                      uint16_t *dst, int64_t ld,
                                                      int64_t col0, int N,
                                                      int64_t grow0, int arow0,
                                                      int rows, int lane) {
  constexpr int LPR = W / 8;                 // lanes per row
  constexpr int RPI = 64 / LPR;              // rows per instruction
#pragma unroll
  for (int it = 0; it < NROWS / RPI; ++it) {
    const int r = it * RPI + lane / LPR;
    const int c8 = (lane % LPR) * 8;
    if (arow0 + r < rows && col0 + c8 < N) {
      const uint4 v = *(const uint4 *)(l + r * W + st_col<W>(r, c8));
      store_coherent16(dst + (grow0 + r) * ld + col0 + c8, v.x, v.y, v.z, v.w);
    }
  }
}

// Tile of workgroup `bid` when every tile has its own workgroup and the
// grid is launched for an upper bound of `total` (the real count lives on
// the device).  Workgroups are handed to the 8 XCDs round-robin by id and,
// on one XCD, in id order; XCD x gets the contiguous range [x*per,
// (x+1)*per), so neighbouring tiles (which share operands) run at the same
// time behind one L2.  Returns -1 for a workgroup without a tile.
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int per = (total + 7) >> 3;
  const int j = bid >> 3;
  if (j >= per) return -1;
  const int t = (bid & 7) * per + j;
  return t < total ? t : -1;
}

// (m-tile, n-tile) of tile `local` among one group's mtiles x NT tiles, in
// bands of GM m-tiles: inside a band the m-tile runs fastest, so a run of
// consecutive tiles covers a GM x (run / GM) block and re-reads neither
// operand from HBM.
__device__ __forceinline__ void banded_mn(int local, int mtiles, int NT,
                                          int GM, int &mt, int &nt) {
  const int band = local / (GM * NT);
  const int first = band * GM;
  const int gm = min(GM, mtiles - first);
  const int r = local - band * GM * NT;
  mt = first + r % gm;
  nt = r / gm;
}

// Workgroups to launch for at most `max_tiles` tiles (see xcd_tile).
inline int64_t tile_grid(int64_t max_tiles) {
  int64_t g = (max_tiles + 7) / 8 * 8;
  return g < 8 ? 8 : g;
}

}  // namespace moe
