// CPU oracle for the MoE expert-layer path.  TEST INFRASTRUCTURE ONLY: the
// product path never links, loads or calls this file; only the tests, the
// smoke check and the benchmark's CPU-baseline leg use it.
//
// Plain, slow, obviously correct: fp64 arithmetic, straight loops, no
// blocking or fusion.  It shares no code with the GPU library.  Each function
// names the passage of the pages it follows:
//   [WideEP-Premise]  "Wide-EPとは?" explainer (scholia-notes), section
//                     "前提:MoE(Mixture of Experts)とは": a router picks a few
//                     experts per token, only they compute, and their results
//                     are added up.
//   [WideEP-Problem]  same page, "MoEの課題": which experts are chosen is not
//                     known in advance (so per-expert row counts are data).
//   [WideEP-Comm]     same page, "前提条件:GPU間の高速通信": tokens are sent to
//                     their expert (dispatch) and results returned (combine).
//   [TE-Grouped]      BioNeMo MoE article, "GroupedLinear Optimizes Expert
//                     Computation in MoE Models": per-expert matrices kept,
//                     all experts submitted as one operation; ScaledSwiGLU
//                     folds the routing probabilities into the expert FFN.
//   [TE-MXFP8]        same article, "MXFP8 Precision Reduces Memory Footprint
//                     for Biological Models": 8-bit values with one scale per
//                     block of 32 consecutive values.
//   [WideEP-EPLB]     "Wide-EPとは?" explainer, section 負荷の偏り:EPLB: skewed
//                     expert loads are evened out between forward passes by
//                     moving experts and copying the heaviest ones.
// Where the pages leave a step open, the reading taken is stated at the
// function.  Parity pins for every function live in the CPU test suite.
//
// Data type codes for tensors passed as void*: 0 = fp32, 1 = bf16 (raw
// uint16 bits), 2 = fp64.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

inline double load(const void *p, int dt, int64_t i) {
  if (dt == 0) return (double)((const float *)p)[i];
  if (dt == 1) {
    uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
  }
  return ((const double *)p)[i];
}

inline size_t elem_size(int dt) { return dt == 0 ? 4 : (dt == 1 ? 2 : 8); }

// SiLU(z) = z * sigmoid(z) (Elfwing et al. 2018; the Swish of Ramachandran
// et al. 2017 with beta = 1).
inline double silu(double z) { return z / (1.0 + std::exp(-z)); }

inline double sigmoid(double z) { return 1.0 / (1.0 + std::exp(-z)); }

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
// Router.  [WideEP-Premise]: the router scores every expert for each token.
// logits[t, e] = sum_h x[t, h] * w_r[e, h] + bias[e]   (bias may be NULL)
// x [T, H], w_r [E, H] (K-contiguous), both of type dt; logits [T, E] fp64.
void orc_router_logits(const void *x, const void *w_r, int dt,
                       const float *bias, int64_t T, int64_t H, int64_t E,
                       double *logits) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h)
        acc += load(x, dt, t * H + h) * load(w_r, dt, e * H + h);
      logits[t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
    }
}

// Softmax over all E experts, keep the k most probable, renormalise the kept
// probabilities to sum to one.  [WideEP-Premise] gives "the router picks k of
// E"; the softmax / top-k / renormalise form is the workload definition.
// Softmax is monotone, so the k most probable experts are the k largest
// logits, and the full-softmax denominator cancels in the renormalisation:
//   w_j = exp(l_j - l_max) / sum over kept i of exp(l_i - l_max).
// Readings where the pages are silent:
//   - ties: equal logits are taken lower expert index first; kept experts
//     are listed by descending logit; -0 equals +0;
//   - a NaN logit ranks below every number (-inf included), so a token with
//     fewer than k finite logits still gets k distinct experts;
//   - weights of non-finite logits: with l_max finite, a NaN or -inf logit
//     weighs 0; with l_max = +inf, the +inf logits share the weight equally;
//     with l_max = -inf or NaN (no kept logit above -inf), the k kept
//     experts share it equally.
// logits [T, E] fp32 in; idx [T, k] int32, w [T, k] fp64 out.
namespace {
// a ranks above b
bool logit_above(double a, double b) {
  if (std::isnan(a)) return false;
  if (std::isnan(b)) return true;
  return a > b;
}
}  // namespace

void orc_topk_softmax(const float *logits, int64_t T, int64_t E, int64_t k,
                      int32_t *idx, double *w) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const float *l = logits + t * E;
    std::vector<char> taken(E, 0);
    for (int64_t j = 0; j < k; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || logit_above(l[e], l[best]))) best = e;
      taken[best] = 1;
      idx[t * k + j] = (int32_t)best;
    }
    const double lmax = l[idx[t * k]];
    double kept = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      const double lj = l[idx[t * k + j]];
      double p;
      if (std::isnan(lmax) || lmax == -INFINITY) p = 1.0;
      else if (lmax == INFINITY) p = lj == INFINITY ? 1.0 : 0.0;
      else p = std::isnan(lj) ? 0.0 : std::exp(lj - lmax);
      w[t * k + j] = p;
      kept += p;
    }
    for (int64_t j = 0; j < k; ++j) w[t * k + j] /= kept;
  }
}

// ---------------------------------------------------------------------------
// Dispatch on one GPU.  [WideEP-Comm] sends every (token, chosen expert) slot
// to its expert; [WideEP-Problem] makes the per-expert counts data.  Here the
// slots routed to this GPU's experts [e_begin, e_begin + n_local) are laid
// out expert by expert; inside an expert, slots keep their flat order
// f = t*k + j (a stable counting sort; reading of "stable permute").  Slots
// of other experts are dropped (inv = -1).
//   counts[e]   = number of slots with idx == e_begin + e
//   offsets[e]  = sum of counts before e; offsets[n_local] = R
//   row_src[r]  = flat slot f placed at row r, for r < R
//   inv[f]      = row of slot f, or -1
void orc_permute(const int32_t *idx, int64_t T, int64_t k, int64_t e_begin,
                 int64_t n_local, int32_t *counts, int32_t *offsets,
                 int32_t *row_src, int32_t *inv) {
  const int64_t F = T * k;
  for (int64_t f = 0; f < F; ++f) inv[f] = -1;
  for (int64_t e = 0; e < n_local; ++e) {
    int32_t c = 0;
    for (int64_t f = 0; f < F; ++f)
      if (idx[f] == e_begin + e) ++c;
    counts[e] = c;
  }
  offsets[0] = 0;
  for (int64_t e = 0; e < n_local; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int64_t e = 0; e < n_local; ++e) {
    int32_t r = offsets[e];
    for (int64_t f = 0; f < F; ++f)
      if (idx[f] == e_begin + e) {
        row_src[r] = (int32_t)f;
        inv[f] = r;
        ++r;
      }
  }
}

// x_perm[r, :] = x[row_src[r] / k, :]  (a byte copy of the token's row)
void orc_gather_rows(const void *x, int dt, int64_t H, int64_t k,
                     const int32_t *row_src, int64_t R, void *x_perm) {
  const size_t rb = (size_t)H * elem_size(dt);
  for (int64_t r = 0; r < R; ++r)
    std::memcpy((char *)x_perm + (size_t)r * rb,
                (const char *)x + (size_t)(row_src[r] / k) * rb, rb);
}

// ---------------------------------------------------------------------------
// Expert FFN on listed rows.  [TE-Grouped]: each expert keeps its own
// matrices; ScaledSwiGLU multiplies the routing probability ("scale") into
// the expert FFN.  SwiGLU (Shazeer 2020) with SiLU, no biases:
//   g = W_gate[e] x,  u = W_up[e] x,  a = s * SiLU(g) (.) u,  y = W_down[e] a
// Row n uses activations xs[n, :] (type xdt), local expert ex[n] and scale
// sc[n] (sc may be NULL: scale 1).  W_gate, W_up [n_local, I, H];
// W_down [n_local, H, I] (type wdt).  a_out [n, I] and y_out [n, H] (fp64)
// may each be NULL.
void orc_expert_ffn_rows(const void *xs, int xdt, const int32_t *ex,
                         const double *sc, const void *w_gate,
                         const void *w_up, const void *w_down, int wdt,
                         int64_t nrows, int64_t H, int64_t I, double *a_out,
                         double *y_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < nrows; ++n) {
    const int64_t e = ex[n];
    const double s = sc ? sc[n] : 1.0;
    std::vector<double> x(H), a(I);
    for (int64_t h = 0; h < H; ++h) x[h] = load(xs, xdt, n * H + h);
    for (int64_t i = 0; i < I; ++i) {
      double g = 0.0, u = 0.0;
      const int64_t base = (e * I + i) * H;
      for (int64_t h = 0; h < H; ++h) {
        g += load(w_gate, wdt, base + h) * x[h];
        u += load(w_up, wdt, base + h) * x[h];
      }
      a[i] = s * silu(g) * u;
    }
    if (a_out)
      for (int64_t i = 0; i < I; ++i) a_out[n * I + i] = a[i];
    if (y_out)
      for (int64_t h = 0; h < H; ++h) {
        double acc = 0.0;
        const int64_t base = (e * H + h) * I;
        for (int64_t i = 0; i < I; ++i) acc += load(w_down, wdt, base + i) * a[i];
        y_out[n * H + h] = acc;
      }
  }
}


// ---------------------------------------------------------------------------
// Combine.  [WideEP-Premise]/[WideEP-Comm]: the chosen experts' results come
// back to the token and are added up.
//   out[t, :] = sum_{j ascending, inv[t,j] >= 0} c_tj * y[inv[t,j], :]
// with c_tj = w[t, j] when w is given, else 1 (the scale already went into
// the expert FFN).  Tokens with no local slot get a zero row.
void orc_combine(const double *y, const int32_t *inv, const double *w,
                 int64_t T, int64_t k, int64_t H, double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) out[t * H + h] = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      const int32_t r = inv[t * k + j];
      if (r < 0) continue;
      const double c = w ? w[t * k + j] : 1.0;
      for (int64_t h = 0; h < H; ++h) out[t * H + h] += c * y[(int64_t)r * H + h];
    }
  }
}

// The whole layer by its definition for listed tokens, without any
// permutation ([WideEP-Premise]):
//   out[t] = sum_{j : e_begin <= idx[t,j] < e_begin+n_local}
//            w[t,j] * W_down[e] ( SiLU(W_gate[e] x_t) (.) W_up[e] x_t )
// tokens [ntok] lists token ids; out [ntok, H] fp64.
void orc_moe_tokens(const void *x, int xdt, const int32_t *idx,
                    const double *w, int64_t k, const int32_t *tokens,
                    int64_t ntok, int64_t e_begin, int64_t n_local,
                    const void *w_gate, const void *w_up, const void *w_down,
                    int wdt, int64_t H, int64_t I, double *out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < ntok; ++n) {
    const int64_t t = tokens[n];
    std::vector<double> xv(H), a(I);
    for (int64_t h = 0; h < H; ++h) xv[h] = load(x, xdt, t * H + h);
    for (int64_t h = 0; h < H; ++h) out[n * H + h] = 0.0;
    for (int64_t j = 0; j < k; ++j) {
      const int64_t e = (int64_t)idx[t * k + j] - e_begin;
      if (e < 0 || e >= n_local) continue;
      for (int64_t i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        const int64_t base = (e * I + i) * H;
        for (int64_t h = 0; h < H; ++h) {
          g += load(w_gate, wdt, base + h) * xv[h];
          u += load(w_up, wdt, base + h) * xv[h];
        }
        a[i] = silu(g) * u;
      }
      const double c = w[t * k + j];
      for (int64_t h = 0; h < H; ++h) {
        double acc = 0.0;
        const int64_t base = (e * H + h) * I;
        for (int64_t i = 0; i < I; ++i) acc += load(w_down, wdt, base + i) * a[i];
        out[n * H + h] += c * acc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP8.  [TE-MXFP8]: 8-bit values, one scale per 32 consecutive values.  The
// pages fix no encoding or rounding; the reading taken is the OCP
// Microscaling Formats specification v1.0: elements in FP8 E4M3 (the OCP "FN"
// variant: bias 7, no infinities, 0x7F / 0xFF are NaN, largest finite 448),
// the shared scale in E8M0 (2^(byte-127)), shared exponent
// X = floor(log2(max|v|)) - 8 (8 being E4M3's largest normal exponent),
// elements v / 2^X rounded to nearest, ties to even, saturating at +-448.
// A block whose values are all zero gets scale byte 0 (its codes encode +-0).

// Value of an E4M3 code, by the format's definition.
double orc_e4m3_value(uint8_t code) {
  const int s = code >> 7, ex = (code >> 3) & 15, m = code & 7;
  if (ex == 15 && m == 7) return NAN;
  double mag = ex == 0 ? std::ldexp((double)m / 8.0, -6)
                       : std::ldexp(1.0 + (double)m / 8.0, ex - 7);
  return s ? -mag : mag;
}

// Code of the E4M3 value nearest to v (ties: even code), saturating.
uint8_t orc_e4m3_encode(double v) {
  const double a = std::fabs(v);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {  // every finite non-negative code
    const double err = std::fabs(orc_e4m3_value((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1))) {
      best = c;
      best_err = err;
    }
  }
  if (a > 448.0) best = 0x7E;  // saturate
  // The sign is kept, also when the magnitude rounds to zero (code 0x80).
  return (uint8_t)(best | (std::signbit(v) ? 0x80 : 0));
}

// orc_e4m3_encode of each of n values.
void orc_e4m3_encode_array(const double *v, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

// E5M2, the other OCP FP8 element format, for the gradient option: bias 15,
// exponent field 31 holds the infinities and NaNs, largest finite value
// 1.75 * 2^15 = 57344, subnormals m/4 * 2^-14.  Its wider range suits
// gradients (the pages leave the gradients' element format open; this build
// offers E4M3, the default, and E5M2).  MX shared exponent with E5M2
// elements: X = floor(log2(max|v|)) - 15 (15 being E5M2's largest normal
// exponent); elements v / 2^X rounded to nearest, ties to even, saturating at
// +-57344.

// Value of an E5M2 code, by the format's definition.
double orc_e5m2_value(uint8_t code) {
  const int s = code >> 7, ex = (code >> 2) & 31, m = code & 3;
  double mag;
  if (ex == 31) mag = m == 0 ? INFINITY : NAN;
  else if (ex == 0) mag = std::ldexp((double)m / 4.0, -14);
  else mag = std::ldexp(1.0 + (double)m / 4.0, ex - 15);
  return s ? -mag : mag;
}

// Code of the E5M2 value nearest to v (ties: even code), saturating at the
// largest finite value.
uint8_t orc_e5m2_encode(double v) {
  const double a = std::fabs(v);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7B; ++c) {  // every finite non-negative code
    const double err = std::fabs(orc_e5m2_value((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1))) {
      best = c;
      best_err = err;
    }
  }
  if (a > 57344.0) best = 0x7B;  // saturate
  return (uint8_t)(best | (std::signbit(v) ? 0x80 : 0));
}

void orc_e5m2_encode_array(const double *v, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_encode(v[i]);
}

// Element formats of an MX block: 0 = E4M3, 1 = E5M2.
static int elem_emax(int fmt) { return fmt == 1 ? 15 : 8; }
static uint8_t elem_encode(int fmt, double v) {
  return fmt == 1 ? orc_e5m2_encode(v) : orc_e4m3_encode(v);
}
static double elem_value(int fmt, uint8_t c) {
  return fmt == 1 ? orc_e5m2_value(c) : orc_e4m3_value(c);
}

// Shared E8M0 scale byte of a block with largest magnitude amax and elements
// of format fmt: X = floor(log2 amax) - emax, clamped to [-127, 127].
uint8_t orc_mx_scale_byte_fmt(double amax, int fmt) {
  if (amax == 0.0) return 0;
  int e2;
  std::frexp(amax, &e2);  // amax = m * 2^e2, m in [0.5, 1)
  int X = (e2 - 1) - elem_emax(fmt);
  if (X < -127) X = -127;
  if (X > 127) X = 127;
  return (uint8_t)(X + 127);
}

uint8_t orc_mx_scale_byte(double amax) { return orc_mx_scale_byte_fmt(amax, 0); }

// Quantise each row of v [rows, cols] in blocks of 32 along the row (the last
// block of a row may be shorter: it behaves as if zero-padded), elements of
// format fmt.  codes [rows, cols]; scales [rows, ceil(cols/32)].
void orc_mx_quantize_rows_fmt(const double *v, int64_t rows, int64_t cols,
                              int fmt, uint8_t *codes, uint8_t *scales) {
  const int64_t nb = (cols + 31) / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t c0 = b * 32, c1 = std::min<int64_t>(cols, c0 + 32);
      double amax = 0.0;
      for (int64_t c = c0; c < c1; ++c) amax = std::fmax(amax, std::fabs(v[r * cols + c]));
      const uint8_t sb = orc_mx_scale_byte_fmt(amax, fmt);
      scales[r * nb + b] = sb;
      const double inv_scale = std::ldexp(1.0, -((int)sb - 127));
      for (int64_t c = c0; c < c1; ++c)
        codes[r * cols + c] = elem_encode(fmt, v[r * cols + c] * inv_scale);
    }
}

void orc_mx_quantize_rows(const double *v, int64_t rows, int64_t cols,
                          uint8_t *codes, uint8_t *scales) {
  orc_mx_quantize_rows_fmt(v, rows, cols, 0, codes, scales);
}

// v[r, c] = value(codes[r, c]) * 2^(scales[r, c/32] - 127), exactly, in fp64.
void orc_mx_dequantize_rows_fmt(const uint8_t *codes, const uint8_t *scales,
                                int64_t rows, int64_t cols, int fmt,
                                double *v) {
  const int64_t nb = (cols + 31) / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      v[r * cols + c] = std::ldexp(elem_value(fmt, codes[r * cols + c]),
                                   (int)scales[r * nb + c / 32] - 127);
}

void orc_mx_dequantize_rows(const uint8_t *codes, const uint8_t *scales,
                            int64_t rows, int64_t cols, double *v) {
  orc_mx_dequantize_rows_fmt(codes, scales, rows, cols, 0, v);
}

// ---------------------------------------------------------------------------
// bfloat16 storage of a value: 8 significant bits (1 implicit + 7 stored),
// 8 exponent bits like fp32.  [TE-MXFP8]: the tensors handed from one
// operation to the next stay in BF16; only the GEMM inputs are MX-quantised.
// Nearest bf16 value, ties to the even significand; values below bf16's
// normal range use its subnormal spacing 2^-133.  Inputs are finite and
// below bf16's largest finite value.
void orc_round_bf16(const double *v, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) {
    const double a = std::fabs(v[i]);
    if (a == 0.0) { out[i] = v[i]; continue; }
    int e2;
    std::frexp(a, &e2);                    // a in [2^(e2-1), 2^e2)
    const int e = std::max(e2 - 1, -126);  // exponent of the binade
    const double ulp = std::ldexp(1.0, e - 7);
    const double q = a / ulp;              // exact: power-of-two division
    double lo = std::floor(q);
    const double frac = q - lo;
    if (frac > 0.5 || (frac == 0.5 && std::fmod(lo, 2.0) == 1.0)) lo += 1.0;
    const double r = lo * ulp;
    out[i] = std::signbit(v[i]) ? -r : r;
  }
}

// ---------------------------------------------------------------------------
// Plain fp64 products used by the MXFP8 training step (the GEMMs of the
// backward pass follow the chain rule on the forward above).
// C[m, n] = sum_k A[m, k] * B[n, k]    (A [M, K], B [N, K], C [M, N])
void orc_matmul_nt(const double *A, const double *B, int64_t M, int64_t N,
                   int64_t K, double *C) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t kk = 0; kk < K; ++kk) acc += A[m * K + kk] * B[n * K + kk];
      C[m * N + n] = acc;
    }
}

// ScaledSwiGLU of given pre-activations ([TE-Grouped]; SwiGLU per Shazeer
// 2020 with the routing scale folded in): a = s * SiLU(g) * u, g, u [rows, I],
// s [rows] (NULL: 1).
void orc_swiglu_rows(const double *g, const double *u, const double *s,
                     int64_t rows, int64_t I, double *a) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < I; ++i) {
      const int64_t o = r * I + i;
      a[o] = (s ? s[r] : 1.0) * silu(g[o]) * u[o];
    }
}

// SwiGLU-with-scale backward, by the chain rule on a = s * SiLU(g) * u:
//   dg = da * s * u * SiLU'(g),  du = da * s * SiLU(g),
//   ds = sum_i da * SiLU(g) * u,
// with SiLU'(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z))).
void orc_swiglu_bwd_rows(const double *da, const double *g, const double *u,
                         const double *s, int64_t rows, int64_t I, double *dg,
                         double *du, double *ds) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int64_t i = 0; i < I; ++i) {
      const int64_t o = r * I + i;
      const double z = g[o], sg = sigmoid(z);
      const double sl = z * sg;
      const double dsl = sg * (1.0 + z * (1.0 - sg));
      dg[o] = da[o] * s[r] * u[o] * dsl;
      du[o] = da[o] * s[r] * sl;
      acc += da[o] * sl * u[o];
    }
    ds[r] = acc;
  }
}



// ---------------------------------------------------------------------------
// Expert-parallel load balancing.  [WideEP-EPLB] "Wide-EPとは?" explainer,
// section 負荷の偏り:EPLB: how often each expert is chosen is skewed; when
// frequently chosen experts sit on one GPU it becomes the bottleneck while
// the others idle; between forward passes the balancer looks at each
// expert's load and rearranges the placement, and gives the heaviest
// experts copies on several GPUs.  The pages give no algorithm; the plain
// reading taken here.  The plan is made from observed loads (the per-expert
// counts of earlier routing):
//   1. replication: S physical slots for E experts (S >= E); every expert
//      gets one slot, and each of the S - E spare slots goes, one at a time,
//      to the expert with the largest load per copy (n_e / r_e; ties: lower
//      expert index);
//   2. the expected rows of copy i of expert e are those of the split in
//      (dispatch, below) applied to the observed n_e;
//   3. placement: G ranks of S / G slots each; copies are placed in order of
//      decreasing expected rows (ties: lower expert, then lower copy), each
//      on the rank with the smallest expected load so far among those with
//      a free slot that do not yet hold the expert (if every rank with a
//      free slot holds it: among those with a free slot; ties: lower rank);
//   4. physical slot numbers: rank g owns slots [g S/G, (g+1) S/G), in
//      increasing (expert, copy) order.
// counts [E] in; out: rep [E] copies per expert, rep_first [E + 1] prefix of
// rep, rep_slot [S] physical slot of copy i of expert e at rep_first[e] + i,
// slot_expert / slot_copy [S] expert and copy index of each slot.
void orc_eplb_plan(const int32_t *counts, int64_t E, int64_t S, int64_t G,
                   int32_t *rep, int32_t *rep_first, int32_t *rep_slot,
                   int32_t *slot_expert, int32_t *slot_copy) {
  for (int64_t e = 0; e < E; ++e) rep[e] = 1;
  for (int64_t extra = 0; extra < S - E; ++extra) {
    int64_t best = 0;
    for (int64_t e = 1; e < E; ++e)
      // n_e / r_e > n_best / r_best, compared exactly
      if ((int64_t)counts[e] * rep[best] > (int64_t)counts[best] * rep[e])
        best = e;
    ++rep[best];
  }
  rep_first[0] = 0;
  for (int64_t e = 0; e < E; ++e) rep_first[e + 1] = rep_first[e] + rep[e];
  struct Copy { int32_t e, i; int64_t rows; };
  std::vector<Copy> cp;
  for (int64_t e = 0; e < E; ++e)
    for (int32_t i = 0; i < rep[e]; ++i) {
      const int64_t n = counts[e], r = rep[e];
      cp.push_back({(int32_t)e, i, (i + 1) * n / r - i * n / r});
    }
  std::stable_sort(cp.begin(), cp.end(), [](const Copy &a, const Copy &b) {
    return a.rows > b.rows;
  });
  const int64_t per = S / G;
  std::vector<int64_t> load(G, 0), used(G, 0);
  std::vector<std::vector<char>> holds(G, std::vector<char>(E, 0));
  std::vector<int32_t> rank_of(S);   // by copy index rep_first[e] + i
  for (const Copy &c : cp) {
    int64_t pick = -1;
    for (int pass = 0; pass < 2 && pick < 0; ++pass)
      for (int64_t g = 0; g < G; ++g) {
        if (used[g] == per || (pass == 0 && holds[g][c.e])) continue;
        if (pick < 0 || load[g] < load[pick]) pick = g;
      }
    load[pick] += c.rows;
    ++used[pick];
    holds[pick][c.e] = 1;
    rank_of[rep_first[c.e] + c.i] = (int32_t)pick;
  }
  std::vector<int64_t> next(G);
  for (int64_t g = 0; g < G; ++g) next[g] = g * per;
  for (int64_t e = 0; e < E; ++e)
    for (int32_t i = 0; i < rep[e]; ++i) {
      const int64_t q = rep_first[e] + i;
      const int64_t s = next[rank_of[q]]++;
      rep_slot[q] = (int32_t)s;
      slot_expert[s] = (int32_t)e;
      slot_copy[s] = i;
    }
}

// Dispatch to this rank's slots [s_begin, s_begin + n_slots) under a plan
// (the current routing, not the loads the plan was made from): with n_e the
// number of current entries of expert e, copy i of e takes the entries at
// positions [floor(i n_e / r_e), floor((i+1) n_e / r_e)) among e's entries
// in ascending flat order f = t*k + j (contiguous ranges, as even as
// possible); inside a slot, entries keep ascending f.  Entries of other
// ranks' slots and indices outside [0, E) are dropped (inv = -1).  Outputs
// as orc_permute over the local slots: counts [n_slots], offsets
// [n_slots + 1], row_src, inv.
void orc_permute_replicated(const int32_t *idx, int64_t T, int64_t k,
                            int64_t E, const int32_t *rep_first,
                            const int32_t *rep_slot, int64_t s_begin,
                            int64_t n_slots, int32_t *counts, int32_t *offsets,
                            int32_t *row_src, int32_t *inv) {
  const int64_t F = T * k;
  std::vector<int64_t> n(E, 0), seen(E, 0);
  for (int64_t f = 0; f < F; ++f)
    if (idx[f] >= 0 && idx[f] < E) ++n[idx[f]];
  std::vector<int64_t> slot_of(F, -1);
  for (int64_t f = 0; f < F; ++f) {
    inv[f] = -1;
    const int32_t e = idx[f];
    if (e < 0 || e >= E) continue;
    const int64_t q = seen[e]++;
    const int64_t r = rep_first[e + 1] - rep_first[e];
    for (int64_t i = 0; i < r; ++i)
      if (i * n[e] / r <= q && q < (i + 1) * n[e] / r)
        slot_of[f] = rep_slot[rep_first[e] + i];
  }
  for (int64_t s = 0; s < n_slots; ++s) {
    int32_t c = 0;
    for (int64_t f = 0; f < F; ++f)
      if (slot_of[f] == s_begin + s) ++c;
    counts[s] = c;
  }
  offsets[0] = 0;
  for (int64_t s = 0; s < n_slots; ++s) offsets[s + 1] = offsets[s] + counts[s];
  for (int64_t s = 0; s < n_slots; ++s) {
    int32_t r = offsets[s];
    for (int64_t f = 0; f < F; ++f)
      if (slot_of[f] == s_begin + s) {
        row_src[r] = (int32_t)f;
        inv[f] = r;
        ++r;
      }
  }
}

}  // extern "C"
