// Host computation of the codebooks' levels and encoder thresholds: NF4, and the
// FP4 (E2M1) and Int4 tables the pages compare it with.
//
// Procedure ("QLoRA: Efficient Finetuning of Quantized LLMs", section
// "NormalFloat: 4 bits for a bell curve", the code-point listing): take
// standard-normal quantiles at 9 probabilities evenly spaced from the offset
// 0.9677083 down to 1/2 and keep the first 8 (positive levels); take 8 such
// points for the negative side, keep the first 7 and negate; add an exact zero;
// sort; divide by the largest magnitude so the ends are exactly -1 and +1.
//
// The quantile function is this file's own: Newton's method on the upper tail
// Q(x) = erfc(x / sqrt 2) / 2 = 1 - p, started at x = 0.  Q is convex and
// decreasing for x >= 0 and every probability used is in (1/2, 1), so the
// iterates increase monotonically to the root.  The probabilities are formed the
// way an evenly spaced grid is usually formed, start + i * step with
// step = (stop - start) / (num - 1), in float64.
//
// Built with -ffp-contract=off so no multiply-add is fused.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "common.h"

namespace qlora {

namespace {

constexpr double kOffset = 0.9677083;

double upper_tail_quantile(double q /* = 1 - p, in (0, 1/2) */) {
  const double inv_sqrt2 = 0.70710678118654752440;
  const double inv_sqrt_2pi = 0.39894228040143267794;
  double x = 0.0;
  for (int it = 0; it < 200; ++it) {
    double tail = 0.5 * std::erfc(x * inv_sqrt2);
    double dens = inv_sqrt_2pi * std::exp(-0.5 * x * x);
    double step = (tail - q) / dens;
    double nx = x + step;
    if (!(nx > x)) break;   // converged: no further increase representable
    x = nx;
  }
  return x;
}

double quantile(double p) { return upper_tail_quantile(1.0 - p); }

float round_down_f32(double v) {
  float f = (float)v;
  if ((double)f > v) f = std::nextafterf(f, -INFINITY);
  return f;
}

struct Codebook {
  float level[16];
  float thr[15];
  void finish(const double* v) {
    for (int i = 0; i < 16; ++i) level[i] = (float)v[i];
    for (int k = 0; k < 15; ++k) thr[k] = round_down_f32(((double)level[k] + (double)level[k + 1]) * 0.5);
  }
  // 4-bit float, 2 exponent bits (bias 1) and 1 mantissa bit: magnitudes m/2 (exponent 0)
  // and 2^(e-1) (1 + m/2), i.e. 0, 0.5, 1, 1.5, 2, 3, 4, 6; divided by the largest (6).
  // Index 0 is the unused entry -4/3 (the next E2M1-like step beyond the range).
  static Codebook fp4() {
    double mag[8];
    for (int c = 0; c < 8; ++c) {
      const int e = c >> 1, m = c & 1;
      mag[c] = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
    }
    double v[16];
    v[0] = -8.0 / 6.0;
    for (int i = 0; i < 7; ++i) v[1 + i] = -mag[7 - i] / 6.0;   // -1 .. -1/12
    for (int i = 0; i < 8; ++i) v[8 + i] = mag[i] / 6.0;        // 0 .. 1
    Codebook cb;
    cb.finish(v);
    return cb;
  }
  // symmetric int4: k / 7, k = -8..7; index 0 (-8/7) is never the nearest level in [-1, 1]
  static Codebook int4() {
    double v[16];
    for (int i = 0; i < 16; ++i) v[i] = (double)(i - 8) / 7.0;
    Codebook cb;
    cb.finish(v);
    return cb;
  }
  Codebook() = default;
  static Codebook nf4() {
    double v[16];
    int n = 0;
    const double step_pos = (0.5 - kOffset) / 8.0;   // 9 points, last (1/2) dropped
    for (int i = 0; i < 8; ++i) v[n++] = quantile((double)i * step_pos + kOffset);
    const double step_neg = (0.5 - kOffset) / 7.0;   // 8 points, last dropped
    for (int i = 0; i < 7; ++i) v[n++] = -quantile((double)i * step_neg + kOffset);
    v[n++] = 0.0;
    // sort ascending (insertion sort, 16 values)
    for (int i = 1; i < 16; ++i) {
      double key = v[i];
      int j = i - 1;
      while (j >= 0 && v[j] > key) { v[j + 1] = v[j]; --j; }
      v[j + 1] = key;
    }
    double mx = 0.0;
    for (int i = 0; i < 16; ++i) mx = std::fmax(mx, std::fabs(v[i]));
    for (int i = 0; i < 16; ++i) v[i] = v[i] / mx;
    Codebook cb;
    cb.finish(v);
    return cb;
  }
};

}  // namespace

static const Codebook& codebook(int which) {
  // computed once; thread-safe initialization
  static const Codebook tables[3] = {Codebook::nf4(), Codebook::fp4(), Codebook::int4()};
  return tables[which];
}

const float* codebook_levels_host(int which) { return codebook(which).level; }

const float* codebook_thresholds_host(int which) { return codebook(which).thr; }

// Order-preserving map between fp32 values and 32-bit keys (-0 and +0 adjacent).
static uint32_t okey(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
static float ofloat(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// For every bin b: lo = the smallest fp32 value whose bin is b (lut_bin is non-decreasing),
// hi = the largest.  A threshold below lo is below every value of the bin, one at or above
// hi is above or equal to every value of it; at most one threshold may lie in [lo, hi).
static ThrLut make_lut(const float* thr) {
  ThrLut L;
  const uint32_t kmin = okey(-INFINITY), kmax = okey(INFINITY);
  uint32_t first[kLutBins + 1];   // first key whose bin is >= b
  for (int b = 0; b <= kLutBins; ++b) {
    if (b == 0) { first[b] = kmin; continue; }
    if (b == kLutBins) { first[b] = kmax + 1u; continue; }
    uint32_t lo = kmin, hi = kmax;   // lut_bin(ofloat(hi)) >= b > lut_bin(ofloat(kmin)) = 0
    while (lo + 1u < hi) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      if (lut_bin(ofloat(mid)) >= b) hi = mid; else lo = mid;
    }
    first[b] = hi;
  }
  for (int b = 0; b < kLutBins; ++b) {
    const uint32_t klo = first[b], khi = first[b + 1] - 1u;   // keys of the bin's values
    int below = 0, inside = 0;
    float t = INFINITY;
    for (int k = 0; k < 15; ++k) {
      const uint32_t kt = okey(thr[k]);
      if (kt < klo) ++below;
      else if (kt < khi) { ++inside; t = thr[k]; }
    }
    if (inside > 1) std::abort();   // never for the three tables: thresholds are >= 0.08 apart
    L.t[b] = t;
    L.base[b] = (uint32_t)below;
  }
  return L;
}

const ThrLut& thr_lut_host(int which) {
  static const ThrLut luts[3] = {make_lut(codebook(0).thr), make_lut(codebook(1).thr), make_lut(codebook(2).thr)};
  return luts[which];
}

const float* nf4_levels_host() { return codebook(0).level; }

const float* nf4_thresholds_host() { return codebook(0).thr; }

}  // namespace qlora
