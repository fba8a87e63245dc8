/*
 * Seeded synthetic inputs for the sparse MoE layer (shared by the GPU path's tests/bench and the
 * CPU oracle). This module holds no arithmetic of the MoE method itself: it only draws numbers.
 *
 * Generator (counter-based, so the bytes do not depend on thread count or call order):
 *   element i of a tensor with seed s hashes the 64-bit key (s << 40) | i with SplitMix64
 *   (Steele, Lea, Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014), takes the
 *   top 53 bits as an open-interval uniform U = (h + 0.5) * 2^-53 in (0, 1), and maps it to a normal
 *   deviate by the inverse normal CDF, evaluated with P. J. Acklam's rational approximation
 *   (relative error below 1.2e-9, far under fp32 rounding). The deviate is computed in double,
 *   scaled by sigma and rounded to fp32 (round-to-nearest-even). bf16 outputs round that fp32 value
 *   to bf16 (round-to-nearest-even on the bit pattern).
 *
 * Element indices are global within a tensor, so a caller may generate any sub-range
 * [first, first + n) of a large tensor (e.g. one expert's weights at a time) and get the same
 * bytes as a whole-tensor draw.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline double uniform_open01(uint64_t seed, uint64_t i) {
  uint64_t key = (seed << 40) | i;
  return ((double)(splitmix64(key) >> 11) + 0.5) * 0x1.0p-53;
}

/* Inverse of the standard normal CDF (Acklam's rational approximation: a central rational
 * function for p in [0.02425, 0.97575], a tail rational function in sqrt(-2 ln p) outside). */
static inline double inv_norm_cdf(double p) {
  static const double a[6] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                              1.383577518672690e+02,  -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[5] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                              6.680131188771972e+01,  -1.328068155288572e+01};
  static const double c[6] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                              -2.549732539343734e+00, 4.374664141464968e+00,  2.938163982698783e+00};
  static const double d[4] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                              3.754408661907416e+00};
  const double p_low = 0.02425;
  if (p < p_low) {
    double q = sqrt(-2.0 * log(p));
    return (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  }
  if (p > 1.0 - p_low) {
    double q = sqrt(-2.0 * log(1.0 - p));
    return -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  }
  double q = p - 0.5, r = q * q;
  return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
         (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
}

static inline float normal_f32(uint64_t seed, uint64_t i, double sigma) {
  return (float)(inv_norm_cdf(uniform_open01(seed, i)) * sigma);
}

static inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  /* finite inputs only (normal deviates never overflow) */
  uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

/* out[j] = sigma * N(0,1) for element indices first + j, j in [0, n). */
void synth_normal_f32(uint64_t seed, uint64_t first, uint64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = normal_f32(seed, first + (uint64_t)j, sigma);
}

/* Same draw, rounded once more to bf16 (bit patterns). */
void synth_normal_bf16(uint64_t seed, uint64_t first, uint64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = f32_to_bf16_rne(normal_f32(seed, first + (uint64_t)j, sigma));
}

/* Router logits with a Zipf-like per-expert skew: logits[t][e] = N(0,1) + b_e,
 * b_e = scale * ln(1/(e+1)) computed in double, rounded to fp32, added in fp32. */
void synth_skewed_logits(uint64_t seed, uint64_t T, uint64_t E, double scale, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < (int64_t)T; ++t) {
    for (uint64_t e = 0; e < E; ++e) {
      float b = (float)(scale * log(1.0 / (double)(e + 1)));
      uint64_t i = (uint64_t)t * E + e;
      out[i] = normal_f32(seed, i, 1.0) + b;
    }
  }
}

/* fp32 -> bf16 bit patterns (round to nearest even), for callers that build bf16 inputs from their
 * own fp32 values. */
void synth_f32_to_bf16(const float* in, uint64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = f32_to_bf16_rne(in[j]);
}
