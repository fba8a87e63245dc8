/*
 * CPU oracle for the sparse mixture-of-experts experts forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's CPU
 * baseline leg may load this library. The GPU library never calls it and shares no code with it.
 *
 * It is a plain, slow, obviously correct restatement of what the layer computes, accumulating in
 * double (fp64). Sources (web pages; "p1".."p5" are the five pages this project is built from):
 *   p1  Transformers docs, "Experts backends" (experts_interface), intro: every MoE backend computes
 *       the same function - per token the router picks k experts, the hidden state is projected
 *       through those experts' parameters and the results are combined with the routing weights;
 *       the "eager" row of the backends table iterates the selected experts.
 *       Backends table rows "deepgemm_megamoe"/"sonicmoe": the expert is a gated MLP (up/gate
 *       projection, SwiGLU, down projection).
 *   p2  Transformers docs, "Fine-grained FP8" (finegrained_fp8), intro bullets: weights quantised to
 *       8 bits per 2-D block of 128x128; activations to 8 bits per group of 128 input channels per
 *       token, with dynamic (per-row, computed at run time) scales.
 *   p4  lira-now "Mixture of Experts" explainer, section 5 (router step by step): logits -> softmax
 *       -> top-k -> renormalise the selected probabilities -> weighted sum of the selected experts'
 *       outputs (its pseudocode block restates the same steps).
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   - top-k is taken on the logits (softmax is strictly increasing, so it is the same set), ordered
 *     by descending logit with ties going to the lower expert index;
 *   - renormalised weights w_j = exp(l_j - l_max) / sum_{j' in top-k} exp(l_j' - l_max): the full
 *     softmax denominator cancels; no epsilon;
 *   - SwiGLU expert y = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + exp(-z)), no biases;
 *   - fp8: OCP E4M3FN (max 448), absmax scaling s = amax / 448 in fp32 (s = 1 for an all-zero
 *     group), code = round-to-nearest-even(v / s) with fp32 division, saturating at +-448; the
 *     expert hidden activation h is quantised by the same per-token 128-group rule before the down
 *     projection;
 *   - the stable permutation orders (token, slot) pairs by expert, and by flat index t*k + j within
 *     an expert;
 *   - UE8M0 scale format (p2, section "UE8M0 scale format"; its note on Blackwell): every block
 *     scale is a power of two stored as one float8_e8m0fnu byte b (value 2^(b-127)). The pages give
 *     no rule for choosing it; here the scale of a group is the smallest power of two 2^e with
 *     448 * 2^e >= amax (so no code saturates; e = 0 for an all-zero group), for weight blocks and
 *     for the dynamic activation groups alike, and codes are E4M3(v * 2^-e), an exact scaling;
 *   - FP4 expert weights (p1 backends notes and p2 "UE8M0 scale format": FP4 experts packed two per
 *     int8 with UE8M0 weight scales; no block size is given): OCP E2M1 (1 sign, 2 exponent bits,
 *     bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), element 2j in the low nibble of byte j,
 *     one UE8M0 scale per 32 consecutive input channels of a row (the MX block), chosen as the
 *     smallest power of two 2^e with 6 * 2^e >= amax, codes E2M1(v * 2^-e) to nearest, ties to
 *     the even code; activations keep the fp8 rule with UE8M0 scales.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_E4M3 = 2, ORACLE_E2M1 = 3 };

/* ---------------------------------------------------------------------------------------------
 * Number formats
 * ------------------------------------------------------------------------------------------- */

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 encodes
 * subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity; the largest finite value is
 * 1.75 * 2^8 = 448. */
double oracle_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int ex = (code >> 3) & 0xF;
  int man = code & 0x7;
  double v;
  if (ex == 0xF && man == 0x7) return NAN;
  if (ex == 0)
    v = ldexp((double)man, -9);
  else
    v = ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -v : v;
}

/* Nearest E4M3FN code to v (ties to the even code), with |v| beyond 448 saturating to 448.
 * The non-negative finite codes 0x00..0x7E are increasing in value, so a binary search finds the
 * bracketing pair and the nearer one is taken. */
uint8_t oracle_e4m3_encode(float v) {
  double a = fabs((double)v);
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 0x7E; /* invariant: value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_value((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - oracle_e4m3_value((uint8_t)lo);
  double dhi = oracle_e4m3_value((uint8_t)hi) - a;
  int code;
  if (dlo < dhi)
    code = lo;
  else if (dhi < dlo)
    code = hi;
  else
    code = (lo % 2 == 0) ? lo : hi; /* tie: even mantissa */
  return sign | (uint8_t)code; /* values that round to zero keep their sign (-0 is 0x80) */
}

/* OCP E2M1 (FP4): code bits s e e m; exponent field 0 encodes 0 and 0.5 (m * 0.5), otherwise
 * 2^(e-1) * (1 + m/2): 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_value(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* Nearest E2M1 code to v (ties to the even code), |v| beyond 6 saturating to 6. */
uint8_t oracle_e2m1_encode(float v) {
  double a = fabs((double)v);
  uint8_t sign = signbit(v) ? 0x8 : 0x0;
  if (a >= 6.0) return sign | 0x7;
  int lo = 0, hi = 7; /* invariant: value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e2m1_value((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - oracle_e2m1_value((uint8_t)lo);
  double dhi = oracle_e2m1_value((uint8_t)hi) - a;
  int code;
  if (dlo < dhi)
    code = lo;
  else if (dhi < dlo)
    code = hi;
  else
    code = (lo % 2 == 0) ? lo : hi; /* tie: even mantissa */
  return sign | (uint8_t)code;
}

static double load_value(const void* p, int dtype, size_t i) {
  switch (dtype) {
    case ORACLE_F32: return (double)((const float*)p)[i];
    case ORACLE_BF16: return oracle_bf16_value(((const uint16_t*)p)[i]);
    case ORACLE_E2M1: {
      uint8_t byte = ((const uint8_t*)p)[i / 2];
      return oracle_e2m1_value((i & 1) ? (byte >> 4) : (byte & 0xF));
    }
    default: return oracle_e4m3_value(((const uint8_t*)p)[i]);
  }
}

/* ---------------------------------------------------------------------------------------------
 * Fine-grained FP8 quantisation rule (p2 intro)
 * ------------------------------------------------------------------------------------------- */

/* UE8M0 (float8_e8m0fnu): byte b encodes 2^(b - 127); 255 encodes NaN. */
double oracle_e8m0_value(uint8_t b) { return b == 255 ? NAN : ldexp(1.0, (int)b - 127); }

/* UE8M0 scale byte of a group with absolute maximum amax: the smallest e with 448 * 2^e >= amax,
 * e = 0 when amax is 0, as b = e + 127 clamped to 0..254. */
uint8_t oracle_ue8m0_scale(float amax) {
  if (!(amax > 0.0f)) return 127;
  int e = (int)ceil(log2((double)amax / 448.0));
  while (ldexp(448.0, e) < (double)amax) ++e;
  while (ldexp(448.0, e - 1) >= (double)amax) --e;
  int b = e + 127;
  if (b < 0) b = 0;
  if (b > 254) b = 254;
  return (uint8_t)b;
}

/* Quantise one group with a UE8M0 scale: b = oracle_ue8m0_scale(amax), q_i = E4M3(v_i * 2^-e). */
static void quantize_group_ue8m0(const float* v, int n, size_t stride, uint8_t* q, size_t qstride,
                                 uint8_t* b_out) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(v[(size_t)i * stride]);
    if (a > amax) amax = a;
  }
  uint8_t b = oracle_ue8m0_scale(amax);
  float inv = ldexpf(1.0f, 127 - (int)b);
  for (int i = 0; i < n; ++i) q[(size_t)i * qstride] = oracle_e4m3_encode(v[(size_t)i * stride] * inv);
  *b_out = b;
}

/* Quantise one group of n fp32 values: s = amax/448 (fp32), q_i = E4M3(v_i / s). */
static void quantize_group(const float* v, int n, size_t stride, uint8_t* q, size_t qstride,
                           float* s_out) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = fabsf(v[(size_t)i * stride]);
    if (a > amax) amax = a;
  }
  float s = (amax > 0.0f) ? amax / 448.0f : 1.0f;
  for (int i = 0; i < n; ++i) q[(size_t)i * qstride] = oracle_e4m3_encode(v[(size_t)i * stride] / s);
  *s_out = s;
}

/* Activations: per row, per group of `group` consecutive input channels.
 * x [M, K] (fp32 or bf16) -> q [M, K] e4m3, s [M, K/group] fp32. K must be a multiple of group. */
void oracle_quantize_act(const void* x, int x_dtype, int M, int K, int group, uint8_t* q, float* s) {
  int G = K / group;
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; ++m) {
    float* row = (float*)malloc(sizeof(float) * (size_t)K);
    for (int i = 0; i < K; ++i) row[i] = (float)load_value(x, x_dtype, (size_t)m * K + i);
    for (int g = 0; g < G; ++g)
      quantize_group(row + (size_t)g * group, group, 1, q + (size_t)m * K + (size_t)g * group, 1,
                     s + (size_t)m * G + g);
    free(row);
  }
}

/* The same with UE8M0 scales: s [M, K/group] e8m0 bytes. */
void oracle_quantize_act_ue8m0(const void* x, int x_dtype, int M, int K, int group, uint8_t* q,
                               uint8_t* s) {
  int G = K / group;
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; ++m) {
    float* row = (float*)malloc(sizeof(float) * (size_t)K);
    for (int i = 0; i < K; ++i) row[i] = (float)load_value(x, x_dtype, (size_t)m * K + i);
    for (int g = 0; g < G; ++g)
      quantize_group_ue8m0(row + (size_t)g * group, group, 1, q + (size_t)m * K + (size_t)g * group,
                           1, s + (size_t)m * G + g);
    free(row);
  }
}

/* Weights: per 2-D block of `block` x `block`. W [N, K] fp32 -> q [N, K] e4m3,
 * s [N/block, K/block] fp32. N and K must be multiples of block. */
void oracle_quantize_weight(const float* W, int N, int K, int block, uint8_t* q, float* s) {
  int NB = N / block, KB = K / block;
#pragma omp parallel for collapse(2) schedule(static)
  for (int nb = 0; nb < NB; ++nb) {
    for (int kb = 0; kb < KB; ++kb) {
      float amax = 0.0f;
      for (int r = 0; r < block; ++r)
        for (int c = 0; c < block; ++c) {
          float a = fabsf(W[(size_t)(nb * block + r) * K + (size_t)kb * block + c]);
          if (a > amax) amax = a;
        }
      float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
      for (int r = 0; r < block; ++r)
        for (int c = 0; c < block; ++c) {
          size_t i = (size_t)(nb * block + r) * K + (size_t)kb * block + c;
          q[i] = oracle_e4m3_encode(W[i] / sc);
        }
      s[(size_t)nb * KB + kb] = sc;
    }
  }
}

/* ---------------------------------------------------------------------------------------------
 * Router (p4 section 5 and its pseudocode)
 * ------------------------------------------------------------------------------------------- */

/* logits[t][e] = sum_i x[t][i] * Wr[e][i], accumulated in double, rounded once to fp32. */
void oracle_router_logits(const void* x, int x_dtype, const float* Wr, int T, int d, int E,
                          float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i)
        acc += load_value(x, x_dtype, (size_t)t * d + i) * (double)Wr[(size_t)e * d + i];
      logits[(size_t)t * E + e] = (float)acc;
    }
}

/* Top-k selection and renormalised softmax weights.
 * ids[t][j]: the j-th largest logit of token t (ties: lower expert index first).
 * w[t][j] = exp(l_j - l_max) / sum_{j'<k} exp(l_j' - l_max), in double, rounded to fp32. */
void oracle_route(const float* logits, int T, int E, int k, int32_t* ids, float* w) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    char* taken = (char*)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower index on ties */
      }
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    free(taken);
    double m = l[ids[(size_t)t * k]];
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += exp((double)l[ids[(size_t)t * k + j]] - m);
    for (int j = 0; j < k; ++j)
      w[(size_t)t * k + j] = (float)(exp((double)l[ids[(size_t)t * k + j]] - m) / sum);
  }
}

/* ---------------------------------------------------------------------------------------------
 * Grouping tokens by expert (p1 backends table, "grouped_mm": sort tokens by selected expert)
 * ------------------------------------------------------------------------------------------- */

/* Pairs p = t*k + j. counts[e] = #pairs routed to e; offsets = exclusive prefix sum (offsets[E] =
 * T*k); sorted_pair lists the pairs expert by expert, ascending p within an expert; pair_pos is its
 * inverse. */
void oracle_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                    int32_t* sorted_pair, int32_t* pair_pos) {
  int P = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int p = 0; p < P; ++p) counts[ids[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int pos = 0;
  for (int e = 0; e < E; ++e)
    for (int p = 0; p < P; ++p)
      if (ids[p] == e) sorted_pair[pos++] = p;
  for (int q = 0; q < P; ++q) pair_pos[sorted_pair[q]] = q;
}

/* The same with UE8M0 scales: s [N/block, K/block] e8m0 bytes. */
void oracle_quantize_weight_ue8m0(const float* W, int N, int K, int block, uint8_t* q, uint8_t* s) {
  int NB = N / block, KB = K / block;
#pragma omp parallel for collapse(2) schedule(static)
  for (int nb = 0; nb < NB; ++nb) {
    for (int kb = 0; kb < KB; ++kb) {
      float amax = 0.0f;
      for (int r = 0; r < block; ++r)
        for (int c = 0; c < block; ++c) {
          float a = fabsf(W[(size_t)(nb * block + r) * K + (size_t)kb * block + c]);
          if (a > amax) amax = a;
        }
      uint8_t b = oracle_ue8m0_scale(amax);
      float inv = ldexpf(1.0f, 127 - (int)b);
      for (int r = 0; r < block; ++r)
        for (int c = 0; c < block; ++c) {
          size_t i = (size_t)(nb * block + r) * K + (size_t)kb * block + c;
          q[i] = oracle_e4m3_encode(W[i] * inv);
        }
      s[(size_t)nb * KB + kb] = b;
    }
  }
}

/* FP4 (MXFP4) weights: W [N, K] fp32 -> q [N, K/2] bytes (element 2j in the low nibble of byte j),
 * s [N, K/32] UE8M0 bytes: per row and block of 32, b = the byte of the smallest power of two 2^e
 * with 6 * 2^e >= amax (127 for an all-zero block), codes E2M1(v * 2^-e). K % 32 == 0. */
void oracle_quantize_weight_mxfp4(const float* W, int N, int K, uint8_t* q, uint8_t* s) {
  int KB = K / 32;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    for (int kb = 0; kb < KB; ++kb) {
      const float* v = W + (size_t)n * K + (size_t)kb * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i)
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
      int b = 127;
      if (amax > 0.0f) {
        int e = (int)ceil(log2((double)amax / 6.0));
        while (ldexp(6.0, e) < (double)amax) ++e;
        while (ldexp(6.0, e - 1) >= (double)amax) --e;
        b = e + 127;
        if (b < 0) b = 0;
        if (b > 254) b = 254;
      }
      float inv = ldexpf(1.0f, 127 - b);
      for (int i = 0; i < 32; i += 2) {
        uint8_t lo = oracle_e2m1_encode(v[i] * inv), hi = oracle_e2m1_encode(v[i + 1] * inv);
        q[(size_t)n * (K / 2) + (size_t)kb * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
      }
      s[(size_t)n * KB + kb] = (uint8_t)b;
    }
  }
}

/* ---------------------------------------------------------------------------------------------
 * Experts (gated MLP with SwiGLU) and the weighted combine (p1 intro; p4 section 5)
 * ------------------------------------------------------------------------------------------- */

typedef struct {
  int d, f;
  int w_dtype;                       /* ORACLE_F32 / ORACLE_BF16 / ORACLE_E4M3 */
  const void *w_gate, *w_up, *w_down; /* [E,f,d], [E,f,d], [E,d,f] */
  const void *s_gate, *s_up, *s_down; /* e4m3 only: [E,f/128,d/128], [E,d/128,f/128] */
  int quant_act;                     /* 1: activations (x and h) follow the fp8 group rule */
  int scale_fmt;                     /* 0: fp32 scales; 1: UE8M0 bytes (weights and activations) */
} oracle_experts;

static double scale_value(const void* s, int scale_fmt, size_t i) {
  return scale_fmt ? oracle_e8m0_value(((const uint8_t*)s)[i]) : (double)((const float*)s)[i];
}

/* Dequantised weight element W[e][r][c] of an [E, R, C] tensor. */
static double weight_value(const void* w, const void* s, int scale_fmt, int dtype, int e, int r,
                           int c, int R, int C) {
  size_t i = ((size_t)e * R + r) * C + c;
  double v = load_value(w, dtype, i);
  if (dtype == ORACLE_E4M3) {
    int CB = C / 128;
    v *= scale_value(s, scale_fmt, ((size_t)e * (R / 128) + r / 128) * CB + c / 128);
  } else if (dtype == ORACLE_E2M1) { /* MX scales: one byte per row per 32 columns */
    v *= oracle_e8m0_value(((const uint8_t*)s)[((size_t)e * R + r) * (C / 32) + c / 32]);
  }
  return v;
}

/* Apply the activation rule to one fp32 row of length n (in place on the dequantised value). */
static void fake_quant_row(double* v, int n, int scale_fmt) {
  float* tmp = (float*)malloc(sizeof(float) * (size_t)n);
  uint8_t* q = (uint8_t*)malloc((size_t)n);
  for (int i = 0; i < n; ++i) tmp[i] = (float)v[i];
  for (int g = 0; g < n / 128; ++g) {
    double s;
    if (scale_fmt) {
      uint8_t b;
      quantize_group_ue8m0(tmp + g * 128, 128, 1, q + g * 128, 1, &b);
      s = oracle_e8m0_value(b);
    } else {
      float sf;
      quantize_group(tmp + g * 128, 128, 1, q + g * 128, 1, &sf);
      s = (double)sf;
    }
    for (int i = 0; i < 128; ++i) v[g * 128 + i] = oracle_e4m3_value(q[g * 128 + i]) * s;
  }
  free(tmp);
  free(q);
}

/* One expert on one input row xr[d] (already in the activation format the layer uses):
 * h[n] = silu(sum_i xr[i] Wg[e][n][i]) * (sum_i xr[i] Wu[e][n][i]); if quant_act, h is then
 * quantised per 128-group; y[o] = sum_n h[n] Wd[e][o][n]. Returns h (before quantisation) too. */
static void expert_row(const oracle_experts* X, int e, const double* xr, double* h_out,
                       double* y_out) {
  int d = X->d, f = X->f;
  double* h = (double*)malloc(sizeof(double) * (size_t)f);
  for (int n = 0; n < f; ++n) {
    double g = 0.0, u = 0.0;
    for (int i = 0; i < d; ++i) {
      g += xr[i] * weight_value(X->w_gate, X->s_gate, X->scale_fmt, X->w_dtype, e, n, i, f, d);
      u += xr[i] * weight_value(X->w_up, X->s_up, X->scale_fmt, X->w_dtype, e, n, i, f, d);
    }
    h[n] = g / (1.0 + exp(-g)) * u;
  }
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)f);
  if (X->quant_act) fake_quant_row(h, f, X->scale_fmt);
  if (y_out)
    for (int o = 0; o < d; ++o) {
      double acc = 0.0;
      for (int n = 0; n < f; ++n)
        acc += h[n] * weight_value(X->w_down, X->s_down, X->scale_fmt, X->w_dtype, e, o, n, d, f);
      y_out[o] = acc;
    }
  free(h);
}

/* The input row of token t as the experts see it (dequantised if quant_act). */
static void input_row(const void* x, int x_dtype, int d, int t, int quant_act, int scale_fmt,
                      double* xr) {
  for (int i = 0; i < d; ++i) xr[i] = load_value(x, x_dtype, (size_t)t * d + i);
  if (quant_act) fake_quant_row(xr, d, scale_fmt);
}

/* Per-pair expert outputs (for checking the two projections separately).
 * For each listed pair (token tok[n], expert exp_of[n]): h[n][0..f) (before any h quantisation)
 * and y[n][0..d) (unweighted expert output). Either output may be NULL. */
void oracle_expert_pairs(int d, int f, int x_dtype, const void* x, int w_dtype, const void* w_gate,
                         const void* w_up, const void* w_down, const void* s_gate,
                         const void* s_up, const void* s_down, int quant_act, int scale_fmt,
                         int n_pairs, const int32_t* tok, const int32_t* exp_of, double* h,
                         double* y) {
  oracle_experts X = {d, f, w_dtype, w_gate, w_up, w_down, s_gate, s_up, s_down, quant_act,
                      scale_fmt};
#pragma omp parallel for schedule(dynamic, 1)
  for (int n = 0; n < n_pairs; ++n) {
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    input_row(x, x_dtype, d, tok[n], quant_act, scale_fmt, xr);
    expert_row(&X, exp_of[n], xr, h ? h + (size_t)n * f : NULL, y ? y + (size_t)n * d : NULL);
    free(xr);
  }
}

/* The layer: for each listed token t (all tokens if tok_list is NULL),
 *   out[t] = sum_{j<k} w[t][j] * expert_{ids[t][j]}(x[t]),
 * a plain per-token loop over the selected experts, accumulated in double.
 * out is [n_tok, d] in the order of tok_list. */
void oracle_moe_forward(int T, int d, int f, int k, int x_dtype, const void* x, int w_dtype,
                        const void* w_gate, const void* w_up, const void* w_down,
                        const void* s_gate, const void* s_up, const void* s_down, int quant_act,
                        int scale_fmt, const int32_t* ids, const float* topk_w, int n_tok,
                        const int32_t* tok_list, double* out) {
  oracle_experts X = {d, f, w_dtype, w_gate, w_up, w_down, s_gate, s_up, s_down, quant_act,
                      scale_fmt};
  if (!tok_list) n_tok = T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int n = 0; n < n_tok; ++n) {
    int t = tok_list ? tok_list[n] : n;
    double* xr = (double*)malloc(sizeof(double) * (size_t)d);
    double* y = (double*)malloc(sizeof(double) * (size_t)d);
    double* o = out + (size_t)n * d;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    input_row(x, x_dtype, d, t, quant_act, scale_fmt, xr);
    for (int j = 0; j < k; ++j) {
      expert_row(&X, ids[(size_t)t * k + j], xr, NULL, y);
      double wj = (double)topk_w[(size_t)t * k + j];
      for (int i = 0; i < d; ++i) o[i] += wj * y[i];
    }
    free(xr);
    free(y);
  }
}

/* Unfused combine: out[t] = sum_{j<k} w[t][j] * y[pair_pos[t*k+j]], y given per sorted pair. */
void oracle_combine_permuted(const double* y, const int32_t* pair_pos, const float* topk_w, int T,
                             int k, int d, double* out) {
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += (double)topk_w[(size_t)t * k + j] * y[(size_t)pair_pos[(size_t)t * k + j] * d + i];
      out[(size_t)t * d + i] = acc;
    }
}

/* ---------------------------------------------------------------------------------------------
 * The same per-token loop with every sum in fp32 (float), for fp32 or bf16 inputs. The layer's
 * stated oracle is a plain fp32 loop; the fp64 functions above compute the same sums with a
 * smaller rounding error and are the reference the GPU is compared with. These two functions
 * exist so that a test can show the two precisions agree far inside the layer tolerance.
 * ------------------------------------------------------------------------------------------- */

/* logits[t][e] = sum_i x[t][i] * Wr[e][i], summed in fp32 in ascending i (fma-free: each product
 * is rounded to fp32, then added). */
void oracle_router_logits_f32(const void* x, int x_dtype, const float* Wr, int T, int d, int E,
                              float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) {
        volatile float prod = (float)load_value(x, x_dtype, (size_t)t * d + i) * Wr[(size_t)e * d + i];
        acc += prod;
      }
      logits[(size_t)t * E + e] = acc;
    }
}

/* out[t] = sum_{j<k} w[t][j] * expert_{ids[t][j]}(x[t]) with the expert evaluated in fp32:
 * g, u summed in ascending i, h = g / (1 + expf(-g)) * u, y summed in ascending n, then the
 * weighted sum over j = 0..k-1 in fp32. Weights fp32 or bf16 (dtype codes as above). */
void oracle_moe_forward_f32(int T, int d, int f, int k, int x_dtype, const void* x, int w_dtype,
                            const void* w_gate, const void* w_up, const void* w_down,
                            const int32_t* ids, const float* topk_w, int n_tok,
                            const int32_t* tok_list, float* out) {
  if (!tok_list) n_tok = T;
#pragma omp parallel for schedule(dynamic, 1)
  for (int n = 0; n < n_tok; ++n) {
    int t = tok_list ? tok_list[n] : n;
    float* xr = (float*)malloc(sizeof(float) * (size_t)d);
    float* h = (float*)malloc(sizeof(float) * (size_t)f);
    float* o = out + (size_t)n * d;
    for (int i = 0; i < d; ++i) {
      xr[i] = (float)load_value(x, x_dtype, (size_t)t * d + i);
      o[i] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      for (int r = 0; r < f; ++r) {
        float g = 0.0f, u = 0.0f;
        for (int i = 0; i < d; ++i) {
          size_t wi = ((size_t)e * f + r) * d + i;
          volatile float pg = xr[i] * (float)load_value(w_gate, w_dtype, wi);
          volatile float pu = xr[i] * (float)load_value(w_up, w_dtype, wi);
          g += pg;
          u += pu;
        }
        h[r] = g / (1.0f + expf(-g)) * u;
      }
      float wj = topk_w[(size_t)t * k + j];
      for (int c = 0; c < d; ++c) {
        float acc = 0.0f;
        for (int r = 0; r < f; ++r) {
          volatile float p = h[r] * (float)load_value(w_down, w_dtype, ((size_t)e * d + c) * f + r);
          acc += p;
        }
        o[c] += wj * acc;
      }
    }
    free(xr);
    free(h);
  }
}
