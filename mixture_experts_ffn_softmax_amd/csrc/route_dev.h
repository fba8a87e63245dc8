// Device pieces of routing shared by the routing kernels and the fused small-batch path: 8-wide
// loads, one token's router logits with one block, and the top-k selection with renormalised
// softmax weights.
//
// Routing steps: lira-now explainer "Mixture of Experts (MoE): a practical explanation",
// section 5 (router step by step) and its pseudocode.
#pragma once
#include "common.h"

namespace moe {

constexpr int kVecExperts = 8;   // experts per pass of the block-level logit kernels

template <typename XT>
__device__ __forceinline__ void load_x8(const XT* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load_x8<float>(const float* p, float (&v)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[c] = a[c];
    v[4 + c] = b[c];
  }
}
template <>
__device__ __forceinline__ void load_x8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[2 * c] = __uint_as_float(w[c] << 16);
    v[2 * c + 1] = __uint_as_float(w[c] & 0xFFFF0000u);
  }
}

// Router logits of one token with a block of 256 threads: thread j covers x[i .. i+8) for
// i = 8 j + 2048 n against 8 experts at a time; the 8 sums are reduced over each wave and then over
// the 4 waves in wave order, and logits[e] (global memory or LDS) gets expert e's sum. Two 2048-wide
// chunks go per iteration with all their loads issued before the first product (rows past the
// last expert read the last expert's row and are dropped), so a token waits on one memory round
// trip per 4096 channels instead of one per expert and chunk; each sum still takes its products in
// ascending i.
template <typename XT>
__device__ void token_logits(const XT* __restrict__ x, const float* __restrict__ wr, int d, int E,
                             float* logits, float (*red)[kVecExperts]) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  for (int e0 = 0; e0 < E; e0 += kVecExperts) {
    float acc[kVecExperts];
    const float* wrow[kVecExperts];
#pragma unroll
    for (int b = 0; b < kVecExperts; ++b) {
      acc[b] = 0.0f;
      wrow[b] = wr + static_cast<size_t>(min(e0 + b, E - 1)) * d;
    }
    int i = threadIdx.x * 8;
    for (; i + 256 * 8 < d; i += 2 * 256 * 8) {   // both chunks: loads, fence, products
      float xv[2][8], wv[2][kVecExperts][8];
      load_x8<XT>(x + i, xv[0]);
      load_x8<XT>(x + i + 256 * 8, xv[1]);
#pragma unroll
      for (int b = 0; b < kVecExperts; ++b) {
        load_x8<float>(wrow[b] + i, wv[0][b]);
        load_x8<float>(wrow[b] + i + 256 * 8, wv[1][b]);
      }
      __builtin_amdgcn_sched_barrier(0);   // every load issued before the first product
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < kVecExperts; ++b)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[b] = fmaf(xv[h][c], wv[h][b][c], acc[b]);
    }
    if (i < d) {   // a last single chunk
      float xv[8], wv[kVecExperts][8];
      load_x8<XT>(x + i, xv);
#pragma unroll
      for (int b = 0; b < kVecExperts; ++b) load_x8<float>(wrow[b] + i, wv[b]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < kVecExperts; ++b)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[b] = fmaf(xv[c], wv[b][c], acc[b]);
    }
#pragma unroll
    for (int b = 0; b < kVecExperts; ++b) {
      const float v = wave_sum(acc[b]);
      if (lane == b) red[wave][b] = v;
    }
    __syncthreads();
    if (threadIdx.x < kVecExperts && e0 + threadIdx.x < E) {
      const int b = threadIdx.x;
      logits[e0 + b] = ((red[0][b] + red[1][b]) + red[2][b]) + red[3][b];
    }
    __syncthreads();
  }
}

// Selection key of expert e with logit x: unsigned 64-bit keys compare as "larger logit, equal
// logits -> lower expert index". High word: the logit's bits mapped to an unsigned order (-0
// taken as +0, so the two zeros tie like equal floats; NaNs order by their bits, above +inf when
// positive and below -inf when negative); low word: ~e. Key 0 stands for "no candidate": every
// real key is larger, since its low word ~e is not zero.
__device__ __forceinline__ uint64_t topk_key(float x, int e) {
  uint32_t b = __float_as_uint(x);
  if (b == 0x80000000u) b = 0u;
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~e);
}
__device__ __forceinline__ float topk_key_value(uint64_t key) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
__device__ __forceinline__ int topk_key_index(uint64_t key) {
  return static_cast<int>(~static_cast<uint32_t>(key));
}

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return (static_cast<uint64_t>(dpp_u32<kCtrl>(static_cast<uint32_t>(v >> 32))) << 32) |
         dpp_u32<kCtrl>(static_cast<uint32_t>(v));
}
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  return __longlong_as_double(static_cast<long long>(dpp_u64<kCtrl>(u)));
}

// Reductions over the G lanes of a group (a power of two, groups aligned to G): DPP steps up to
// 16 lanes (every lane ends with the group's result, formed by the same association in every
// lane), cross-row shuffles beyond.
__device__ __forceinline__ uint64_t group_max_key(uint64_t v, int G) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  if (G > 1) v = mx(v, dpp_u64<kDppXor1>(v));
  if (G > 2) v = mx(v, dpp_u64<kDppXor2>(v));
  if (G > 4) v = mx(v, dpp_u64<kDppHalfMirror>(v));
  if (G > 8) v = mx(v, dpp_u64<kDppMirror>(v));
  for (int o = 16; o < G; o <<= 1) {
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, 64);
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, 64);
    v = mx(v, (static_cast<uint64_t>(hi) << 32) | lo);
  }
  return v;
}
__device__ __forceinline__ double group_sum_f64(double s, int G) {
  if (G > 1) s += dpp_f64<kDppXor1>(s);
  if (G > 2) s += dpp_f64<kDppXor2>(s);
  if (G > 4) s += dpp_f64<kDppHalfMirror>(s);
  if (G > 8) s += dpp_f64<kDppMirror>(s);
  for (int o = 16; o < G; o <<= 1) s += __shfl_xor(s, o, 64);
  return s;
}

// Top-k + renormalised softmax weights. A group of G lanes (a power of two: pow2(E) up to 16 lanes,
// more only when k > 16 so that every pick has its own lane) handles one token (row: its E logits,
// in global memory or LDS; every lane of the group active); each lane holds VPL selection keys
// (expert e = lane_in_group + G * v). Each of the k rounds takes the largest key of every lane,
// then of the group, and clears the winner's key where it sits; lane j of the group keeps the
// j-th selection, so the experts come out in descending order with the lower-index tie rule.
template <int VPL>
__device__ __forceinline__ void topk_select(const float* row, bool tok_ok, int E, int k, int G,
                                            int gl, int32_t* ids, float* w) {
  uint64_t key[VPL];
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    const int e = gl + G * q;
    const float x = row[min(e, E - 1)];   // in bounds for every lane; the key drops e >= E
    key[q] = (tok_ok && e < E) ? topk_key(x, e) : 0ull;
  }
  uint64_t first = 0, mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < VPL; ++q) best = key[q] > best ? key[q] : best;
    best = group_max_key(best, G);
    // keys are unique (the expert index is in the low word), so one slot of one lane matches
    const uint32_t won = static_cast<uint32_t>(best);
#pragma unroll
    for (int q = 0; q < VPL; ++q) key[q] = static_cast<uint32_t>(key[q]) == won ? 0ull : key[q];
    if (j == 0) first = best;
    if (gl == j) mine = best;
  }
  // The k weights in double, rounded once to fp32: the result is the correctly rounded value of
  // exp(l_j - l_max) / sum exp(l - l_max) except within ~1e-16 of a rounding boundary, so it does
  // not depend on the order of the sum (k exponentials per token: negligible work).
  const double a = (gl < k) ? exp(static_cast<double>(topk_key_value(mine)) -
                                  static_cast<double>(topk_key_value(first)))
                            : 0.0;
  const double s = group_sum_f64(a, G);
  if (tok_ok && gl < k) {
    ids[gl] = topk_key_index(mine);
    w[gl] = static_cast<float>(a / s);
  }
}


// Lanes per token of topk_select: pow2(E) up to 16, more only when k > 16 so that every pick has
// its own lane (k <= 32 <= kWave).
inline int topk_group_lanes(int E, int k) {
  int G = 1;
  while (G < E && G < 16) G <<= 1;
  while (G < k) G <<= 1;
  return G;
}

// topk_select's VPL template argument for E experts over G lanes (a power of two, 1..64).
inline int topk_vpl(int E, int G) {
  const int v = (E + G - 1) / G;
  return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : v <= 8 ? 8 : v <= 16 ? 16 : v <= 32 ? 32 : 64;
}

}  // namespace moe
