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

// "a is a better candidate than b": larger logit, equal logits -> lower expert index;
// index < 0 means "no candidate".
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  if (ib < 0) return ia >= 0;
  if (ia < 0) return false;
  return va > vb || (va == vb && ia < ib);
}

// Top-k + renormalised softmax weights. A group of G lanes (a power of two: pow2(E) up to 16 lanes,
// more only when k > 16 so that every pick has its own lane) handles one token (row: its E logits, in global memory or LDS); each lane holds
// VPL logits (expert e = lane_in_group + G * v). k rounds of a lane-local scan plus a butterfly
// argmax inside the group pick the experts in descending order; the lane whose slot index equals
// the round keeps the winner, so lane j of the group ends with the j-th selection.
template <int VPL>
__device__ __forceinline__ void topk_select(const float* row, bool tok_ok, int E, int k, int G,
                                            int gl, int32_t* ids, float* w) {
  float v[VPL];
  uint64_t taken = 0;
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    int e = gl + G * q;
    v[q] = (tok_ok && e < E) ? row[e] : 0.0f;
  }
  float my_v = 0.0f, vmax = 0.0f;
  int my_i = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      int e = gl + G * q;
      bool cand = e < E && !((taken >> q) & 1ull);
      if (cand && better(v[q], e, bv, bi)) { bv = v[q]; bi = e; }
    }
    for (int o = G >> 1; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (j == 0) vmax = bv;
#pragma unroll
    for (int q = 0; q < VPL; ++q)
      if (gl + G * q == bi) taken |= 1ull << q;
    if (gl == j) { my_v = bv; my_i = bi; }
  }
  // The k weights in double, rounded once to fp32: the result is the correctly rounded value of
  // exp(l_j - l_max) / sum exp(l - l_max) except within ~1e-16 of a rounding boundary, so it does
  // not depend on the order of the sum (k exponentials per token: negligible work).
  const double a = (gl < k) ? exp(static_cast<double>(my_v) - static_cast<double>(vmax)) : 0.0;
  double s = a;
  for (int o = G >> 1; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (tok_ok && gl < k) {
    ids[gl] = my_i;
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
