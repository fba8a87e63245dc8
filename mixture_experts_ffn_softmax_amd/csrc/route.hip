// Router kernels: optional fp32 router GEMM (logits = x . Wr^T) and the wavefront-level
// softmax -> top-k -> renormalise selection.
//
// Routing steps: lira-now explainer "Mixture of Experts (MoE): a practical explanation",
// section 5 (router step by step) and its pseudocode.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kLogitTokensPerWave = 4;
constexpr int kLogitExpertChunk = 8;

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p, size_t i);
template <>
__device__ __forceinline__ float load_x<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

// One wave computes the logits of 4 tokens against a chunk of 8 experts at a time: every router
// weight element it loads is used for 4 tokens. Lanes stride over d in runs of 4 elements.
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ wr, int T,
                                                            int d, int E,
                                                            float* __restrict__ logits) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int t0 = (blockIdx.x * (blockDim.x / kWave) + wave) * kLogitTokensPerWave;
  if (t0 >= T) return;
  const int nt = min(kLogitTokensPerWave, T - t0);
  for (int e0 = 0; e0 < E; e0 += kLogitExpertChunk) {
    const int ne = min(kLogitExpertChunk, E - e0);
    float acc[kLogitTokensPerWave][kLogitExpertChunk];
#pragma unroll
    for (int a = 0; a < kLogitTokensPerWave; ++a)
#pragma unroll
      for (int b = 0; b < kLogitExpertChunk; ++b) acc[a][b] = 0.0f;
    for (int i = lane * 4; i < d; i += kWave * 4) {
      const int n = min(4, d - i);
      float xv[kLogitTokensPerWave][4];
#pragma unroll
      for (int a = 0; a < kLogitTokensPerWave; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          xv[a][c] = (a < nt && c < n) ? load_x(x, static_cast<size_t>(t0 + a) * d + i + c) : 0.0f;
#pragma unroll
      for (int b = 0; b < kLogitExpertChunk; ++b) {
        if (b >= ne) break;
        float wv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          wv[c] = c < n ? wr[static_cast<size_t>(e0 + b) * d + i + c] : 0.0f;
#pragma unroll
        for (int a = 0; a < kLogitTokensPerWave; ++a)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[a][b] = fmaf(xv[a][c], wv[c], acc[a][b]);
      }
    }
#pragma unroll
    for (int a = 0; a < kLogitTokensPerWave; ++a)
#pragma unroll
      for (int b = 0; b < kLogitExpertChunk; ++b) {
        float s = wave_sum(acc[a][b]);
        if (lane == a * kLogitExpertChunk + b && a < nt && b < ne)
          logits[static_cast<size_t>(t0 + a) * E + e0 + b] = s;
      }
  }
}

// "a is a better candidate than b": larger logit, equal logits -> lower expert index;
// index < 0 means "no candidate".
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  if (ib < 0) return ia >= 0;
  if (ia < 0) return false;
  return va > vb || (va == vb && ia < ib);
}

// Top-k + renormalised softmax weights. A group of G lanes (G a power of two, G = 64 when E > 64)
// handles one token; each lane holds VPL logits (expert e = lane_in_group + G * v). k rounds of a
// butterfly argmax inside the group pick the experts in descending order; the lane whose slot
// index equals the round keeps the winner, so lane j of the group ends with the j-th selection.
template <int VPL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int G,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ w) {
  const int lane = lane_id();
  const int gl = lane & (G - 1);
  const int groups_per_wave = kWave / G;
  const int t = (blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * groups_per_wave +
                lane / G;
  const bool tok_ok = t < T;
  float v[VPL];
  unsigned taken = 0;
#pragma unroll
  for (int q = 0; q < VPL; ++q) {
    int e = gl + G * q;
    v[q] = (tok_ok && e < E) ? logits[static_cast<size_t>(t) * E + e] : 0.0f;
  }
  float my_v = 0.0f, vmax = 0.0f;
  int my_i = -1;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
      int e = gl + G * q;
      bool cand = e < E && !((taken >> q) & 1u);
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
      if (gl + G * q == bi) taken |= 1u << q;
    if (gl == j) { my_v = bv; my_i = bi; }
  }
  float a = (gl < k) ? expf(my_v - vmax) : 0.0f;
  float s = a;
  for (int o = G >> 1; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (tok_ok && gl < k) {
    ids[static_cast<size_t>(t) * k + gl] = my_i;
    w[static_cast<size_t>(t) * k + gl] = a / s;
  }
}

}  // namespace

hipError_t launch_router_logits(const void* x, moe_dtype x_dtype, const float* wr, int T, int d,
                                int E, float* logits, hipStream_t stream) {
  const int tokens_per_block = 4 * kLogitTokensPerWave;
  dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
  if (x_dtype == MOE_BF16)
    hipLaunchKernelGGL(router_logits_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), wr, T, d, E, logits);
  else
    hipLaunchKernelGGL(router_logits_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(x), wr, T, d, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                               hipStream_t stream) {
  int G = 1;
  while (G < E && G < kWave) G <<= 1;
  const int vpl = (E + G - 1) / G;
  const int tokens_per_block = 4 * (kWave / G);
  dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
#define MOE_TOPK_CASE(N)                                                                      \
  case N:                                                                                     \
    hipLaunchKernelGGL(topk_softmax_kernel<N>, grid, block, 0, stream, logits, T, E, k, G, ids, \
                       w);                                                                    \
    break;
  switch (vpl <= 1 ? 1 : vpl <= 2 ? 2 : vpl <= 4 ? 4 : vpl <= 8 ? 8 : 16) {
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(16)
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

}  // namespace moe
