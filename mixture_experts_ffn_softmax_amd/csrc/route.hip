// Router kernels: optional fp32 router GEMM (logits = x . Wr^T) and the wavefront-level
// softmax -> top-k -> renormalise selection.
//
// Routing steps: lira-now explainer "Mixture of Experts (MoE): a practical explanation",
// section 5 (router step by step) and its pseudocode.
#include "common.h"
#include "launch.h"
#include "route_dev.h"

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

// Any d and alignment: one wave computes the logits of 4 tokens against a chunk of 8 experts at a
// time; every router weight element it loads is used for 4 tokens. Lanes stride over d in runs
// of 4 elements.
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

// Vector path (d % 8 == 0, 16-byte aligned rows): a block of 4 waves computes the logits of
// kVecTokens tokens against 8 experts at a time. Lane l of wave w covers x[t][i .. i+8) for
// i = (64 w + l) * 8 + 2048 j, so each wave reads 1 KB contiguous per token and the block splits K
// four ways. Each lane ends with 64 partial sums (8 tokens x 8 experts); recursive halving over
// the wave (32 + 16 + ... + 1 exchanges) leaves the full wave sum of entry l in lane l, and the
// four waves' sums are added through LDS in wave order.
constexpr int kVecTokens = 8;

// One halving step: lanes with bit H set keep entries [H, 2H), the others [0, H); each adds the
// partner's copy of the kept half, received in exchange for the half it gives away.
template <int H>
__device__ __forceinline__ void halve(float (&v)[64], int lane) {
  const bool upper = (lane & H) != 0;
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const float send = upper ? v[j] : v[j + H];
    const float keep = upper ? v[j + H] : v[j];
    v[j] = keep + __shfl_xor(send, H, 64);
  }
}

// After the call lane l holds the sum over the wave of v[l] (all 64 entries reduced at once).
__device__ __forceinline__ float wave_reduce_scatter64(float (&v)[64], int lane) {
  halve<32>(v, lane);
  halve<16>(v, lane);
  halve<8>(v, lane);
  halve<4>(v, lane);
  halve<2>(v, lane);
  halve<1>(v, lane);
  return v[0];
}

template <typename XT>
__global__ __launch_bounds__(256) void router_logits_vec_kernel(const XT* __restrict__ x,
                                                                const float* __restrict__ wr,
                                                                int T, int d, int E,
                                                                float* __restrict__ logits) {
  __shared__ float red[4][64];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kVecTokens;
  // Tokens past T and experts past E read the last token's or expert's row; their sums are
  // dropped. All of a chunk's loads are issued before its first product (one memory round trip
  // per 2048 channels); each sum takes its products in ascending channel order.
  const XT* xrow[kVecTokens];
#pragma unroll
  for (int a = 0; a < kVecTokens; ++a) xrow[a] = x + static_cast<size_t>(min(t0 + a, T - 1)) * d;
  for (int e0 = 0; e0 < E; e0 += kVecExperts) {
    float acc[64];
#pragma unroll
    for (int q = 0; q < 64; ++q) acc[q] = 0.0f;
    const float* wrow[kVecExperts];
#pragma unroll
    for (int b = 0; b < kVecExperts; ++b) wrow[b] = wr + static_cast<size_t>(min(e0 + b, E - 1)) * d;
    for (int i = (wave * kWave + lane) * 8; i < d; i += 4 * kWave * 8) {
      float xv[kVecTokens][8], wv[kVecExperts][8];
#pragma unroll
      for (int a = 0; a < kVecTokens; ++a) load_x8<XT>(xrow[a] + i, xv[a]);
#pragma unroll
      for (int b = 0; b < kVecExperts; ++b) load_x8<float>(wrow[b] + i, wv[b]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < kVecExperts; ++b)
#pragma unroll
        for (int a = 0; a < kVecTokens; ++a)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[a * 8 + b] = fmaf(xv[a][c], wv[b][c], acc[a * 8 + b]);
    }
    red[wave][lane] = wave_reduce_scatter64(acc, lane);
    __syncthreads();
    if (wave == 0) {
      const float s = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
      const int t = t0 + lane / 8, e = e0 + lane % 8;
      if (t < T && e < E) logits[static_cast<size_t>(t) * E + e] = s;
    }
    __syncthreads();
  }
}

// Few tokens (a decode step): one block per token, so the router weights are read by many CUs at
// once instead of a handful.
template <typename XT>
__global__ __launch_bounds__(256) void router_logits_tok_kernel(const XT* __restrict__ x,
                                                                const float* __restrict__ wr,
                                                                int d, int E,
                                                                float* __restrict__ logits) {
  __shared__ float red[4][kVecExperts];
  const int t = blockIdx.x;
  token_logits<XT>(x + static_cast<size_t>(t) * d, wr, d, E, logits + static_cast<size_t>(t) * E,
                   red);
}

// Top-k for T tokens: groups of G lanes, one token each (topk_select).
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
  const size_t tt = tok_ok ? static_cast<size_t>(t) : 0;
  topk_select<VPL>(logits + tt * E, tok_ok, E, k, G, gl, ids + tt * k, w + tt * k);
}

}  // namespace

hipError_t launch_router_logits(const void* x, moe_dtype x_dtype, const float* wr, int T, int d,
                                int E, float* logits, hipStream_t stream) {
  const bool vec = d % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(wr) & 15) == 0;
  if (vec && T < 256) {
    // fewer than 32 blocks of the token-group kernel would leave most CUs idle
    if (x_dtype == MOE_BF16)
      hipLaunchKernelGGL(router_logits_tok_kernel<uint16_t>, dim3(T), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(x), wr, d, E, logits);
    else
      hipLaunchKernelGGL(router_logits_tok_kernel<float>, dim3(T), dim3(256), 0, stream,
                         static_cast<const float*>(x), wr, d, E, logits);
    return hipGetLastError();
  }
  if (vec) {
    dim3 grid((T + kVecTokens - 1) / kVecTokens), block(256);
    if (x_dtype == MOE_BF16)
      hipLaunchKernelGGL(router_logits_vec_kernel<uint16_t>, grid, block, 0, stream,
                         static_cast<const uint16_t*>(x), wr, T, d, E, logits);
    else
      hipLaunchKernelGGL(router_logits_vec_kernel<float>, grid, block, 0, stream,
                         static_cast<const float*>(x), wr, T, d, E, logits);
    return hipGetLastError();
  }
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
  const int G = topk_group_lanes(E, k);
  const int tokens_per_block = 4 * (kWave / G);
  dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
#define MOE_TOPK_CASE(N)                                                                      \
  case N:                                                                                     \
    hipLaunchKernelGGL(topk_softmax_kernel<N>, grid, block, 0, stream, logits, T, E, k, G, ids, \
                       w);                                                                    \
    break;
  switch (topk_vpl(E, G)) {
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(16)
    MOE_TOPK_CASE(32)
    MOE_TOPK_CASE(64)
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

}  // namespace moe
