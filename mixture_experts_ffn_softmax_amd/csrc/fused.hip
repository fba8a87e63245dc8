// Fused small-batch path, its routing launch: one token per workgroup.
//
// The single fused MoE kernel idea (AWS fused-MoE news page: one kernel for routing, both expert
// projections and the combine), taken as far as it pays on gfx950: routing, top-k and the
// activation quantisation in one launch, no permutation (the expert kernels find each expert's
// pairs in the routing ids themselves), then the expert projections and the combine. This kernel
// computes a token's router logits (or reads given ones), picks its top k with renormalised
// softmax weights (lira-now explainer, section 5) and quantises its activations to e4m3 per 128
// channels for fp8 / FP4 experts (Transformers "Fine-grained FP8" page).
#include "common.h"
#include "launch.h"
#include "route_dev.h"

namespace moe {
namespace {

struct FusedRouteArgs {
  const void* x;              // [T, d]
  const float* logits_in;     // [T, E], or null: computed from wr
  const float* wr;            // [E, d] fp32
  float* logits_out;          // optional [T, E] (computed logits only)
  int d, E, k, G;
  int32_t* ids;               // [T, k]
  float* w;                   // [T, k]
  uint8_t* xq;                // fp8: e4m3 codes [T, d]
  void* xs;                   // fp8: scales [T, d/128], fp32 or (UE8M0) e8m0 bytes
};

template <typename XT, int VPL, bool kQuant, bool kUE>
__global__ __launch_bounds__(256) void fused_route_kernel(FusedRouteArgs a) {
  __shared__ float lg[kMaxExperts];
  __shared__ float red[4][kVecExperts];
  const int t = blockIdx.x;
  const XT* xr = static_cast<const XT*>(a.x) + static_cast<size_t>(t) * a.d;
  const float* row;
  if (a.logits_in) {
    row = a.logits_in + static_cast<size_t>(t) * a.E;
  } else {
    token_logits<XT>(xr, a.wr, a.d, a.E, lg, red);   // ends with a barrier
    row = lg;
    if (a.logits_out)
      for (int e = threadIdx.x; e < a.E; e += 256) a.logits_out[static_cast<size_t>(t) * a.E + e] = lg[e];
  }
  if (static_cast<int>(threadIdx.x) < a.G)
    topk_select<VPL>(row, true, a.E, a.k, a.G, threadIdx.x, a.ids + static_cast<size_t>(t) * a.k,
                     a.w + static_cast<size_t>(t) * a.k);
  if constexpr (kQuant) {
    // 128-channel groups, 16 lanes each (the rule of the activation quantiser)
    const int ng = a.d / kFp8Group;
    for (int g0 = 0; g0 < ng; g0 += 16) {
      const int grp = g0 + static_cast<int>(threadIdx.x) / 16;
      const bool active = grp < ng;
      const int col = grp * kFp8Group + (threadIdx.x & 15) * 8;
      float v[8];
      if (active) {
        load_x8<XT>(xr + col, v);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
      }
      uint32_t lo, hi;
      int byte;
      const float s = quant_group16<kUE>(v, lo, hi, &byte);
      if (active) {
        *reinterpret_cast<uint2*>(a.xq + static_cast<size_t>(t) * a.d + col) = make_uint2(lo, hi);
        if ((threadIdx.x & 15) == 0) {
          const size_t si = static_cast<size_t>(t) * ng + grp;
          if constexpr (kUE) static_cast<uint8_t*>(a.xs)[si] = static_cast<uint8_t>(byte);
          else static_cast<float*>(a.xs)[si] = s;
        }
      }
    }
  }
}

template <typename XT, int VPL>
void launch_route_q(const FusedRouteArgs& a, int T, bool quant, bool ue, hipStream_t stream) {
  const dim3 grid(T), block(256);
  if (!quant)
    hipLaunchKernelGGL((fused_route_kernel<XT, VPL, false, false>), grid, block, 0, stream, a);
  else if (ue)
    hipLaunchKernelGGL((fused_route_kernel<XT, VPL, true, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fused_route_kernel<XT, VPL, true, false>), grid, block, 0, stream, a);
}

template <typename XT>
void launch_route_x(const FusedRouteArgs& a, int T, int vpl, bool quant, bool ue,
                    hipStream_t stream) {
  switch (vpl) {
    case 1: launch_route_q<XT, 1>(a, T, quant, ue, stream); break;
    case 2: launch_route_q<XT, 2>(a, T, quant, ue, stream); break;
    case 4: launch_route_q<XT, 4>(a, T, quant, ue, stream); break;
    case 8: launch_route_q<XT, 8>(a, T, quant, ue, stream); break;
    case 16: launch_route_q<XT, 16>(a, T, quant, ue, stream); break;
    case 32: launch_route_q<XT, 32>(a, T, quant, ue, stream); break;
    default: launch_route_q<XT, 64>(a, T, quant, ue, stream); break;
  }
}

}  // namespace

hipError_t launch_fused_route(const void* x, moe_dtype x_dtype, const float* logits,
                              const float* wr, float* logits_out, int T, int d, int E, int k,
                              int32_t* ids, float* w, uint8_t* xq, void* xs, bool ue,
                              hipStream_t stream) {
  FusedRouteArgs a{};
  a.x = x;
  a.logits_in = logits;
  a.wr = wr;
  a.logits_out = logits ? nullptr : logits_out;
  a.d = d;
  a.E = E;
  a.k = k;
  a.G = topk_group_lanes(E, k);
  a.ids = ids;
  a.w = w;
  a.xq = xq;
  a.xs = xs;
  const int vpl = topk_vpl(E, a.G);
  const bool quant = xq != nullptr;
  if (x_dtype == MOE_BF16) launch_route_x<uint16_t>(a, T, vpl, quant, ue, stream);
  else launch_route_x<float>(a, T, vpl, quant, ue, stream);
  return hipGetLastError();
}

}  // namespace moe
