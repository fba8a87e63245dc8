// Weighted combine of each token's k expert outputs (Transformers "Experts backends" page,
// introduction; lira-now explainer, section 5 step 6: y = sum_i w_i * expert_i(x)).
// Sums run in fp32 over j = 0..k-1 in order; one rounding to the output type.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, size_t i, float v) {
  p[i] = f32_to_bf16_bits(v);
}

// Any d and alignment: each thread produces 4 consecutive output elements of one token row.
template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y, int layout,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int d, OT* __restrict__ out) {
  const int per_row = (d + 3) / 4;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * per_row) return;
  const int t = static_cast<int>(idx / per_row);
  const int c0 = static_cast<int>(idx - static_cast<size_t>(t) * per_row) * 4;
  const int n = min(4, d - c0);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (layout == MOE_Y_SLOTS) {
    for (int j = 0; j < k; ++j) {
      const size_t base = (static_cast<size_t>(t) * k + j) * d + c0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < n) acc[c] += ld(y, base + c);
    }
  } else if (layout == MOE_Y_PERMUTED) {
    for (int j = 0; j < k; ++j) {
      const size_t p = static_cast<size_t>(t) * k + j;
      const int pos = pair_pos[p];
      if (pos < 0 || pos >= T * k) continue;  // a pair that moe_permute left out (bad expert id)
      const float wj = topk_w[p];
      const size_t base = static_cast<size_t>(pos) * d + c0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < n) acc[c] = fmaf(wj, ld(y, base + c), acc[c]);
    }
  } else {
    const size_t base = static_cast<size_t>(t) * d + c0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (c < n) acc[c] = ld(y, base + c);
  }
  const size_t ob = static_cast<size_t>(t) * d + c0;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (c < n) st(out, ob + c, acc[c]);
}

// Vector path (d % 8 == 0, 16-byte aligned buffers): each thread produces 8 consecutive output
// elements of one token row with 16-byte loads and stores; same arithmetic as above.
template <typename T>
__device__ __forceinline__ void ld8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void ld8<float>(const float* p, float (&v)[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[c] = a[c];
    v[4 + c] = b[c];
  }
}
template <>
__device__ __forceinline__ void ld8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v[2 * c] = __uint_as_float(w[c] << 16);
    v[2 * c + 1] = __uint_as_float(w[c] & 0xFFFF0000u);
  }
}

template <typename T>
__device__ __forceinline__ void st8(T* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void st8<float>(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
}
template <>
__device__ __forceinline__ void st8<uint16_t>(uint16_t* p, const float (&v)[8]) {
  u32x4_t w;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    w[c] = f32_to_bf16_bits(v[2 * c]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * c + 1])) << 16);
  *reinterpret_cast<u32x4_t*>(p) = w;
}

template <typename YT, typename OT>
__global__ __launch_bounds__(256) void combine_vec_kernel(const YT* __restrict__ y, int layout,
                                                          const int32_t* __restrict__ pair_pos,
                                                          const float* __restrict__ topk_w, int T,
                                                          int k, int d, OT* __restrict__ out) {
  const int per_row = d / 8;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * per_row) return;
  const int t = static_cast<int>(idx / per_row);
  const int c0 = static_cast<int>(idx - static_cast<size_t>(t) * per_row) * 8;
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float v[8];
  if (layout == MOE_Y_SLOTS) {
    for (int j = 0; j < k; ++j) {
      ld8(y + (static_cast<size_t>(t) * k + j) * d + c0, v);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] += v[c];
    }
  } else if (layout == MOE_Y_PERMUTED) {
    for (int j = 0; j < k; ++j) {
      const size_t p = static_cast<size_t>(t) * k + j;
      const int pos = pair_pos[p];
      if (pos < 0 || pos >= T * k) continue;
      const float wj = topk_w[p];
      ld8(y + static_cast<size_t>(pos) * d + c0, v);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(wj, v[c], acc[c]);
    }
  } else {
    ld8(y + static_cast<size_t>(t) * d + c0, acc);
  }
  st8(out + static_cast<size_t>(t) * d + c0, acc);
}

}  // namespace

hipError_t launch_combine(const void* y, moe_dtype y_dtype, moe_y_layout layout,
                          const int32_t* pair_pos, const float* topk_w, int T, int k, int d,
                          void* out, moe_dtype out_dtype, hipStream_t stream) {
  const bool vec = d % 8 == 0 &&
                   ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  const size_t n = static_cast<size_t>(T) * (vec ? d / 8 : (d + 3) / 4);
  dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
  const int L = static_cast<int>(layout);
#define MOE_COMBINE(YT, OT)                                                                    \
  if (vec)                                                                                     \
    hipLaunchKernelGGL((combine_vec_kernel<YT, OT>), grid, block, 0, stream,                   \
                       static_cast<const YT*>(y), L, pair_pos, topk_w, T, k, d,                \
                       static_cast<OT*>(out));                                                 \
  else                                                                                         \
    hipLaunchKernelGGL((combine_kernel<YT, OT>), grid, block, 0, stream,                       \
                       static_cast<const YT*>(y), L, pair_pos, topk_w, T, k, d,                \
                       static_cast<OT*>(out))
  if (y_dtype == MOE_BF16 && out_dtype == MOE_BF16) {
    MOE_COMBINE(uint16_t, uint16_t);
  } else if (y_dtype == MOE_BF16) {
    MOE_COMBINE(uint16_t, float);
  } else if (out_dtype == MOE_BF16) {
    MOE_COMBINE(float, uint16_t);
  } else {
    MOE_COMBINE(float, float);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
