// Fine-grained FP8 quantisation (Transformers "Fine-grained FP8" page, introduction): activations
// per token per 128 input channels with run-time scales, weights per 128x128 block.
// Rule for one group/block: s = amax / 448 (fp32, IEEE division; s = 1 if all zero),
// q = e4m3(v / s), round-to-nearest-even, saturating at +-448. With UE8M0 scales (same page,
// "UE8M0 scale format": scales stored as float8_e8m0fnu bytes, powers of two): the byte b of the
// smallest power of two 2^e with 448 * 2^e >= amax, q = e4m3(v * 2^-e) (an exact scaling).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

template <typename XT>
__device__ __forceinline__ void load8(const XT* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  uint4 r = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One wave covers 4 groups of one row: 16 lanes per group, 8 consecutive elements per lane.
template <typename XT, bool kUe8m0>
__global__ __launch_bounds__(256) void quantize_act_kernel(const XT* __restrict__ x, int M, int K,
                                                           const int32_t* __restrict__ row_index,
                                                           uint8_t* __restrict__ q,
                                                           void* __restrict__ scales) {
  const int G = K / kFp8Group;
  const int waves_per_row = (G + 3) / 4;
  const int wid = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int row = wid / waves_per_row;
  if (row >= M) return;
  const int lane = lane_id();
  const int g = (wid - row * waves_per_row) * 4 + lane / 16;
  const bool active = g < G;
  const int src_row = row_index ? row_index[row] : row;
  const int col = g * kFp8Group + (lane & 15) * 8;
  float v[8];
  if (active) {
    load8(x + static_cast<size_t>(src_row) * K + col, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  uint32_t lo, hi;
  int b;
  const float s = quant_group16<kUe8m0>(v, lo, hi, &b);
  if (!active) return;
  if ((lane & 15) == 0) {
    if constexpr (kUe8m0)
      static_cast<uint8_t*>(scales)[static_cast<size_t>(row) * G + g] = static_cast<uint8_t>(b);
    else
      static_cast<float*>(scales)[static_cast<size_t>(row) * G + g] = s;
  }
  *reinterpret_cast<uint2*>(q + static_cast<size_t>(row) * K + col) = make_uint2(lo, hi);
}

// One block of 256 threads per 128x128 block: each thread owns 64 elements (16 rows x 4 columns
// per pass, 4 bytes of output each), block-wide amax through LDS.
template <typename WT, bool kUe8m0>
__global__ __launch_bounds__(256) void quantize_weight_kernel(const WT* __restrict__ w, int N,
                                                              int K, uint8_t* __restrict__ q,
                                                              void* __restrict__ scales) {
  const int KB = K / kFp8Group, NB = N / kFp8Group;
  const int kb = blockIdx.x % KB;
  const int nb = (blockIdx.x / KB) % NB;
  const size_t mat = blockIdx.x / (KB * NB);
  const WT* src = w + mat * N * static_cast<size_t>(K);
  uint8_t* dst = q + mat * N * static_cast<size_t>(K);
  const int c4 = (threadIdx.x & 31) * 4;   // column within block
  const int r0 = threadIdx.x >> 5;         // 0..7
  float v[16][4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const size_t off = static_cast<size_t>(nb * kFp8Group + r0 + 8 * i) * K + kb * kFp8Group + c4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x;
      if constexpr (sizeof(WT) == 2) x = bf16_bits_to_f32(src[off + c]);
      else x = src[off + c];
      v[i][c] = x;
      amax = fmaxf(amax, fabsf(x));
    }
  }
  amax = wave_max(amax);
  __shared__ float red[4];
  if (lane_id() == 0) red[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // fp32 rule: divide by s; UE8M0: multiply by 2^-e
  const int b = ue8m0_byte(amax);
  const float s = kUe8m0 ? ldexpf(1.0f, 127 - b) : (amax > 0.0f ? amax / 448.0f : 1.0f);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const size_t off = static_cast<size_t>(nb * kFp8Group + r0 + 8 * i) * K + kb * kFp8Group + c4;
    uint32_t packed = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      packed |= e4m3_encode(kUe8m0 ? v[i][c] * s : v[i][c] / s) << (8 * c);
    *reinterpret_cast<uint32_t*>(dst + off) = packed;
  }
  if (threadIdx.x == 0) {
    if constexpr (kUe8m0) static_cast<uint8_t*>(scales)[(mat * NB + nb) * KB + kb] = static_cast<uint8_t>(b);
    else static_cast<float*>(scales)[(mat * NB + nb) * KB + kb] = s;
  }
}

// FP4 with MX scales: one thread per 32-element block of a row (packed 16 bytes + a scale byte).
template <typename WT>
__global__ __launch_bounds__(256) void quantize_weight_mx4_kernel(const WT* __restrict__ w,
                                                                  size_t nblocks,
                                                                  uint8_t* __restrict__ q,
                                                                  uint8_t* __restrict__ scales) {
  const size_t blk = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  const WT* src = w + blk * 32;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (sizeof(WT) == 2) v[i] = bf16_bits_to_f32(src[i]);
    else v[i] = src[i];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int b = mx4_byte(amax);
  const float inv = ldexpf(1.0f, 127 - b);
  u32x4_t o;
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) word |= e2m1_encode(v[wd * 8 + j] * inv) << (4 * j);
    o[wd] = word;
  }
  *reinterpret_cast<u32x4_t*>(q + blk * 16) = o;
  scales[blk] = static_cast<uint8_t>(b);
}

// Packed E2M1 rows -> matrix-fragment order: one thread moves the 16 bytes (32 values) that one
// lane of a 16x128 fragment holds. Fragment (b, n16, c) is 1 KB at ((b * N/16 + n16) * KB + c);
// within it lane l = r + 16 g holds row 16 n16 + r, K = 128 c + 32 g .. + 31.
__global__ __launch_bounds__(256) void tile_weight_fp4_kernel(const uint8_t* __restrict__ q,
                                                              size_t nchunks, int KB,
                                                              uint8_t* __restrict__ out) {
  const size_t t = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= nchunks) return;
  const int l = static_cast<int>(t & 63);
  const size_t frag = t >> 6;                  // (b * N/16 + n16) * KB + c
  const size_t rowgrp = frag / KB;             // b * N/16 + n16
  const int c = static_cast<int>(frag - rowgrp * KB);
  const size_t row = rowgrp * 16 + (l & 15);   // b * N + n
  const uint8_t* src = q + row * (static_cast<size_t>(KB) * 64) + c * 64 + (l >> 4) * 16;
  *reinterpret_cast<u32x4_t*>(out + t * 16) = *reinterpret_cast<const u32x4_t*>(src);
}

// e8m0 bytes -> their fp32 values 2^(b - 127) (exact).
__global__ __launch_bounds__(256) void e8m0_expand_kernel(const uint8_t* __restrict__ b, size_t n,
                                                          float* __restrict__ out) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    out[i] = ldexpf(1.0f, static_cast<int>(b[i]) - 127);
}

}  // namespace

hipError_t launch_quantize_act(const void* x, moe_dtype x_dtype, int M, int K,
                               const int32_t* row_index, uint8_t* q, void* scales, bool ue8m0,
                               hipStream_t stream) {
  const int G = K / kFp8Group;
  const long waves = static_cast<long>(M) * ((G + 3) / 4);
  dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
  const bool bf16 = x_dtype == MOE_BF16;
  if (bf16 && ue8m0)
    hipLaunchKernelGGL((quantize_act_kernel<uint16_t, true>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), M, K, row_index, q, scales);
  else if (bf16)
    hipLaunchKernelGGL((quantize_act_kernel<uint16_t, false>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), M, K, row_index, q, scales);
  else if (ue8m0)
    hipLaunchKernelGGL((quantize_act_kernel<float, true>), grid, block, 0, stream,
                       static_cast<const float*>(x), M, K, row_index, q, scales);
  else
    hipLaunchKernelGGL((quantize_act_kernel<float, false>), grid, block, 0, stream,
                       static_cast<const float*>(x), M, K, row_index, q, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_weight(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                                  uint8_t* q, void* scales, bool ue8m0, hipStream_t stream) {
  const long blocks = static_cast<long>(batch) * (N / kFp8Group) * (K / kFp8Group);
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const bool bf16 = w_dtype == MOE_BF16;
  if (bf16 && ue8m0)
    hipLaunchKernelGGL((quantize_weight_kernel<uint16_t, true>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(w), N, K, q, scales);
  else if (bf16)
    hipLaunchKernelGGL((quantize_weight_kernel<uint16_t, false>), grid, block, 0, stream,
                       static_cast<const uint16_t*>(w), N, K, q, scales);
  else if (ue8m0)
    hipLaunchKernelGGL((quantize_weight_kernel<float, true>), grid, block, 0, stream,
                       static_cast<const float*>(w), N, K, q, scales);
  else
    hipLaunchKernelGGL((quantize_weight_kernel<float, false>), grid, block, 0, stream,
                       static_cast<const float*>(w), N, K, q, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_weight_mx4(const void* w, moe_dtype w_dtype, size_t nblocks,
                                      uint8_t* q, uint8_t* scales, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((nblocks + 255) / 256)), block(256);
  if (w_dtype == MOE_BF16)
    hipLaunchKernelGGL(quantize_weight_mx4_kernel<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(w), nblocks, q, scales);
  else
    hipLaunchKernelGGL(quantize_weight_mx4_kernel<float>, grid, block, 0, stream,
                       static_cast<const float*>(w), nblocks, q, scales);
  return hipGetLastError();
}

hipError_t launch_tile_weight_fp4(const uint8_t* q, size_t rows, int K, uint8_t* out,
                                  hipStream_t stream) {
  const size_t nchunks = rows * (K / 32);   // 16-byte chunks (32 values each)
  hipLaunchKernelGGL(tile_weight_fp4_kernel, dim3(static_cast<unsigned>((nchunks + 255) / 256)),
                     dim3(256), 0, stream, q, nchunks, K / 128, out);
  return hipGetLastError();
}

hipError_t launch_e8m0_expand(const uint8_t* b, size_t n, float* out, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096));
  hipLaunchKernelGGL(e8m0_expand_kernel, dim3(blocks), dim3(256), 0, stream, b, n, out);
  return hipGetLastError();
}

}  // namespace moe
