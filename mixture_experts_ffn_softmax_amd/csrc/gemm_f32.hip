// fp32 grouped GEMMs (VALU, LDS-tiled) for layers kept in fp32 end to end, plus the device-side
// tile table shared by every grouped GEMM.
//
// Gate/up projection with the SwiGLU epilogue, and the down projection with the unpermute /
// weighting epilogue (Transformers "Experts backends" page: backends table rows grouped_mm,
// deepgemm_megamoe, sonicmoe; y = W_down (silu(W_gate x) * (W_up x))).
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// tile_cum_a / tile_cum_b: exclusive scans of ceil(M_e / bm_a) and ceil(M_e / bm_b).
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int bm_a, int bm_b,
                                                          int32_t* __restrict__ cum_a,
                                                          int32_t* __restrict__ cum_b) {
  __shared__ int sa[kMaxExperts], sb[kMaxExperts];
  const int e = threadIdx.x;
  int na = 0, nb = 0;
  if (e < E) {
    const int m = offsets[e + 1] - offsets[e];
    na = (m + bm_a - 1) / bm_a;
    nb = (m + bm_b - 1) / bm_b;
  }
  sa[e] = na;
  sb[e] = nb;
  __syncthreads();
  for (int o = 1; o < kMaxExperts; o <<= 1) {
    int va = e >= o ? sa[e - o] : 0, vb = e >= o ? sb[e - o] : 0;
    __syncthreads();
    sa[e] += va;
    sb[e] += vb;
    __syncthreads();
  }
  if (e < E) {
    cum_a[e + 1] = sa[e];
    cum_b[e + 1] = sb[e];
  }
  if (e == 0) {
    cum_a[0] = 0;
    cum_b[0] = 0;
  }
}

constexpr int kF32BM = 64;
constexpr int kF32BK = 16;
constexpr int kF32BN1 = 32;  // h columns per gate/up tile
constexpr int kF32BN2 = 64;  // output columns per down tile

// h[pos][n] = silu(sum_i a[pos][i] Wg[e][n][i]) * (sum_i a[pos][i] Wu[e][n][i]).
// Thread (ty, tx): rows ty*4..+4, h columns tx*2..+2.
__global__ __launch_bounds__(256) void gateup_f32_kernel(
    const float* __restrict__ a, int a_gather, const int32_t* __restrict__ sorted_pair, int k,
    const float* __restrict__ wg, const float* __restrict__ wu, int d, int f,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_cum, int E,
    float* __restrict__ h) {
  const int NT = (f + kF32BN1 - 1) / kF32BN1;
  TileCoord tc;
  if (!map_tile(tile_cum, offsets, E, kF32BM, NT, tc)) return;
  __shared__ float As[kF32BK][kF32BM + 1];
  __shared__ float Gs[kF32BK][kF32BN1 + 1];
  __shared__ float Us[kF32BK][kF32BN1 + 1];
  __shared__ int arow[kF32BM];
  const int tid = threadIdx.x;
  if (tid < kF32BM) {
    const int r = min(tid, tc.rows - 1);
    const int pos = tc.row0 + r;
    arow[tid] = a_gather ? sorted_pair[pos] / k : pos;
  }
  __syncthreads();
  const int n0 = tc.ntile * kF32BN1;
  const float* wgE = wg + static_cast<size_t>(tc.e) * f * d;
  const float* wuE = wu + static_cast<size_t>(tc.e) * f * d;
  const int ty = tid / 16, tx = tid % 16;
  float g[4][2] = {}, u[4][2] = {};
  for (int k0 = 0; k0 < d; k0 += kF32BK) {
    for (int q = tid; q < kF32BM * kF32BK; q += 256) {
      const int r = q / kF32BK, c = q % kF32BK;
      As[c][r] = (k0 + c < d) ? a[static_cast<size_t>(arow[r]) * d + k0 + c] : 0.0f;
    }
    for (int q = tid; q < kF32BN1 * kF32BK; q += 256) {
      const int r = q / kF32BK, c = q % kF32BK;
      const int n = min(n0 + r, f - 1);
      const bool ok = k0 + c < d;
      Gs[c][r] = ok ? wgE[static_cast<size_t>(n) * d + k0 + c] : 0.0f;
      Us[c][r] = ok ? wuE[static_cast<size_t>(n) * d + k0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kF32BK; ++c) {
      float av[4], gv[2], uv[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        gv[j] = Gs[c][tx * 2 + j];
        uv[j] = Us[c][tx * 2 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          g[i][j] = fmaf(av[i], gv[j], g[i][j]);
          u[i][j] = fmaf(av[i], uv[j], u[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= tc.rows) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + tx * 2 + j;
      if (n < f) {
        const float gg = g[i][j];
        h[static_cast<size_t>(tc.row0 + r) * f + n] = gg / (1.0f + expf(-gg)) * u[i][j];
      }
    }
  }
}

// y rows of the down projection, written in the requested layout.
__global__ __launch_bounds__(256) void down_f32_kernel(
    const float* __restrict__ h, const float* __restrict__ wd, int d, int f,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_cum, int E,
    const int32_t* __restrict__ sorted_pair, const float* __restrict__ topk_w, int k,
    int y_layout, float* __restrict__ y) {
  const int NT = (d + kF32BN2 - 1) / kF32BN2;
  TileCoord tc;
  if (!map_tile(tile_cum, offsets, E, kF32BM, NT, tc)) return;
  __shared__ float As[kF32BK][kF32BM + 1];
  __shared__ float Bs[kF32BK][kF32BN2 + 1];
  const int tid = threadIdx.x;
  const int n0 = tc.ntile * kF32BN2;
  const float* wdE = wd + static_cast<size_t>(tc.e) * d * f;
  const int ty = tid / 16, tx = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < f; k0 += kF32BK) {
    for (int q = tid; q < kF32BM * kF32BK; q += 256) {
      const int r = q / kF32BK, c = q % kF32BK;
      const int rr = min(r, tc.rows - 1);
      As[c][r] = (k0 + c < f) ? h[static_cast<size_t>(tc.row0 + rr) * f + k0 + c] : 0.0f;
    }
    for (int q = tid; q < kF32BN2 * kF32BK; q += 256) {
      const int r = q / kF32BK, c = q % kF32BK;
      const int n = min(n0 + r, d - 1);
      Bs[c][r] = (k0 + c < f) ? wdE[static_cast<size_t>(n) * f + k0 + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kF32BK; ++c) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[c][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= tc.rows) continue;
    const int pos = tc.row0 + r;
    const int pair = sorted_pair[pos];
    const float wgt = topk_w ? topk_w[pair] : 1.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= d) continue;
      if (y_layout == MOE_Y_PERMUTED)
        y[static_cast<size_t>(pos) * d + n] = acc[i][j];
      else if (y_layout == MOE_Y_SLOTS)
        y[static_cast<size_t>(pair) * d + n] = wgt * acc[i][j];
      else
        atomicAdd(&y[static_cast<size_t>(pair / k) * d + n], wgt * acc[i][j]);
    }
  }
}

inline unsigned grid_for(int P, int E, int BM, int NT) {
  long n = static_cast<long>(max_row_tiles(P, E, BM)) * NT;
  return static_cast<unsigned>((n + 7) / 8 * 8);
}

}  // namespace

hipError_t launch_tile_table(const int32_t* offsets, int E, int bm_a, int bm_b, int32_t* cum_a,
                             int32_t* cum_b, hipStream_t stream) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(kMaxExperts), 0, stream, offsets, E, bm_a,
                     bm_b, cum_a, cum_b);
  return hipGetLastError();
}

int f32_tile_rows() { return kF32BM; }

hipError_t launch_experts_f32(const ExpertsLaunch& L, hipStream_t stream) {
  const int P = L.T * L.k;
  const int NT1 = (L.f + kF32BN1 - 1) / kF32BN1;
  const int NT2 = (L.d + kF32BN2 - 1) / kF32BN2;
  float* h = static_cast<float*>(L.h);
  if (L.run_gate_up)
    hipLaunchKernelGGL(gateup_f32_kernel, dim3(grid_for(P, L.E, kF32BM, NT1)), dim3(256), 0, stream,
                     static_cast<const float*>(L.a), L.a_gather, L.sorted_pair, L.k,
                     static_cast<const float*>(L.w_gate), static_cast<const float*>(L.w_up), L.d,
                     L.f, L.offsets, L.tile_cum_a, L.E, h);
  if (L.run_down)
    hipLaunchKernelGGL(down_f32_kernel, dim3(grid_for(P, L.E, kF32BM, NT2)), dim3(256), 0, stream, h,
                     static_cast<const float*>(L.w_down), L.d, L.f, L.offsets, L.tile_cum_b, L.E,
                     L.sorted_pair, L.topk_w, L.k, L.y_layout, static_cast<float*>(L.y));
  return hipGetLastError();
}

}  // namespace moe
