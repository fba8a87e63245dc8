// Small-batch (decode) bf16 expert GEMMs: weight streaming with the large weight dimension on
// the matrix unit's M side.
//
// When only a few tokens reach each expert, putting tokens on the MFMA M side would leave most of
// the 16 or 32 rows empty. The AWS fused-MoE news page (sections on reordering the product for
// WGMMA and on swap-AB in MoE workloads) swaps the operands so that the expert-weight dimension
// fills the fixed-size side; the Transformers "Experts backends" page (decode-time switch) moves
// decoding to a kernel built for small token counts. Here: v_mfma_f32_16x16x32_bf16 with 16
// weight rows as A and 16 tokens as B; each weight byte is read exactly once per 64 tokens.
//
// Work split: one workgroup owns a panel of weight rows of one expert (gate/up: 32 gate rows and
// the matching 32 up rows; down: 64 rows) for all of that expert's tokens. Its 4 waves split K in
// 128-element chunks (chunk c goes to wave c % 4) and reduce through LDS. Within a chunk lane
// (r = l % 16, g = l / 16) loads 64 contiguous bytes (k = 32 g .. 32 g + 31) of its row, and the
// four MFMAs of the chunk take 8 of those elements each; the token operand uses the same k
// assignment, so every product pairs matching k.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kDecodeGateRows = 32;   // gate rows (and as many up rows) per gate/up workgroup
constexpr int kDecodeDownRows = 64;   // W_down rows per down workgroup
constexpr int kDecodeTokens = 64;     // tokens per pass (4 groups of 16)
constexpr int kGateUp = 0;
constexpr int kDown = 1;

struct DecodeArgs {
  const uint16_t* a;          // gate/up: x [T, K] (gather) ; down: h [P, K]
  int a_gather;
  const int32_t* sorted_pair;
  int k;
  const uint16_t* w0;         // W_gate or W_down [E, N, K]
  const uint16_t* w1;         // W_up
  int K, N;
  const int32_t* offsets;
  uint16_t* h;
  void* y;
  int y_layout, y_bf16;
  const float* topk_w;
};

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int MODE>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeArgs p) {
  constexpr int kRows = MODE == kGateUp ? kDecodeGateRows : kDecodeDownRows;
  const int nrb = (p.N + kRows - 1) / kRows;
  const int e = blockIdx.x / nrb;
  const int rb = blockIdx.x - e * nrb;
  const int row0 = p.offsets[e];
  const int M = p.offsets[e + 1] - row0;
  if (M == 0) return;

  __shared__ f32x4_t red[4][4][4][64];  // [wave][row group][token group][lane], 64 KB

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const size_t wstride = static_cast<size_t>(p.N) * p.K;

  // A rows: 4 groups of 16 weight rows.
  const uint16_t* arow[4];
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    int n;
    const uint16_t* base;
    if (MODE == kGateUp) {
      n = rb * kRows + (rg & 1) * 16 + r16;
      base = (rg < 2 ? p.w0 : p.w1) + e * wstride;
    } else {
      n = rb * kRows + rg * 16 + r16;
      base = p.w0 + e * wstride;
    }
    arow[rg] = base + static_cast<size_t>(min(n, p.N - 1)) * p.K + g * 32;
  }
  const int nchunks = p.K / 128;

  for (int tc0 = 0; tc0 < M; tc0 += kDecodeTokens) {
    const int ntg = min(4, (M - tc0 + 15) / 16);
    const uint16_t* brow[4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int ti = min(tc0 + tg * 16 + r16, M - 1);
      const int pos = row0 + ti;
      const int src = p.a_gather ? p.sorted_pair[pos] / p.k : pos;
      brow[tg] = p.a + static_cast<size_t>(src) * p.K + g * 32;
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int c = wave; c < nchunks; c += 4) {
      const int kb = c * 128;
      u32x4_t av[4][4], bv[4][4];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
#pragma unroll
        for (int u = 0; u < 4; ++u) av[rg][u] = ld16(arow[rg] + kb + u * 8);
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
        if (tg < ntg)
#pragma unroll
          for (int u = 0; u < 4; ++u) bv[tg][u] = ld16(brow[tg] + kb + u * 8);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
          if (tg < ntg)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
              acc[rg][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  as_bf16x8(av[rg][u]), as_bf16x8(bv[tg][u]), acc[rg][tg], 0, 0, 0);
    }

#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) red[wave][rg][tg][lane] = acc[rg][tg];
    __syncthreads();

    // Wave w finishes token group w. Output layout of a 16x16 block: lane l holds token l % 16
    // and weight rows 4 * (l / 16) + i, i = 0..3.
    const int tg = wave;
    const int ti = tc0 + tg * 16 + r16;
    if (tg < ntg && ti < M) {
      f32x4_t s[4];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        s[rg] = red[0][rg][tg][lane] + red[1][rg][tg][lane] + red[2][rg][tg][lane] +
                red[3][rg][tg][lane];
      const int pos = row0 + ti;
      if (MODE == kGateUp) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int n = rb * kRows + half * 16 + 4 * g;
          if (n < p.N) {
            u32x2_t o;
            o[0] = f32_to_bf16_bits(silu_mul(s[half][0], s[half + 2][0])) |
                   (static_cast<uint32_t>(f32_to_bf16_bits(silu_mul(s[half][1], s[half + 2][1]))) << 16);
            o[1] = f32_to_bf16_bits(silu_mul(s[half][2], s[half + 2][2])) |
                   (static_cast<uint32_t>(f32_to_bf16_bits(silu_mul(s[half][3], s[half + 2][3]))) << 16);
            *reinterpret_cast<u32x2_t*>(p.h + static_cast<size_t>(pos) * p.N + n) = o;
          }
        }
      } else {
        const int pair = p.sorted_pair[pos];
        const float wgt = p.topk_w ? p.topk_w[pair] : 1.0f;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = rb * kRows + rg * 16 + 4 * g;
          if (n >= p.N) continue;
          f32x4_t v = s[rg];
          if (p.y_layout == MOE_Y_ACC_F32) {
            float* dst = static_cast<float*>(p.y) + static_cast<size_t>(pair / p.k) * p.N + n;
#pragma unroll
            for (int i = 0; i < 4; ++i) atomicAdd(dst + i, wgt * v[i]);
            continue;
          }
          size_t idx;
          if (p.y_layout == MOE_Y_PERMUTED) {
            idx = static_cast<size_t>(pos) * p.N + n;
          } else {
            idx = static_cast<size_t>(pair) * p.N + n;
            v = v * wgt;
          }
          if (p.y_bf16) {
            u32x2_t o;
            o[0] = f32_to_bf16_bits(v[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
            o[1] = f32_to_bf16_bits(v[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.y) + idx) = o;
          } else {
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(p.y) + idx) = v;
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

int decode_tile_rows() { return 64; }  // unused by the decode kernels; keeps the tile table valid

hipError_t launch_experts_bf16_decode(const ExpertsLaunch& L, hipStream_t stream) {
  DecodeArgs g{};
  g.a = static_cast<const uint16_t*>(L.a);
  g.a_gather = L.a_gather;
  g.sorted_pair = L.sorted_pair;
  g.k = L.k;
  g.w0 = static_cast<const uint16_t*>(L.w_gate);
  g.w1 = static_cast<const uint16_t*>(L.w_up);
  g.K = L.d;
  g.N = L.f;
  g.offsets = L.offsets;
  g.h = static_cast<uint16_t*>(L.h);
  const unsigned grid1 = static_cast<unsigned>(L.E) * ((L.f + kDecodeGateRows - 1) / kDecodeGateRows);
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[0]), stream);
  hipLaunchKernelGGL(decode_bf16_kernel<kGateUp>, dim3(grid1), dim3(256), 0, stream, g);
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[1]), stream);

  DecodeArgs dn{};
  dn.a = static_cast<const uint16_t*>(L.h);
  dn.a_gather = 0;
  dn.sorted_pair = L.sorted_pair;
  dn.k = L.k;
  dn.w0 = static_cast<const uint16_t*>(L.w_down);
  dn.K = L.f;
  dn.N = L.d;
  dn.offsets = L.offsets;
  dn.y = L.y;
  dn.y_layout = L.y_layout;
  dn.y_bf16 = L.y_bf16;
  dn.topk_w = L.topk_w;
  const unsigned grid2 = static_cast<unsigned>(L.E) * ((L.d + kDecodeDownRows - 1) / kDecodeDownRows);
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[2]), stream);
  hipLaunchKernelGGL(decode_bf16_kernel<kDown>, dim3(grid2), dim3(256), 0, stream, dn);
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[3]), stream);
  return hipGetLastError();
}

}  // namespace moe
