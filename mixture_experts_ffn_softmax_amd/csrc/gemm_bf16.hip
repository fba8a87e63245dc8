// bf16 grouped GEMMs on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Gate/up projection fused with SwiGLU, then the down projection with the unpermute / routing
// weight epilogue (Transformers "Experts backends" page, backends table rows grouped_mm,
// deepgemm_megamoe and sonicmoe: tokens grouped by expert, one grouped GEMM, gated MLP with
// SwiGLU). The rows of both GEMMs are the expert-sorted pairs; the gate/up GEMM reads each pair's
// token row straight from x (gather on load), so no permuted copy of x is needed.
//
// Tiling: 256 x 256 output tile per workgroup, K staged 64 at a time through LDS (double
// buffered, 2 x 64 KB). Four waves each own a 128 x 128 quadrant = 4 x 4 MFMA 32x32 blocks, so
// every A fragment read from LDS feeds 4 MFMAs and every B fragment 4 MFMAs. LDS rows are 128 B;
// the 16-byte chunk c of row r is stored at chunk position c ^ (r & 7), which makes both the
// row-wise stores and the MFMA fragment reads (32 rows x one chunk) bank-conflict free.
// For the gate/up GEMM the 256 B-rows of a tile are 128 gate rows and the same 128 up rows, so
// each wave holds matching gate and up accumulators and applies SwiGLU in registers.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kTileElems = kBM * kBK;   // bf16 elements per operand tile
constexpr int kGateUp = 0;
constexpr int kDown = 1;

struct Bf16GemmArgs {
  const uint16_t* a;          // gate/up: x [T, K] or x_perm [P, K]; down: h [P, K]
  int a_gather;
  const int32_t* sorted_pair;
  int k;                      // experts per token
  const uint16_t* b0;         // gate/up: W_gate [E, N, K]; down: W_down [E, N, K]
  const uint16_t* b1;         // gate/up: W_up [E, N, K]
  int K, N;
  const int32_t* offsets;
  const int32_t* tile_cum;
  int E;
  uint16_t* h;                // gate/up output [P, N]
  void* y;                    // down output
  int y_layout, y_bf16;
  const float* topk_w;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

// Loads the thread's 8 A chunks and 8 B chunks (16 bytes each) of one K slice; B rows 0..127 of
// the tile (i < 4) come from b0, rows 128..255 from b1.
__device__ __forceinline__ void gload8(u32x4_t (&ra)[8], u32x4_t (&rb)[8], const char* abase,
                                       const char* b0base, const char* b1base,
                                       const uint32_t (&aoff)[8], const uint32_t (&boff)[8],
                                       uint32_t kbytes) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ra[i] = *reinterpret_cast<const u32x4_t*>(abase + aoff[i] + kbytes);
    rb[i] = *reinterpret_cast<const u32x4_t*>((i < 4 ? b0base : b1base) + boff[i] + kbytes);
  }
}

__device__ __forceinline__ u32x2_t pack_bf16x4(float4 v) {
  u32x2_t o;
  o[0] = f32_to_bf16_bits(v.x) | (static_cast<uint32_t>(f32_to_bf16_bits(v.y)) << 16);
  o[1] = f32_to_bf16_bits(v.z) | (static_cast<uint32_t>(f32_to_bf16_bits(v.w)) << 16);
  return o;
}

__device__ __forceinline__ void lstore8(uint16_t* buf, const u32x4_t (&ra)[8], const u32x4_t (&rb)[8],
                                        const uint32_t (&soff)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    *reinterpret_cast<u32x4_t*>(buf + soff[i]) = ra[i];
    *reinterpret_cast<u32x4_t*>(buf + kTileElems + soff[i]) = rb[i];
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(Bf16GemmArgs p) {
  const int NT = MODE == kGateUp ? (p.N + 127) / 128 : (p.N + kBN - 1) / kBN;
  TileCoord tc;
  if (!map_tile(p.tile_cum, p.offsets, p.E, kBM, NT, tc)) return;

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * kTileElems];
  __shared__ int row_pair[kBM];
  __shared__ float row_w[kBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  if (MODE == kDown) {
    const int rr = min(tid, tc.rows - 1);
    const int pair = p.sorted_pair[tc.row0 + rr];
    row_pair[tid] = pair;
    row_w[tid] = p.topk_w ? p.topk_w[pair] : 1.0f;
  }

  // Global -> register -> LDS staging: thread covers rows i*32 + tid/8 (i = 0..7), 16-byte chunk
  // tid%8 of the 128-byte K slice. Addresses are 32-bit byte offsets from uniform bases.
  const int lrow = tid >> 3, lch = tid & 7;
  const char* abase = reinterpret_cast<const char*>(p.a);
  const size_t wstride = static_cast<size_t>(p.N) * p.K;
  const char* b0base = reinterpret_cast<const char*>(p.b0 + tc.e * wstride);
  const char* b1base = MODE == kGateUp ? reinterpret_cast<const char*>(p.b1 + tc.e * wstride)
                                       : b0base;
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = i * 32 + lrow;
    const int pos = tc.row0 + min(r, tc.rows - 1);
    const int arow = p.a_gather ? p.sorted_pair[pos] / p.k : pos;
    aoff[i] = (static_cast<uint32_t>(arow) * p.K + lch * 8) * 2u;
    const int n = MODE == kGateUp ? min(tc.ntile * 128 + (r & 127), p.N - 1)
                                  : min(tc.ntile * kBN + r, p.N - 1);
    boff[i] = (static_cast<uint32_t>(n) * p.K + lch * 8) * 2u;
  }
  uint32_t soff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) soff[i] = swz(i * 32 + lrow, lch);

  u32x4_t ra[8], rb[8];

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nst = p.K / kBK;
  gload8(ra, rb, abase, b0base, b1base, aoff, boff, 0u);
  lstore8(smem, ra, rb, soff);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    if (s + 1 < nst) {
      const uint32_t kb = static_cast<uint32_t>(s + 1) * kBK * 2u;
      gload8(ra, rb, abase, b0base, b1base, aoff, boff, kb);
    }
    const uint16_t* As = smem + buf * 2 * kTileElems;
    const uint16_t* Bs = As + kTileElems;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + swz(wm * 128 + i * 32 + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int brow = MODE == kGateUp
                             ? ((j < 2) ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32)
                             : wn * 128 + j * 32;
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + swz(brow + (lane & 31), ch));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nst) lstore8(smem + (buf ^ 1) * 2 * kTileElems, ra, rb, soff);
    __syncthreads();
  }

  // Accumulator layout of a 32x32 block: lane l holds column l % 32 and rows
  // 8 * (r / 4) + 4 * (l / 32) + r % 4 for r = 0..15. Results go through LDS so that global
  // stores are whole 16-byte row segments.
  if (MODE == kGateUp) {
    // h tile [256 rows][128 cols] bf16, row stride 136 elements.
    constexpr int kHS = 136;
    uint16_t* hs = smem;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = wn * 64 + j * 32 + (lane & 31);
          hs[row * kHS + col] = f32_to_bf16_bits(silu_mul(acc[i][j][r], acc[i][j + 2][r]));
        }
    __syncthreads();
    const int n0 = tc.ntile * 128;
    for (int it = 0; it < 16; ++it) {
      const int q = it * 256 + tid;
      const int row = q >> 4, ch = q & 15;
      if (row < tc.rows && n0 + ch * 8 < p.N)
        *reinterpret_cast<u32x4_t*>(p.h + static_cast<size_t>(tc.row0 + row) * p.N + n0 + ch * 8) =
            *reinterpret_cast<const u32x4_t*>(hs + row * kHS + ch * 8);
    }
  } else {
    // Four passes of 64 rows staged as fp32 [64][260].
    constexpr int kYS = 260;
    float* ys = reinterpret_cast<float*>(smem);
    const int n0 = tc.ntile * kBN;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (wm == (q >> 1)) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * (q & 1) + ii;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = ii * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
              const int col = wn * 128 + j * 32 + (lane & 31);
              ys[row * kYS + col] = acc[i][j][r];
            }
        }
      }
      __syncthreads();
      for (int it = 0; it < 16; ++it) {
        const int e = it * 256 + tid;
        const int rl = e >> 6, c4 = (e & 63) * 4;
        const int row = q * 64 + rl;
        const int col = n0 + c4;
        if (row < tc.rows && col < p.N) {
          float4 v = *reinterpret_cast<const float4*>(ys + rl * kYS + c4);
          if (p.y_layout == MOE_Y_PERMUTED) {
            const size_t idx = static_cast<size_t>(tc.row0 + row) * p.N + col;
            if (p.y_bf16) {
              u32x2_t o = pack_bf16x4(v);
              *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.y) + idx) = o;
            } else {
              *reinterpret_cast<float4*>(static_cast<float*>(p.y) + idx) = v;
            }
          } else {
            const float wgt = row_w[row];
            v.x *= wgt; v.y *= wgt; v.z *= wgt; v.w *= wgt;
            const int pair = row_pair[row];
            if (p.y_layout == MOE_Y_SLOTS) {
              const size_t idx = static_cast<size_t>(pair) * p.N + col;
              if (p.y_bf16) {
                u32x2_t o = pack_bf16x4(v);
                *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.y) + idx) = o;
              } else {
                *reinterpret_cast<float4*>(static_cast<float*>(p.y) + idx) = v;
              }
            } else {
              float* dst = static_cast<float*>(p.y) + static_cast<size_t>(pair / p.k) * p.N + col;
              atomicAdd(dst + 0, v.x);
              atomicAdd(dst + 1, v.y);
              atomicAdd(dst + 2, v.z);
              atomicAdd(dst + 3, v.w);
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

inline unsigned grid_for(int P, int E, int NT) {
  long n = static_cast<long>(max_row_tiles(P, E, kBM)) * NT;
  return static_cast<unsigned>((n + 7) / 8 * 8);
}

}  // namespace

int bf16_tile_rows_gateup() { return kBM; }
int bf16_tile_rows_down() { return kBM; }

hipError_t launch_experts_bf16(const ExpertsLaunch& L, hipStream_t stream) {
  const int P = L.T * L.k;
  Bf16GemmArgs g{};
  g.a = static_cast<const uint16_t*>(L.a);
  g.a_gather = L.a_gather;
  g.sorted_pair = L.sorted_pair;
  g.k = L.k;
  g.b0 = static_cast<const uint16_t*>(L.w_gate);
  g.b1 = static_cast<const uint16_t*>(L.w_up);
  g.K = L.d;
  g.N = L.f;
  g.offsets = L.offsets;
  g.tile_cum = L.tile_cum_a;
  g.E = L.E;
  g.h = static_cast<uint16_t*>(L.h);
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[0]), stream);
  hipLaunchKernelGGL(gemm_bf16_kernel<kGateUp>, dim3(grid_for(P, L.E, (L.f + 127) / 128)),
                     dim3(256), 0, stream, g);
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[1]), stream);

  Bf16GemmArgs dn{};
  dn.a = static_cast<const uint16_t*>(L.h);
  dn.a_gather = 0;
  dn.sorted_pair = L.sorted_pair;
  dn.k = L.k;
  dn.b0 = static_cast<const uint16_t*>(L.w_down);
  dn.K = L.f;
  dn.N = L.d;
  dn.offsets = L.offsets;
  dn.tile_cum = L.tile_cum_b;
  dn.E = L.E;
  dn.y = L.y;
  dn.y_layout = L.y_layout;
  dn.y_bf16 = L.y_bf16;
  dn.topk_w = L.topk_w;
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[2]), stream);
  hipLaunchKernelGGL(gemm_bf16_kernel<kDown>, dim3(grid_for(P, L.E, (L.d + kBN - 1) / kBN)),
                     dim3(256), 0, stream, dn);
  if (L.ev) hipEventRecord(static_cast<hipEvent_t>(L.ev[3]), stream);
  return hipGetLastError();
}

}  // namespace moe
