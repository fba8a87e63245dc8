// Small-batch (decode) fine-grained FP8 expert GEMMs: e4m3 weight streaming with the weight rows
// on the matrix unit's M side.
//
// The swap-AB idea of the bf16 decode kernels (AWS fused-MoE news page, sections on reordering the
// product for WGMMA and on swap-AB in MoE workloads; Transformers "Experts backends" page,
// decode-time switch to a small-batch kernel) with the e4m3 operands of the Transformers
// "Fine-grained FP8" page: weights in 128x128 blocks with one scale each, activations per token
// per 128 channels. One v_mfma_scale_f32_16x16x128_f8f6f4 takes 16 weight rows (A) and 16 tokens
// (B) over one 128-wide K block, i.e. exactly one weight scale per row group and one activation
// scale per token. With fp32 scales its result is promoted by w_scale * x_scale; with UE8M0
// scales (same page, "UE8M0 scale format") the bytes go to the instruction, which accumulates
// across K blocks. The streamed weight bytes are half those of the bf16 kernels.
//
// Work split as in the bf16 K-split kernel: a workgroup owns 64 weight rows of one expert (gate/up:
// 32 gate rows and the matching 32 up rows; down: 64 rows) for all of that expert's tokens, in
// passes of 64 tokens; its 4 waves take the 128-wide K blocks in turn and reduce through LDS. The
// gate/up kernel writes h in fp32, since one 128-channel group of h spans four workgroups; the
// caller quantises it per (pair, 128 channels) before the down kernel.
//
// FP4 experts (Transformers "Experts backends" page, notes on FP4 quantised experts; "Fine-grained
// FP8" page, "UE8M0 scale format"): weights E2M1, two per byte, with one e8m0 scale per row per 32
// input channels, against the same e4m3 activations. The instruction takes its A operand as FP4
// (format code 4: 32 values in the low four registers of each lane) and a scale per lane. Within
// one 128-wide K block, lane group g (lanes 16g..16g+15) holds K = 32g..32g+31 of an FP4 operand,
// but of an 8-bit operand K = 16g..16g+15 in its first 16 bytes and 64+16g..64+16g+15 in its last
// 16 (measured on gfx950); a lane's scale covers K = 32g..32g+31 in both. So each lane passes its
// own weight block's byte, and the e4m3 activations are fetched as the two 16-byte pieces that
// line up with the FP4 weights. The e4m3 weights are fetched the same way: then the four lanes of a
// row read one contiguous 64-byte piece per load. The E2M1 weights come in matrix-fragment order
// (each 16-row, 128-wide block is the 1 KB one load reads, lane by lane), which streams markedly
// faster than 16 scattered row pieces. Half the streamed bytes of the fp8 weights.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kFdGateRows = 32;   // gate rows (and as many up rows) per gate/up workgroup
constexpr int kFdDownRows = 64;   // W_down rows per down workgroup
constexpr int kGateUp = 0;
constexpr int kDown = 1;

struct Fp8DecodeArgs {
  const uint8_t* a;           // gate/up: x codes [T, K] (gathered); down: h codes [P, K]
  const void* a_s;            // activation scales [rows, K/128]: fp32, or e8m0 bytes (UE8M0)
  int a_gather;
  const int32_t* sorted_pair;
  int k;
  const uint8_t* w0;          // W_gate or W_down [E, N, K] e4m3, or [E, N, K/2] packed E2M1
  const uint8_t* w1;          // W_up
  const void* s0;             // block scales of w0 [E, N/128, K/128]: fp32, or e8m0 bytes;
                              // E2M1: e8m0 bytes [E, N, K/32]
  const void* s1;
  int K, N;
  const int32_t* offsets;
  float* h32;                 // gate/up output h [P, N] fp32
  void* y;                    // down output
  int y_layout, y_bf16;
  const float* topk_w;
  // fused small-batch path (see ExpertsLaunch): routing ids [P]
  const int32_t* ids;
  int P;
};

__device__ __forceinline__ i32x8_t ld16x2g(const uint8_t* p, const uint8_t* q) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(q);
  i32x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

__device__ __forceinline__ i32x8_t ld16g(const uint8_t* p) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p);
  i32x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// 2^(b - 127) as fp32 bits (b = 0 is the subnormal 2^-127): an e8m0 byte turned into the fp32 scale
// it stands for, exactly.
__device__ __forceinline__ uint32_t e8m0_f32_bits(uint32_t b) { return b ? b << 23 : 0x00400000u; }

// kW4: E2M1 weights with per-32 MX scales (implies kUE). kTG: groups of 16 tokens per pass over
// the weights (fewer groups hold fewer registers and less LDS, so more waves stream at once).
// kFused: the fused small-batch path (pairs from the routing ids; h and slots indexed by pair).
template <int MODE, bool kUE, bool kW4, int kTG, bool kFused>
__global__ __launch_bounds__(256) void decode_fp8_kernel(Fp8DecodeArgs p) {
  constexpr int kRows = MODE == kGateUp ? kFdGateRows : kFdDownRows;
  constexpr int kTokens = 16 * kTG;
  const int nrb = (p.N + kRows - 1) / kRows;
  const int e = blockIdx.x / nrb;
  const int rb = blockIdx.x - e * nrb;
  __shared__ int32_t plist[kFused ? kFusedMaxPairs : 1];   // fused: this expert's pairs
  __shared__ int wsum[4];
  int row0, M;
  if constexpr (kFused) {
    row0 = 0;
    M = expert_pair_list<256, kFusedMaxPairs>(p.ids, p.P, e, plist, wsum);
  } else {
    row0 = p.offsets[e];
    M = p.offsets[e + 1] - row0;
  }
  if (M <= 0) return;
  // i-th token row of this expert: its h / slot row (pos) and its pair (t * k + j)
  auto pos_of = [&](int i) { return kFused ? plist[i] : row0 + i; };
  auto pair_of = [&](int i) { return kFused ? plist[i] : p.sorted_pair[row0 + i]; };

  __shared__ f32x4_t red[4][4][kTG][64];  // [wave][row group][token group][lane], 16 KB each
  // Weight scales for every K block, staged once: 128x128 blocks, one per row group (fp32 bits
  // or the e8m0 byte), or for E2M1 the MX bytes of all 64 rows (dynamic, below). Loads of them
  // in the K loop would cost the texture-address unit about as much as the weight stream.
  __shared__ uint32_t wss[4][256];
  // Where UE8M0 scales are applied: E2M1 weights always pass them to the instruction (the
  // per-32 weight scales cannot be taken out of a 128-wide block's sum); e4m3 weights with one
  // token group scale each block's product afterwards, which saves the scale-operand load ahead
  // of every scaled MFMA and was measured faster with one group, slower with two or four.
  constexpr bool kScaleInMfma = kW4 || (kUE && kTG > 1);
  extern __shared__ uint32_t wsx[];   // E2M1: [64 rows][KB | 1 dwords]: byte 4c+g = block (c, g)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int rowb = kW4 ? p.K / 2 : p.K;   // bytes per weight row
  const size_t wstride = static_cast<size_t>(p.N) * rowb;
  const int KB = p.K / 128, NB = p.N / 128;

  // A rows (4 groups of 16 weight rows); a group lies inside one 128-row scale block.
  const uint8_t* arow[4];
  const void* ascale[4];   // 128x128 scales: this expert's scale row of the group's row block
#pragma unroll
  for (int rg = 0; rg < 4; ++rg) {
    int n;
    const uint8_t* base;
    const void* sbase;
    if (MODE == kGateUp) {
      n = rb * kRows + (rg & 1) * 16;
      base = (rg < 2 ? p.w0 : p.w1) + e * wstride;
      sbase = rg < 2 ? p.s0 : p.s1;
    } else {
      n = rb * kRows + rg * 16;
      base = p.w0 + e * wstride;
      sbase = p.s0;
    }
    const int row = min(n + r16, p.N - 1);
    if constexpr (kW4) {
      // fragment order: the 16 rows' 128-wide K block c is 1 KB at (n / 16 * KB + c) * 1 KB
      ascale[rg] = nullptr;   // MX scales: staged per row below
      arow[rg] = base + static_cast<size_t>(n / 16) * KB * 1024 + lane * 16;
    } else {
      const int nb = min(n, p.N - 1) / 128;
      const size_t sidx = (static_cast<size_t>(e) * NB + nb) * KB;
      ascale[rg] = kUE ? static_cast<const void*>(static_cast<const uint8_t*>(sbase) + sidx)
                       : static_cast<const void*>(static_cast<const float*>(sbase) + sidx);
      arow[rg] = base + static_cast<size_t>(row) * rowb + g * 16;
    }
  }
  const int S = KB | 1;   // odd dword stride: the 16 rows a load touches sit in distinct banks
  if constexpr (kW4) {
    for (int i = tid; i < 64 * KB; i += 256) {
      const int lr = i / KB, j = i - lr * KB;   // LDS row rg * 16 + r, dword j of the row
      const int rg = lr >> 4;
      const int n = MODE == kGateUp ? rb * kRows + (rg & 1) * 16 + (lr & 15) : rb * kRows + lr;
      const void* sb = (MODE == kGateUp && rg >= 2) ? p.s1 : p.s0;
      const uint8_t* src = static_cast<const uint8_t*>(sb) +
                           (static_cast<size_t>(e) * p.N + min(n, p.N - 1)) * (p.K / 32);
      wsx[lr * S + j] = reinterpret_cast<const uint32_t*>(src)[j];
    }
  } else {
    for (int i = tid; i < 4 * KB; i += 256) {
      const int rg = i / KB, c = i - rg * KB;
      const uint32_t b = kUE ? static_cast<const uint8_t*>(ascale[rg])[c] : 0u;
      wss[rg][c] = kScaleInMfma ? b
                   : kUE ? e8m0_f32_bits(b)
                   : __float_as_uint(static_cast<const float*>(ascale[rg])[c]);
    }
  }
  __syncthreads();
  // E2M1: this lane's scale bytes, row rg * 16 + r16, block g of K block c at + 4c
  const uint8_t* wsl = reinterpret_cast<const uint8_t*>(wsx) + r16 * S * 4 + g;

  for (int tc0 = 0; tc0 < M; tc0 += kTokens) {
    const int ntg = min(kTG, (M - tc0 + 15) / 16);
    const uint8_t* brow[kTG];
    size_t bscale[kTG];   // index of the token's first scale
#pragma unroll
    for (int tg = 0; tg < kTG; ++tg) {
      const int ti = min(tc0 + tg * 16 + r16, M - 1);
      const int pos = pos_of(ti);
      const int src = p.a_gather ? pair_of(ti) / p.k : pos;
      brow[tg] = p.a + static_cast<size_t>(src) * p.K + g * 16;
      bscale[tg] = static_cast<size_t>(src) * KB;
    }
    f32x4_t acc[4][kTG];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg) acc[rg][tg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int c = wave; c < KB; c += 4) {
      const int kb = c * 128;
      i32x8_t av[4], bv[kTG];
      float bs[kTG];    // fp32 scales
      int bx[kTG];      // UE8M0: e8m0 bytes
      int ewl[4];   // E2M1: each lane's own block scale byte
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        if constexpr (kW4) {
          av[rg] = ld16g(arow[rg] + c * 1024);
          ewl[rg] = wsl[rg * 16 * S * 4 + c * 4];
        } else {
          av[rg] = ld16x2g(arow[rg] + kb, arow[rg] + kb + 64);
        }
      }
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg)
        if (tg < ntg) {
          bv[tg] = ld16x2g(brow[tg] + kb, brow[tg] + kb + 64);
          if constexpr (kScaleInMfma)
            bx[tg] = static_cast<const uint8_t*>(p.a_s)[bscale[tg] + c];
          else if constexpr (kUE)
            bs[tg] = __uint_as_float(e8m0_f32_bits(static_cast<const uint8_t*>(p.a_s)[bscale[tg] + c]));
          else
            bs[tg] = static_cast<const float*>(p.a_s)[bscale[tg] + c];
        }
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg) {
        if (tg >= ntg) continue;
        if constexpr (kScaleInMfma) {
          // the weight byte (each lane's MX byte for E2M1) and the token's e8m0 byte go to the
          // instruction. Each block's product starts from zero and is added afterwards: with a
          // token group or two the few accumulators would otherwise chain every MFMA to the
          // previous K block's.
          const int ex = bx[tg];
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int ew = kW4 ? ewl[rg] : static_cast<int>(wss[rg][c]);
            acc[rg][tg] += __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                av[rg], bv[tg], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, kW4 ? 4 : 0, 0, 0, ew, 0, ex);
          }
        } else {
          // one weight scale per 128x128 block and one activation scale per token and block:
          // the block's product is scaled after the instruction. UE8M0 scales are powers of
          // two, so while their product stays above 2^-149 this rounds exactly as the
          // instruction's own scaling would.
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const float sc = __uint_as_float(wss[rg][c]) * bs[tg];
            const f32x4_t part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                av[rg], bv[tg], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[rg][tg][q] = fmaf(part[q], sc, acc[rg][tg][q]);
          }
        }
      }
    }

#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int tg = 0; tg < kTG; ++tg) red[wave][rg][tg][lane] = acc[rg][tg];
    __syncthreads();

    // Wave w finishes token group w. Output layout of a 16x16 block: lane l holds token l % 16
    // and weight rows 4 * (l / 16) + i, i = 0..3.
    const int tg = wave;
    const int ti = tc0 + tg * 16 + r16;
    if (tg < ntg && ti < M) {   // ntg <= kTG: red is indexed in bounds
      f32x4_t s[4];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        s[rg] = red[0][rg][tg][lane] + red[1][rg][tg][lane] + red[2][rg][tg][lane] +
                red[3][rg][tg][lane];
      const int pos = pos_of(ti);
      if (MODE == kGateUp) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int n = rb * kRows + half * 16 + 4 * g;
          if (n < p.N) {
            f32x4_t hv;
#pragma unroll
            for (int i = 0; i < 4; ++i) hv[i] = silu_mul(s[half][i], s[half + 2][i]);
            *reinterpret_cast<f32x4_t*>(p.h32 + static_cast<size_t>(pos) * p.N + n) = hv;
          }
        }
      } else {
        const int pair = pair_of(ti);
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

template <int MODE, int kTG, bool kF>
void launch_tg(const Fp8DecodeArgs& a, dim3 grid, bool ue, bool w4, hipStream_t stream) {
  // E2M1: the 64 rows' MX scale bytes, rows padded to an odd number of dwords
  const unsigned mx_lds = static_cast<unsigned>(64 * ((a.K / 128) | 1) * 4);
  if (w4) hipLaunchKernelGGL((decode_fp8_kernel<MODE, true, true, kTG, kF>), grid, dim3(256),
                             mx_lds, stream, a);
  else if (ue) hipLaunchKernelGGL((decode_fp8_kernel<MODE, true, false, kTG, kF>), grid,
                                  dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((decode_fp8_kernel<MODE, false, false, kTG, kF>), grid, dim3(256), 0,
                          stream, a);
}

// Token groups per pass from the mean pairs per expert: a pass holds a typical expert's tokens
// with room for the spread; an expert with more makes further passes over its weights.
inline int token_groups(int P, int E) {
  const int mean = (P + E - 1) / E;
  return mean <= 8 ? 1 : (mean <= 24 ? 2 : 4);
}

template <int MODE, bool kF>
hipError_t launch_one(const Fp8DecodeArgs& a, int E, int P, bool ue, bool w4, hipStream_t stream) {
  constexpr int kRows = MODE == kGateUp ? kFdGateRows : kFdDownRows;
  const dim3 grid(static_cast<unsigned>(E * ((a.N + kRows - 1) / kRows)));
  const int tg = token_groups(P, E);
  if (tg == 1) launch_tg<MODE, 1, kF>(a, grid, ue, w4, stream);
  else if (tg == 2) launch_tg<MODE, 2, kF>(a, grid, ue, w4, stream);
  else launch_tg<MODE, 4, kF>(a, grid, ue, w4, stream);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const Fp8DecodeArgs& a, int E, int P, bool ue, bool w4, bool fused,
                       hipStream_t stream) {
  return fused ? launch_one<MODE, true>(a, E, P, ue, w4, stream)
               : launch_one<MODE, false>(a, E, P, ue, w4, stream);
}

}  // namespace

hipError_t launch_experts_fp8_decode(const ExpertsLaunch& L, hipStream_t stream) {
  const int P = L.T * L.k;
  const bool ue = L.scale_ue8m0 != 0;
  Fp8DecodeArgs g{};
  g.a = static_cast<const uint8_t*>(L.a);
  g.a_s = ue ? L.a_scale_bytes : static_cast<const void*>(L.a_scales);
  g.a_gather = L.a_gather;
  g.sorted_pair = L.sorted_pair;
  g.k = L.k;
  g.w0 = static_cast<const uint8_t*>(L.w_gate);
  g.w1 = static_cast<const uint8_t*>(L.w_up);
  g.s0 = L.s_gate;
  g.s1 = L.s_up;
  g.K = L.d;
  g.N = L.f;
  g.offsets = L.offsets;
  g.h32 = L.h32;
  const bool w4 = L.w_fp4 != 0;
  const bool fused = L.pair_ids != nullptr;
  if (w4 && !ue) return hipErrorNotSupported;   // MX scales are e8m0 bytes
  uint8_t* hq = static_cast<uint8_t*>(L.h);
  g.ids = L.pair_ids;
  g.P = P;
  // h -> e4m3 codes with per-(pair, 128-channel) scales: e8m0 bytes or fp32, as the down kernel
  // reads them (rows in h's own order: sorted, or by pair on the fused path)
  void* hs = ue ? static_cast<void*>(L.h_scale_bytes) : static_cast<void*>(L.h_scales);
  if (L.run_gate_up) {
    hipError_t e = launch_mode<kGateUp>(g, L.E, P, ue, w4, fused, stream);
    if (e != hipSuccess) return e;
    e = launch_quantize_act(L.h32, MOE_F32, P, L.f, nullptr, hq, hs, ue, stream);
    if (e != hipSuccess) return e;
  }
  if (!L.run_down) return hipSuccess;

  Fp8DecodeArgs dn{};
  dn.a = hq;
  dn.a_s = hs;
  dn.a_gather = 0;
  dn.sorted_pair = L.sorted_pair;
  dn.k = L.k;
  dn.w0 = static_cast<const uint8_t*>(L.w_down);
  dn.s0 = L.s_down;
  dn.K = L.f;
  dn.N = L.d;
  dn.offsets = L.offsets;
  dn.y = L.y;
  dn.y_layout = L.y_layout;
  dn.y_bf16 = L.y_bf16;
  dn.topk_w = L.topk_w;
  dn.ids = L.pair_ids;
  dn.P = P;
  return launch_mode<kDown>(dn, L.E, P, ue, w4, fused, stream);
}

}  // namespace moe
