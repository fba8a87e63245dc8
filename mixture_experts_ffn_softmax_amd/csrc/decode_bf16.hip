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
//
// Experts with at most 16 tokens (the usual decode case), or every expert when the batch has at
// most 32 tokens (in passes of 16), take streaming kernels instead, one wave per workgroup owning
// its weight rows for all of K, so no cross-wave reduction and no barrier is needed. Gate/up: a wave owns 8 gate rows and the matching 8 up rows; each stage moves 256
// K-elements of the 16 rows (512 contiguous bytes per row) into a two-slot LDS ring by DMA, one
// stage ahead, and the 16 tokens' slices of the same stages are loaded into registers at the same
// depth. Down: a wave owns 32 W_down rows; each 128-wide stage brings the rows and the
// 16 token rows of h into a three-slot ring by DMA.
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
  int small_max;              // experts with at most this many tokens belong to the streaming
                              // kernel (0: this kernel takes every expert)
  int stream_max;             // the streaming kernels take experts with 1 .. stream_max tokens
  // fused small-batch path (see ExpertsLaunch): routing ids [P]
  const int32_t* ids;
  int P;
};

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// Down-projection outputs n .. n + 3 of one pair (sorted position pos): fp32 accumulation into
// y [T, N] by atomics, the unweighted row pos of y [P, N], or the weighted slot of the pair.
__device__ __forceinline__ void store_down(const DecodeArgs& p, int pos, int pair, int n,
                                           f32x4_t v) {
  const float wgt = p.topk_w ? p.topk_w[pair] : 1.0f;
  if (p.y_layout == MOE_Y_ACC_F32) {
    float* dst = static_cast<float*>(p.y) + static_cast<size_t>(pair / p.k) * p.N + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(dst + i, wgt * v[i]);
    return;
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

// kFused: the fused small-batch path (pairs from the routing ids; h and slots indexed by pair).
template <int MODE, bool kFused>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeArgs p) {
  constexpr int kRows = MODE == kGateUp ? kDecodeGateRows : kDecodeDownRows;
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
  if (M <= p.small_max) return;  // empty, or the streaming kernel's expert
  auto pos_of = [&](int i) { return kFused ? plist[i] : row0 + i; };
  auto pair_of = [&](int i) { return kFused ? plist[i] : p.sorted_pair[row0 + i]; };

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
      const int pos = pos_of(ti);
      const int src = p.a_gather ? pair_of(ti) / p.k : pos;
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
      const int pos = pos_of(ti);
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
        const int pair = pair_of(ti);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int n = rb * kRows + rg * 16 + 4 * g;
          if (n < p.N) store_down(p, pos, pair, n, s[rg]);
        }
      }
    }
    __syncthreads();
  }
}

// ---- streaming gate/up kernel (experts of 1..16 tokens; every expert, in passes, at T <= 32) 
constexpr int kStrRows = 16;                       // weight rows per wave
constexpr int kStrRing = 2;                        // LDS slots
constexpr int kStrAhead = kStrRing - 1;            // stages in flight

// Stage `st` (clamped to the last stage) of the wave's 16 rows into `slot` (KS K-elements per
// row, i.e. CPR = KS / 8 chunks of 16 bytes): instruction i moves rows (64 / CPR) i .. +64/CPR-1;
// lane l brings logical chunk (l % CPR) ^ (row % CPR) of local row (64 / CPR) i + l / CPR to LDS
// position l, so chunk q of row r sits at physical chunk q ^ (r % CPR) of that row.
template <int KS>
__device__ __forceinline__ void str_dma(const char* slot, const uint32_t (&voff)[KS / 32],
                                        i32x4_t rsrc0, i32x4_t rsrc1, int st, int nst) {
  const uint32_t kb = static_cast<uint32_t>(min(st, nst - 1)) * KS * 2u;
  const uint32_t base = lds_offset(slot);
#pragma unroll
  for (int i = 0; i < KS / 32; ++i)
    dma16(base + i * 1024, voff[i], i >= KS / 64 ? rsrc1 : rsrc0, kb);  // rows 8..15: W_up
}

template <int KS, bool kFused>
__global__ __launch_bounds__(64) void decode_stream_kernel(DecodeArgs p) {
  constexpr int kStage = kStrRows * KS * 2;        // bytes per slot
  constexpr int kCpr = KS / 8;                     // 16-byte chunks per row per stage
  constexpr int kNi = KS / 32;                     // DMA instructions (and MFMAs) per stage
  constexpr int kLoads = 2 * kNi;                  // vector loads per stage (DMA + tokens)
  constexpr int kOut = 8;                          // h channels per wave (8 gate + 8 up rows)
  const int nrb = (p.N + kOut - 1) / kOut;
  const int e = blockIdx.x / nrb;
  const int rb = blockIdx.x - e * nrb;
  // 16 KB, so that ten workgroups fit a CU (measured on Mixtral-shaped decode: two slots with ten
  // workgroups per CU 0.322 ms, three with six 0.326, four with five 0.329; 128- or 512-wide
  // stages in two slots 0.326). On the fused path the pass's 16 pairs are gathered in the first
  // slot before any DMA lands there.
  __shared__ __attribute__((aligned(1024))) char ring[kStrRing * kStage];
  int32_t* plist = reinterpret_cast<int32_t*>(ring);
  const int lane = threadIdx.x;
  const int r16 = lane & 15, g = lane >> 4;
  int row0, M;
  if constexpr (kFused) {
    row0 = 0;
    M = expert_pair_list<64, 16>(p.ids, p.P, e, plist, plist + 16);
  } else {
    row0 = p.offsets[e];
    M = p.offsets[e + 1] - row0;
  }
  if (M == 0 || M > p.stream_max) return;
  const size_t wstride = static_cast<size_t>(p.N) * p.K;
  const uint32_t wbytes = static_cast<uint32_t>(p.N) * p.K * 2u;
  const i32x4_t rs0 = make_rsrc(p.w0 + e * wstride, wbytes);
  const i32x4_t rs1 = make_rsrc(p.w1 + e * wstride, wbytes);
  // DMA lane offsets: instruction i, lane l -> local row r (rows 0..7 gate, 8..15 up, both for
  // h channels rb * 8 + r % 8), logical chunk (l % CPR) ^ (r % CPR).
  uint32_t voff[kNi];
#pragma unroll
  for (int i = 0; i < kNi; ++i) {
    const int r = i * (64 / kCpr) + lane / kCpr;
    const int n = rb * 8 + (r & 7);
    const int c = (lane % kCpr) ^ (r % kCpr);
    voff[i] = static_cast<uint32_t>(min(n, p.N - 1)) * p.K * 2u + c * 16;
  }
  const int nst = p.K / KS;
  // passes of 16 tokens (one unless the expert has more)
  for (int tc0 = 0; tc0 < M; tc0 += 16) {
  const int mp = min(16, M - tc0);
  // token r16's pair (its h row on the fused path) and the row of x it reads
  const int t = min(r16, mp - 1);
  int pos, src;
  if constexpr (kFused) {
    if (tc0 > 0) expert_pair_list<64, 16>(p.ids, p.P, e, plist, plist + 16, tc0);
    pos = plist[t];
    src = p.a_gather ? pos / p.k : pos;
    __syncthreads();   // the list is read before the ring is refilled
  } else {
    pos = row0 + tc0 + t;
    src = p.a_gather ? p.sorted_pair[pos] / p.k : pos;
  }
  // token operand: lane (t = l % 16, g = l / 16) holds k = 32 u + 8 g .. +7 of token t
  const uint16_t* trow = p.a + static_cast<size_t>(src) * p.K + g * 8;
  u32x4_t tok[kStrRing][kNi];
  // Lanes of tokens past the pass's last load nothing (their output columns are not stored): the
  // token operand's bytes through the texture path shrink with the pass's token count. Lanes of
  // token 0 are always live, so every load instruction issues and the per-stage count holds.
  const bool tok_live = r16 < mp;
  auto load_tok = [&](u32x4_t (&tv)[kNi], int st) {
    const int kb = min(st, nst - 1) * KS;
#pragma unroll
    for (int u = 0; u < kNi; ++u)
      tv[u] = tok_live ? *reinterpret_cast<const u32x4_t*>(trow + kb + u * 32)
                       : u32x4_t{0u, 0u, 0u, 0u};
  };
  // prologue: stages 0 .. kStrAhead - 1
#pragma unroll
  for (int q = 0; q < kStrAhead; ++q) {
    str_dma<KS>(ring + q * kStage, voff, rs0, rs1, q, nst);
    load_tok(tok[q], q);
  }
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // Stage S in slot S % kStrRing: wait until stage S has landed (the kStrAhead - 1 newer stages
  // may still be in flight), issue stage S + kStrAhead into the slot stage S - 1 used (its LDS
  // reads were consumed by that stage's MFMAs), then KS / 32 MFMAs of 16 weight rows x 16 tokens
  // x 32 K.
#define MOE_STR_STAGE(Q, S)                                                                   \
  {                                                                                           \
    constexpr int QN = (Q + kStrAhead) % kStrRing;                                            \
    wait_vmcnt<kLoads * (kStrAhead - 1)>();                                                   \
    str_dma<KS>(ring + QN * kStage, voff, rs0, rs1, (S) + kStrAhead, nst);                    \
    load_tok(tok[QN], (S) + kStrAhead);                                                       \
    const char* sl = ring + (Q) * kStage;                                                     \
    _Pragma("unroll") for (int u = 0; u < kNi; ++u) {                                         \
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(                                  \
          sl + r16 * (KS * 2) + (((4 * u + g) ^ (r16 % kCpr)) << 4));                          \
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, tok[Q][u]), \
                                                    acc, 0, 0, 0);                            \
    }                                                                                         \
  }
  for (int s = 0; s < nst; s += kStrRing) {
    MOE_STR_STAGE(0, s)
    if (s + 1 < nst) MOE_STR_STAGE(1, s + 1)
    if constexpr (kStrRing >= 3) {
      if (s + 2 < nst) MOE_STR_STAGE(2, s + 2)
    }
    if constexpr (kStrRing >= 4) {
      if (s + 3 < nst) MOE_STR_STAGE(3, s + 3)
    }
  }
#undef MOE_STR_STAGE
  wait_vmcnt<0>();  // the clamped re-reads past the last stage

  // Output layout: lane l holds token l % 16 and local weight rows 4 (l / 16) + i; rows 0..7
  // (lanes 0..31) are gate, rows 8..15 (lanes 32..63) the matching up rows.
  f32x4_t up;
#pragma unroll
  for (int i = 0; i < 4; ++i) up[i] = __shfl_xor(acc[i], 32, 64);
  const int n = rb * 8 + 4 * g;
  if (r16 < mp && g < 2 && n < p.N) {   // r16 < mp: t == r16
    u32x2_t o;
    o[0] = f32_to_bf16_bits(silu_mul(acc[0], up[0])) |
           (static_cast<uint32_t>(f32_to_bf16_bits(silu_mul(acc[1], up[1]))) << 16);
    o[1] = f32_to_bf16_bits(silu_mul(acc[2], up[2])) |
           (static_cast<uint32_t>(f32_to_bf16_bits(silu_mul(acc[3], up[3]))) << 16);
    *reinterpret_cast<u32x2_t*>(p.h + static_cast<size_t>(pos) * p.N + n) = o;
  }
  }  // passes
}


// ---- streaming down kernel (experts of 1..16 tokens; every expert, in passes, at T <= 32) ----
// One wave owns 32 consecutive W_down rows (two 16-row A operands that share each token operand,
// so a token byte read serves two weight bytes) for all of K = f. Each 128-wide K stage moves the
// 32 weight rows (256 contiguous bytes each) and the expert's 16 token rows of h into one slot of
// a three-slot LDS ring by DMA, two stages ahead. Both operands arrive by DMA: with no other
// vector memory loads in the loop, the one vmcnt wait per stage is the only wait on memory (the
// compiler, which does not see the DMA instructions, would otherwise wait for token loads with
// counts that drain the ring). Measured on Mixtral-shaped decode: 0.159 ms for the down GEMM
// against 0.182 ms for the K-split kernel; workgroups of two or four such waves sharing one
// token slot per stage (a four-slot ring, a barrier per stage) took 0.161 and 0.166 ms. The same
// form for the gate/up GEMM (16 gate + 16 up rows per wave, x rows gathered by DMA) took 0.353
// against 0.344 ms for the streaming gate/up kernel above (then with its four-slot ring).
constexpr int kSdRows = 32;                      // W_down rows per wave
constexpr int kSdKS = 128;                       // K per stage
constexpr int kSdW = kSdRows * kSdKS * 2;        // weight bytes per stage (8 KB)
constexpr int kSdSlot = kSdW + 16 * kSdKS * 2;   // + 16 token rows (4 KB)
constexpr int kSdRing = 3;
constexpr int kSdAhead = kSdRing - 1;
constexpr int kSdLoads = kSdSlot / 1024;         // DMA instructions per stage

template <bool kFused>
__global__ __launch_bounds__(64) void decode_stream_down_kernel(DecodeArgs p) {
  const int nrb = p.N / kSdRows;                 // N = d, a multiple of 128 on this path
  const int e = blockIdx.x / nrb;
  const int rb = blockIdx.x - e * nrb;
  // 36 KB, so that four workgroups fit a CU. On the fused path the pass's 16 pairs are gathered
  // in the first slot before any DMA lands there.
  __shared__ __attribute__((aligned(1024))) char ring[kSdRing * kSdSlot];
  int32_t* plist = reinterpret_cast<int32_t*>(ring);
  const int lane = threadIdx.x;
  const int r16 = lane & 15, g = lane >> 4;
  int row0, M;
  if constexpr (kFused) {
    row0 = 0;
    M = expert_pair_list<64, 16>(p.ids, p.P, e, plist, plist + 16);
  } else {
    row0 = p.offsets[e];
    M = p.offsets[e + 1] - row0;
  }
  if (M == 0 || M > p.stream_max) return;
  const uint32_t row_bytes = static_cast<uint32_t>(p.K) * 2u;
  const size_t wstride = static_cast<size_t>(p.N) * p.K;
  const i32x4_t rw = make_rsrc(p.w0 + e * wstride, static_cast<uint32_t>(wstride * 2u));
  const i32x4_t rh = make_rsrc(p.a, static_cast<uint32_t>(p.P) * row_bytes);
  // Weight DMA: instruction i, lane l -> local row r = 4 i + l / 16, logical chunk (l % 16) ^ r.
  const int n0 = rb * kSdRows;
  uint32_t voff[kSdW / 1024];
#pragma unroll
  for (int i = 0; i < kSdW / 1024; ++i) {
    const int r = 4 * i + lane / 16;
    voff[i] = static_cast<uint32_t>(n0 + r) * row_bytes +
              static_cast<uint32_t>(((lane & 15) ^ (r & 15)) << 4);
  }
  const int nst = p.K / kSdKS;
  // passes of 16 tokens (one unless the expert has more)
  for (int tc0 = 0; tc0 < M; tc0 += 16) {
  const int mp = min(16, M - tc0);
  if (kFused && tc0 > 0) expert_pair_list<64, 16>(p.ids, p.P, e, plist, plist + 16, tc0);
  // h row of the pass's token t: its pair on the fused path, its sorted position otherwise
  auto hrow_of = [&](int t) { return kFused ? plist[t] : row0 + tc0 + t; };
  // Token DMA: instruction j brings token rows 4 j .. 4 j + 3 of the slot (lane l: row
  // tr = 4 j + l / 16, filled from token min(tr, mp - 1)), logical chunk (l % 16) ^ tr.
  uint32_t toff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tr = 4 * j + lane / 16;
    toff[j] = static_cast<uint32_t>(hrow_of(min(tr, mp - 1))) * row_bytes +
              static_cast<uint32_t>(((lane & 15) ^ tr) << 4);
  }
  const int my_row = hrow_of(min(r16, mp - 1));
  if constexpr (kFused) __syncthreads();   // the list is read before the ring is refilled
  auto issue = [&](int q, int st) {
    const uint32_t kb = static_cast<uint32_t>(min(st, nst - 1)) * kSdKS * 2u;
    const uint32_t base = lds_offset(ring + q * kSdSlot);
#pragma unroll
    for (int i = 0; i < kSdW / 1024; ++i) dma16(base + i * 1024, voff[i], rw, kb);
#pragma unroll
    for (int j = 0; j < 4; ++j)   // token rows past the pass's last: only lane 0 moves (a duplicate)
      if (4 * j + lane / 16 < mp || lane == 0) dma16(base + kSdW + j * 1024, toff[j], rh, kb);
  };
#pragma unroll
  for (int q = 0; q < kSdAhead; ++q) issue(q, q);
  f32x4_t acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
  // Stage S in slot S % 3: wait until it has landed (the next stage may still be in flight),
  // issue stage S + 2 into the slot stage S - 1 used, then 4 K-steps of 32 x (two 16-row weight
  // groups x 16 tokens). Lane (r16, g) reads logical chunk 4 u + g of weight rows r16 and
  // 16 + r16 and of token row r16.
#define MOE_SD_STAGE(Q, S)                                                                   \
  {                                                                                          \
    wait_vmcnt<kSdLoads * (kSdAhead - 1)>();                                                 \
    issue(((Q) + kSdAhead) % kSdRing, (S) + kSdAhead);                                       \
    const char* sl = ring + (Q) * kSdSlot;                                                   \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) {                                          \
      const int ch = ((4 * u + g) ^ r16) << 4;                                               \
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(sl + r16 * 256 + ch);           \
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(sl + (16 + r16) * 256 + ch);    \
      const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(sl + kSdW + r16 * 256 + ch);     \
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc0, 0, 0, 0);                  \
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc1, 0, 0, 0);                  \
    }                                                                                        \
  }
  for (int s = 0; s < nst; s += kSdRing) {
    MOE_SD_STAGE(0, s)
    if (s + 1 < nst) MOE_SD_STAGE(1, s + 1)
    if (s + 2 < nst) MOE_SD_STAGE(2, s + 2)
  }
#undef MOE_SD_STAGE
  wait_vmcnt<0>();  // the clamped re-reads past the last stage

  // lane l holds token l % 16 and weight rows 4 (l / 16) + i of each 16-row group (the pair is
  // read only now: a load in flight beside the DMA would make the compiler wait on the ring)
  if (r16 < mp) {
    const int pair = kFused ? my_row : p.sorted_pair[my_row];
    store_down(p, my_row, pair, n0 + 4 * g, acc0);
    store_down(p, my_row, pair, n0 + 16 + 4 * g, acc1);
  }
  }  // passes
}

}  // namespace

constexpr int kStrK = 256;  // K per stage of the streaming kernel
// Batches of at most this many tokens give no expert more than this many pairs when each token's
// k experts are distinct (the router's are): the streaming kernels then take every expert, in
// one or two passes of 16 tokens, and the K-split kernels are not launched (each launch costs
// ~4 us even when all its workgroups exit at once). Experts with more pairs stay correct, in more
// passes.
constexpr int kStreamAllTokens = 32;


hipError_t launch_experts_bf16_decode(const ExpertsLaunch& L, hipStream_t stream) {
  const bool fused = L.pair_ids != nullptr;
  const int P = L.T * L.k;
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
  g.ids = L.pair_ids;
  g.P = P;
  const unsigned grid1 = static_cast<unsigned>(L.E) * ((L.f + kDecodeGateRows - 1) / kDecodeGateRows);
  // the streaming kernel needs whole K stages
  const bool stream_small = L.d % kStrK == 0;
  const bool gu_all = stream_small && L.T <= kStreamAllTokens;
  g.small_max = stream_small ? 16 : 0;
  g.stream_max = gu_all ? P : 16;
  const unsigned grid1s = static_cast<unsigned>(L.E) * ((L.f + 7) / 8);
  if (L.run_gate_up && stream_small) {
    if (fused)
      hipLaunchKernelGGL((decode_stream_kernel<kStrK, true>), dim3(grid1s), dim3(64), 0, stream, g);
    else
      hipLaunchKernelGGL((decode_stream_kernel<kStrK, false>), dim3(grid1s), dim3(64), 0, stream,
                         g);
  }
  if (L.run_gate_up && !gu_all) {
    if (fused)
      hipLaunchKernelGGL((decode_bf16_kernel<kGateUp, true>), dim3(grid1), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((decode_bf16_kernel<kGateUp, false>), dim3(grid1), dim3(256), 0, stream,
                         g);
  }
  if (!L.run_down) return hipGetLastError();

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
  // the streaming kernel needs whole K stages and whole 32-row panels
  const bool stream_down = L.f % kSdKS == 0 && L.d % kSdRows == 0;
  const bool dn_all = stream_down && L.T <= kStreamAllTokens;
  dn.small_max = stream_down ? 16 : 0;
  dn.stream_max = dn_all ? P : 16;
  dn.ids = L.pair_ids;
  dn.P = P;
  if (stream_down) {
    const unsigned grid2s = static_cast<unsigned>(L.E) * (L.d / kSdRows);
    if (fused)
      hipLaunchKernelGGL((decode_stream_down_kernel<true>), dim3(grid2s), dim3(64), 0, stream, dn);
    else
      hipLaunchKernelGGL((decode_stream_down_kernel<false>), dim3(grid2s), dim3(64), 0, stream,
                         dn);
  }
  if (dn_all) return hipGetLastError();
  if (fused)
    hipLaunchKernelGGL((decode_bf16_kernel<kDown, true>), dim3(grid2), dim3(256), 0, stream, dn);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<kDown, false>), dim3(grid2), dim3(256), 0, stream, dn);
  return hipGetLastError();
}

}  // namespace moe
