// Fine-grained FP8 grouped GEMMs: e4m3 x e4m3 on the gfx950 matrix cores with fp32 accumulation.
//
// Transformers "Fine-grained FP8" page, introduction: weights carry one scale per 128x128 block,
// activations one dynamic scale per token per 128 input channels. A K range of 128 therefore has
// one activation scale per row and one weight scale per 128 output columns, so
//     y[r][n] = sum_kb  sa[r][kb] * sw[n/128][kb] * sum_{k in kb} qa[r][k] * qw[n][k].
// One v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0 scales) computes exactly the inner sum of one
// 16x16 block for one kb; its fp32 result is scaled by sa * sw and added to the accumulator.
// With UE8M0 scales (same page, "UE8M0 scale format": every scale a power of two, stored as an
// e8m0 byte) the MFMA applies sa and sw itself as its per-row and per-column block scales and
// accumulates across kb directly: no per-block promotion. Activation scales reach the kernel as
// fp32 powers of two; the e8m0 byte of one is its exponent field.
// The gate/up GEMM applies SwiGLU and re-quantises h per (pair, 128 channels) in its epilogue,
// since h is the input of the down projection, a quantised linear too; the down GEMM writes y in
// the requested layout (Transformers "Experts backends" page: gated MLP, weighted combine).
//
// Tiling: 128 pair rows x 256 weight rows per workgroup (gate/up: 128 gate + the same 128 up
// rows, i.e. one full 128-channel group of h), 8 waves in a 2 x 4 grid, each 64 rows x 64
// weight rows = 4 x 4 MFMA blocks of 16 x 16. K is staged 128 at a time (one scale block)
// through a ring of three LDS stages filled two stages ahead by global -> LDS DMA. With UE8M0
// scales an expert's rows come in 256-row blocks: a block of more than 128 rows runs as one
// 256-row tile (8 waves of 64 x 128, a ring of two stages), a shorter one as a 128-row tile.
//
// FP4 experts (kW4; Transformers "Experts backends" page, FP4 quantised experts; "Fine-grained
// FP8" page, "UE8M0 scale format"): E2M1 weights in matrix-fragment order, so a stage's weight
// rows are sixteen contiguous 1 KB fragments (one DMA instruction each, read back lane by lane),
// and one e8m0 byte per weight row per 32 channels, DMA'd as a dword per row per stage. The
// instruction takes B as FP4 (format code 4) with a scale per lane; a lane of an FP4 operand holds
// K = 32g .. 32g + 31 of its block, an 8-bit one K = 16g .. 16g + 15 and 64 + 16g .. 64 + 16g + 15
// (gfx950), so the e4m3 activations are read as 16-byte chunks g and 4 + g of the stage row.
#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBMf = 128;                          // pair rows per tile
constexpr int kBNf = 256;                          // weight rows per tile
constexpr int kBKf = 128;                          // K per stage (one scale block)
constexpr int kAf = kBMf * kBKf;                   // A bytes per stage (16 KB)
constexpr int kBf = kBNf * kBKf;                   // B bytes per stage (32 KB)
constexpr int kStageF = kAf + kBf + kBMf * 4;      // + activation scales of the tile rows
constexpr int kBf4 = kBNf * kBKf / 2;              // E2M1 weight bytes per stage (16 KB)
constexpr int kStageF4 = kAf + kBf4 + kBMf * 4 + kBNf * 4;   // + MX scale dwords of the rows
constexpr int kRingF = 3;
constexpr int kBMp = 256;                          // pair rows per 256-row tile
constexpr int kStageP = kBMp * kBKf + kBf + kBMp * 4;   // 256-row tile stage (65 KB)
constexpr int kHStage = kBMp * 132 * 4;            // gate/up epilogue: h [256][132] fp32
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kRingBytes = cmax(cmax(kRingF * kStageF, 2 * kStageP), kHStage);   // e4m3 weights
constexpr int kMaxKBlocks = 256;                 // K <= 32768
constexpr int kGateUp = 0;
constexpr int kDown = 1;

struct Fp8GemmArgs {
  const uint8_t* a;          // gate/up: x codes [T, K] (rows gathered); down: h codes [P, K]
  const float* a_s;          // activation scales [rows, K/128]
  int a_gather, a_rows;
  const int32_t* sorted_pair;
  int k;
  const uint8_t* b0;         // gate/up: W_gate [E, N, K]; down: W_down [E, N, K]
  const uint8_t* b1;         // gate/up: W_up
  const void* s0;            // block scales of b0 [E, N/128, K/128]: fp32, or e8m0 bytes (UE8M0);
                             // E2M1 weights: MX bytes [E, N, K/32]
  const void* s1;            // block scales of b1
  int K, N;
  const int32_t* offsets;
  const int32_t* tile_cum;
  int E;
  uint8_t* hq;               // gate/up output codes [P, N]
  float* hs;                 // gate/up output scales [P, N/128]
  void* y;                   // down output
  int y_layout, y_bf16;
  const float* topk_w;
};

// 128-byte LDS rows: chunk c of row r sits at position c ^ ((r >> 1) & 7), so 16 consecutive rows
// read at one logical chunk cover 16 distinct 16-byte slots of a 256-byte bank line.
__device__ __forceinline__ int swzf(int row, int chunk) {
  return row * kBKf + ((chunk ^ ((row >> 1) & 7)) << 4);
}

struct DmaF {
  i32x4_t ra, rs, rb0, rb1;
  uint32_t aoff[8], boff[4], soff;
  uint32_t brow16;           // e4m3 weights: byte offset of 16 weight rows (uniform)
  i32x4_t rbs0, rbs1;        // E2M1: MX scales of b0 / b1
  uint32_t bsoff;            // E2M1: this lane's weight row's MX scale offset
};

// Stage `st` of a BM-row tile into `buf`. Stages past the last one (the prefetches the loop issues
// beyond the end) get offsets past every buffer's range: the loads return zeros without touching
// memory, their buffers are never read, and every stage issues the same instructions, so the
// loop's vmcnt waits stay uniform (byte offsets stay below 2^31, so offset + 2^31 does not wrap).
// Only waves 0..3, one per SIMD, issue it (the SIMD's other wave keeps its MFMA and promotion work
// going while the DMA wave waits for the texture unit's queue; measured 5-6 % faster than all 8
// waves sharing it): wave w fills A rows (w * BM / 32 + i) * 8 .. +7, B rows (8w + i) * 8 .. +7
// (one KB per instruction, lane l -> row l / 8, chunk position l % 8; B rows 0..127 from rb0,
// 128..255 from rb1) and the scales of A rows w * BM / 4 .. (w + 1) * BM / 4 - 1.
// E2M1 (kW4, BM = 128): wave w fills weight fragments 4w .. 4w + 3 (16 rows x 128 K each, 1 KB
// apart in global memory by K block: fragments 0..7 from rb0, 8..15 from rb1) and the MX scale
// dwords of weight rows 64 w .. 64 w + 63 (rows 0..127 from rbs0, 128..255 from rbs1).
template <bool kW4, int BM>
__device__ __forceinline__ void dmaf(const char* buf, const DmaF& d, int st, int nst, int wave,
                                     int lane) {
  if (wave >= 4) return;
  constexpr int kA = BM * kBKf;
  const bool in = st < nst;
  const uint32_t sc = in ? static_cast<uint32_t>(st) : 0u;
  const uint32_t past = in ? 0u : 0x80000000u;
  const uint32_t kb = sc * kBKf + past;
  const uint32_t base = lds_offset(buf);
#pragma unroll
  for (int i = 0; i < BM / 32; ++i)
    dma16(base + (wave * (BM / 32) + i) * 1024, d.aoff[i], d.ra, kb);
  if constexpr (kW4) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(base + kA + (wave * 4 + i) * 1024, d.boff[i], wave < 2 ? d.rb0 : d.rb1,
            sc * 1024u + past);
    dma4(base + kA + kBf4 + kBMf * 4 + wave * 256, d.bsoff, wave < 2 ? d.rbs0 : d.rbs1,
         sc * 4u + past);
    if (lane < 32) dma4(base + kA + kBf4 + wave * 128, d.soff, d.rs, sc * 4u + past);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dma16(base + kA + (wave * 8 + i) * 1024, d.boff[i & 1], wave < 2 ? d.rb0 : d.rb1,
            kb + (i >> 1) * d.brow16);
    if (BM == 256 || lane < 32) dma4(base + kA + kBf + wave * BM, d.soff, d.rs, sc * 4u + past);
  }
}

__device__ __forceinline__ i32x8_t ld32(const char* p0, const char* p1) {
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(p0);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(p1);
  i32x8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// One tile of the grouped GEMM. kPair: a 256-row tile (an expert's rows 0..255 of one 256-row
// block holding more than 128 rows), 8 waves in a 4 x 2 grid of 64 rows x 128 weight rows (4 x 8
// MFMA blocks), a ring of two stages filled one stage ahead. Otherwise a 128-row tile, 8 waves in a
// 2 x 4 grid of 64 x 64 (4 x 4 blocks), a ring of three stages filled two ahead. Per 128-wide K
// block the pair tile moves 64 KB through the texture path for twice the MFMA work of the 128-row
// tile's 48 KB.
template <int MODE, bool kUE, bool kW4, bool kPair>
__device__ __forceinline__ void fp8_tile(const Fp8GemmArgs p, const TileCoord tc, char* ring,
                                         const uint32_t* wsc, const int* row_pair,
                                         const float* row_w) {
  static_assert(!kPair || (kUE && !kW4), "256-row tiles: e4m3 weights with UE8M0 scales only");
  constexpr int BM = kPair ? kBMp : kBMf;
  constexpr int MI = 4, NJ = kPair ? 8 : 4;        // 16x16 blocks per wave
  constexpr int WN = kPair ? 2 : 4;                // waves across the weight rows
  constexpr int kRing = kPair ? 2 : kRingF;
  constexpr int kA = BM * kBKf;                    // A bytes per stage
  constexpr int kStg = kW4 ? kStageF4 : kA + kBf + BM * 4;   // bytes per ring stage
  constexpr int kSA = kA + (kW4 ? kBf4 : kBf);     // activation scales within a stage
  constexpr int kSB = kSA + kBMf * 4;              // E2M1: MX scale dwords within a stage
  constexpr int kDmaPerStage = kW4 ? 10 : BM / 32 + 9;   // DMA instructions per issuing wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * 64;
  // weight rows of this wave inside the tile: gate/up -> 128 / WN gate rows + the same up rows
  const int brow0 = MODE == kGateUp ? wn * (128 / WN) : wn * (256 / WN);
  // a wave whose 64 rows all lie past the tile's last row skips its fragment reads and MFMAs
  const bool active = arow0 < tc.rows;

  const int KB = p.K / kBKf;
  const uint32_t wbytes = static_cast<uint32_t>(p.N) * (kW4 ? p.K / 2 : p.K);   // one expert
  const size_t wstride = wbytes;
  // The DMA's resources are wave-uniform; reading them from the first lane keeps them in SGPRs
  // where the compiler's uniformity analysis would otherwise lose track of them.
  auto uni = [](i32x4_t r) {
    return i32x4_t{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                   __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3])};
  };
  DmaF d;
  d.ra = uni(make_rsrc(p.a, static_cast<uint32_t>(p.a_rows) * p.K));
  d.rs = uni(make_rsrc(p.a_s, static_cast<uint32_t>(p.a_rows) * KB * 4u));
  d.rb0 = uni(make_rsrc(p.b0 + tc.e * wstride, wbytes));
  d.rb1 = MODE == kGateUp ? uni(make_rsrc(p.b1 + tc.e * wstride, wbytes)) : d.rb0;
  auto src_row = [&](int r) {
    const int pos = tc.row0 + min(r, tc.rows - 1);
    return p.a_gather ? p.sorted_pair[pos] / p.k : pos;
  };
#pragma unroll
  for (int i = 0; i < BM / 32; ++i) {
    const int r = (wave * (BM / 32) + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    d.aoff[i] = static_cast<uint32_t>(src_row(r)) * p.K + c * 16;
  }
  if constexpr (kW4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int fi = wave * 4 + i;   // fragment = 16 tile rows
      const int n16 = MODE == kGateUp ? tc.ntile * 8 + (fi & 7)
                                      : min(tc.ntile * 16 + fi, p.N / 16 - 1);
      d.boff[i] = static_cast<uint32_t>(n16) * KB * 1024u + lane * 16;
    }
    const size_t sstride = static_cast<size_t>(p.N) * (p.K / 32);
    d.rbs0 = make_rsrc(static_cast<const uint8_t*>(p.s0) + tc.e * sstride,
                       static_cast<uint32_t>(sstride));
    d.rbs1 = MODE == kGateUp ? make_rsrc(static_cast<const uint8_t*>(p.s1) + tc.e * sstride,
                                         static_cast<uint32_t>(sstride))
                             : d.rbs0;
    const int r = (wave & 3) * 64 + lane;   // weight row of the tile (waves 0..3 issue)
    const int n = MODE == kGateUp ? tc.ntile * 128 + (r & 127) : min(tc.ntile * kBNf + r, p.N - 1);
    d.bsoff = static_cast<uint32_t>(n) * (p.K / 32);
  } else {
    // B row of the issuing wave's instruction i = 2 m + b is r0 + 8 b + 16 m, and the swizzle
    // repeats every 16 rows: the lane offset of instruction b plus a uniform 16 m rows. Rows past
    // N (a down tile over the last 128 columns) lie past the expert's weights and read as zeros.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int r = wave * 64 + 8 * b + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int n = MODE == kGateUp ? tc.ntile * 128 + (r & 127) : tc.ntile * kBNf + r;
      d.boff[b] = static_cast<uint32_t>(n) * p.K + c * 16;
    }
    d.brow16 = 16u * p.K;
  }
  d.soff = static_cast<uint32_t>(src_row(wave * (BM / 4) + (lane & (BM / 4 - 1)))) * KB * 4u;

  // weight scales of this wave's blocks, [2][kMaxKBlocks] in LDS
  const uint32_t* sw0 = wsc + (MODE == kGateUp ? 0 : (brow0 >> 7)) * kMaxKBlocks;
  const uint32_t* sw1 = wsc + (MODE == kGateUp ? 1 : (brow0 >> 7)) * kMaxKBlocks;
  (void)sw0;
  (void)sw1;

  f32x4_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int nst = KB;
#pragma unroll
  for (int s = 0; s < kRing - 1; ++s) dmaf<kW4, BM>(ring + s * kStg, d, s, nst, wave, lane);

  // lane -> (row / column l % 16, 32-byte k slice l / 16) of a 16x16x128 MFMA operand
  const int lr = lane & 15, lk = lane >> 4;
  // weight row of block j: gate/up -> gate rows for j < NJ / 2, the matching up rows after
  auto brow = [&](int j) {
    return MODE == kGateUp ? (j < NJ / 2 ? brow0 + j * 16 : 128 + brow0 + (j - NJ / 2) * 16)
                           : brow0 + j * 16;
  };
  auto stage = [&](const char* cur, char* nxt, int s) {
    // this wave's DMA of stage s is done (the kRing - 2 stages after it may be pending)
    wait_vmcnt<(kRing - 2) * kDmaPerStage>();
    __builtin_amdgcn_s_barrier();
    dmaf<kW4, BM>(nxt, d, s + kRing - 1, nst, wave, lane);
    if (!active) return;
    i32x8_t fa[MI];
    f32x4_t sa[MI];
    int ea[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = arow0 + i * 16 + lr;
      // E2M1 weights: the e4m3 chunks in the 8-bit operand's K order (lk, 4 + lk)
      fa[i] = kW4 ? ld32(cur + swzf(row, lk), cur + swzf(row, 4 + lk))
                  : ld32(cur + swzf(row, 2 * lk), cur + swzf(row, 2 * lk + 1));
      if constexpr (kUE) {
        // the e8m0 byte of the lane's row: exponent field of its power-of-two fp32 scale
        ea[i] = (*reinterpret_cast<const uint32_t*>(cur + kSA + row * 4) >> 23) & 0xFF;
      } else {
        sa[i] = *reinterpret_cast<const f32x4_t*>(cur + kSA + (arow0 + i * 16 + 4 * lk) * 4);
      }
    }
    // weight fragments four blocks at a time (the pair tile's eight in two groups)
#pragma unroll
    for (int g = 0; g < NJ; g += 4) {
      i32x8_t fb[4];
      int ebw[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = brow(g + jj);
        if constexpr (kW4) {
          // fragment row / 16, 16 bytes per lane; the lane's MX byte: row + lr, block lk
          const u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(cur + kAf + (row >> 4) * 1024 + lane * 16);
          fb[jj] = i32x8_t{static_cast<int>(w4[0]), static_cast<int>(w4[1]),
                           static_cast<int>(w4[2]), static_cast<int>(w4[3]), 0, 0, 0, 0};
          ebw[jj] = static_cast<const uint8_t*>(static_cast<const void*>(cur))[kSB + (row + lr) * 4 + lk];
        } else {
          fb[jj] = ld32(cur + kA + swzf(row + lr, 2 * lk), cur + kA + swzf(row + lr, 2 * lk + 1));
        }
      }
      // block j = g + jj holds up rows (second weight-scale block) for j >= NJ / 2 in gate/up
      auto up = [&](int jj) { return MODE == kGateUp && g + jj >= NJ / 2; };
      if constexpr (kW4) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[i][g + jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa[i], fb[jj], acc[i][g + jj], 0, 4, 0, ea[i], 0, ebw[jj]);
      } else if constexpr (kUE) {
        const int eb0 = static_cast<int>(sw0[s]), eb1 = static_cast<int>(sw1[s]);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[i][g + jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa[i], fb[jj], acc[i][g + jj], 0, 0, 0, ea[i], 0, up(jj) ? eb1 : eb0);
      } else {
        const float w0 = __uint_as_float(sw0[s]), w1 = __uint_as_float(sw1[s]);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const f32x4_t s0v = sa[i] * w0, s1v = sa[i] * w1;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4_t part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa[i], fb[jj], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
            const f32x4_t sc = up(jj) ? s1v : s0v;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][g + jj][q] = fmaf(part[q], sc[q], acc[i][g + jj][q]);
          }
        }
      }
    }
  };
  if constexpr (kRing == 3 && kUE && !kW4) {
    // 128-row tiles with UE8M0 scales: the fragments of stage s + 1 are read while the second
    // half of stage s's MFMAs runs. Stage s: MFMAs of row blocks 0..1 from registers; wait for this wave's DMA of
    // stage s + 1 and its own LDS reads, barrier (stage s + 1 in LDS, every wave done reading
    // stage s); DMA of stage s + 3 into stage s's buffer; reads of stage s + 1; MFMAs of row
    // blocks 2..3 of stage s. With e4m3 weights and UE8M0 scales these 128-row tiles are the
    // remainders past an expert's 256-row tiles, mostly one active wave row. The slot pointer is
    // picked from an array at run time, so the compiler emits these reads as flat loads, which
    // also wait for the wave's outstanding DMA; as built, this measured 2 % faster on the
    // DeepSeek-V3-shaped gate/up than the read-after-barrier order below, and 3 % faster than the
    // same overlap with the slots addressed as ring + slot * size (LDS reads). On full 128-row
    // tiles (fp32 scales, E2M1 weights) the overlap was slower in both builds (LDS reads: 11 % and
    // 5 %), so those keep the schedule below.)
    struct Fr {
      i32x8_t fa[MI], fb[4];
      f32x4_t sa[MI];
      int ea[MI], ebw[4];
    };
    auto load = [&](const char* cur, Fr& F) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = arow0 + i * 16 + lr;
        F.fa[i] = kW4 ? ld32(cur + swzf(row, lk), cur + swzf(row, 4 + lk))
                      : ld32(cur + swzf(row, 2 * lk), cur + swzf(row, 2 * lk + 1));
        if constexpr (kUE)
          F.ea[i] = (*reinterpret_cast<const uint32_t*>(cur + kSA + row * 4) >> 23) & 0xFF;
        else
          F.sa[i] = *reinterpret_cast<const f32x4_t*>(cur + kSA + (arow0 + i * 16 + 4 * lk) * 4);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = brow(jj);
        if constexpr (kW4) {
          const u32x4_t w4 = *reinterpret_cast<const u32x4_t*>(cur + kAf + (row >> 4) * 1024 + lane * 16);
          F.fb[jj] = i32x8_t{static_cast<int>(w4[0]), static_cast<int>(w4[1]),
                             static_cast<int>(w4[2]), static_cast<int>(w4[3]), 0, 0, 0, 0};
          F.ebw[jj] = static_cast<const uint8_t*>(static_cast<const void*>(cur))[kSB + (row + lr) * 4 + lk];
        } else {
          F.fb[jj] = ld32(cur + kA + swzf(row + lr, 2 * lk), cur + kA + swzf(row + lr, 2 * lk + 1));
        }
      }
    };
    auto mma = [&](const Fr& F, int s, int i0) {
      auto up = [&](int jj) { return MODE == kGateUp && jj >= NJ / 2; };
#pragma unroll
      for (int i = i0; i < i0 + MI / 2; ++i) {
        if constexpr (kW4) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                F.fa[i], F.fb[jj], acc[i][jj], 0, 4, 0, F.ea[i], 0, F.ebw[jj]);
        } else if constexpr (kUE) {
          const int eb0 = static_cast<int>(sw0[s]), eb1 = static_cast<int>(sw1[s]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                F.fa[i], F.fb[jj], acc[i][jj], 0, 0, 0, F.ea[i], 0, up(jj) ? eb1 : eb0);
        } else {
          const float w0 = __uint_as_float(sw0[s]), w1 = __uint_as_float(sw1[s]);
          const f32x4_t s0v = F.sa[i] * w0, s1v = F.sa[i] * w1;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4_t part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                F.fa[i], F.fb[jj], f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
            const f32x4_t sc = up(jj) ? s1v : s0v;
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][jj][q] = fmaf(part[q], sc[q], acc[i][jj][q]);
          }
        }
      }
    };
    char* const bufs[3] = {ring, ring + kStg, ring + 2 * kStg};
    wait_vmcnt<kDmaPerStage>();   // this wave's DMA of stage 0 (stage 1's may be pending)
    __builtin_amdgcn_s_barrier();
    dmaf<kW4, BM>(bufs[2], d, 2, nst, wave, lane);
    Fr F;
    if (active) load(bufs[0], F);
    for (int s = 0; s < nst; ++s) {
      if (active) mma(F, s, 0);
      wait_vmcnt_lgkm0<kDmaPerStage>();   // DMA of stage s + 1 and this wave's reads of stage s
      __builtin_amdgcn_s_barrier();
      dmaf<kW4, BM>(bufs[s % 3], d, s + 3, nst, wave, lane);
      Fr N;
      if (active && s + 1 < nst) load(bufs[(s + 1) % 3], N);
      if (active) mma(F, s, MI / 2);
      F = N;
    }
  } else if constexpr (kRing == 3) {
    char* const st0 = ring;
    char* const st1 = ring + kStg;
    char* const st2 = ring + 2 * kStg;
    for (int s = 0; s < nst; s += 3) {
      stage(st0, st2, s);
      if (s + 1 < nst) stage(st1, st0, s + 1);
      if (s + 2 < nst) stage(st2, st1, s + 2);
    }
  } else {
    char* const st0 = ring;
    char* const st1 = ring + kStg;
    for (int s = 0; s < nst; s += 2) {
      stage(st0, st1, s);
      if (s + 1 < nst) stage(st1, st0, s + 1);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // Accumulator layout of a 16x16 block: lane l holds column l % 16, rows 4 (l / 16) + q.
  if (MODE == kGateUp) {
    // h tile [BM rows][128 channels] fp32 (row stride 132), then per-row quantisation.
    constexpr int kHS = 132;
    float* hsb = reinterpret_cast<float*>(ring);
    if (active) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = arow0 + i * 16 + 4 * lk + q;
            const int col = brow0 + j * 16 + lr;
            hsb[row * kHS + col] = silu_mul(acc[i][j][q], acc[i][j + NJ / 2][q]);
          }
    }
    __syncthreads();
#pragma unroll
    for (int half = 0; half < BM / 128; ++half) {
      const int row = half * 128 + (tid >> 2), part = tid & 3;
      float v[32];
      float amax = 0.0f;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const f32x4_t t = *reinterpret_cast<const f32x4_t*>(hsb + row * kHS + part * 32 + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[c + q] = t[q];
          amax = fmaxf(amax, fabsf(t[q]));
        }
      }
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      // fp32 rule: s = amax / 448, codes of v / s; UE8M0: s = 2^e, codes of v * 2^-e (exact)
      const int eb = ue8m0_byte(amax);
      const float s = kUE ? ldexpf(1.0f, eb - 127) : (amax > 0.0f ? amax / 448.0f : 1.0f);
      const float inv = ldexpf(1.0f, 127 - eb);
      if (row < tc.rows) {
        const size_t prow = static_cast<size_t>(tc.row0 + row);
        u32x4_t o[2];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            word |= e4m3_encode(kUE ? v[w * 4 + b] * inv : v[w * 4 + b] / s) << (8 * b);
          o[w >> 2][w & 3] = word;
        }
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(p.hq + prow * p.N + tc.ntile * 128 + part * 32);
        dst[0] = o[0];
        dst[1] = o[1];
        if (part == 0) p.hs[prow * (p.N / 128) + tc.ntile] = s;
      }
    }
  } else {
    // Passes of 64 rows staged as fp32 [64][260], one per wave row of the grid.
    constexpr int kYS = 260;
    float* ys = reinterpret_cast<float*>(ring);
    const int n0 = tc.ntile * kBNf;
#pragma unroll
    for (int pass = 0; pass < BM / 64; ++pass) {
      if (pass * 64 >= tc.rows) break;   // uniform: no rows left to write
      if (wm == pass) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              ys[(i * 16 + 4 * lk + q) * kYS + brow0 + j * 16 + lr] = acc[i][j][q];
      }
      __syncthreads();
      for (int e = tid; e < 64 * 64; e += 512) {
        const int rl = e >> 6, c4 = (e & 63) * 4;
        const int row = pass * 64 + rl;
        const int col = n0 + c4;
        if (row < tc.rows && col < p.N) {
          float4 v = *reinterpret_cast<const float4*>(ys + rl * kYS + c4);
          if (p.y_layout == MOE_Y_PERMUTED) {
            const size_t idx = static_cast<size_t>(tc.row0 + row) * p.N + col;
            if (p.y_bf16) {
              u32x2_t o;
              o[0] = f32_to_bf16_bits(v.x) | (static_cast<uint32_t>(f32_to_bf16_bits(v.y)) << 16);
              o[1] = f32_to_bf16_bits(v.z) | (static_cast<uint32_t>(f32_to_bf16_bits(v.w)) << 16);
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
                u32x2_t o;
                o[0] = f32_to_bf16_bits(v.x) | (static_cast<uint32_t>(f32_to_bf16_bits(v.y)) << 16);
                o[1] = f32_to_bf16_bits(v.z) | (static_cast<uint32_t>(f32_to_bf16_bits(v.w)) << 16);
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

// The tile table holds 256-row tiles (E2M1 weights: 128-row tiles). A 256-row block with more
// than 128 rows runs as one pair tile; a block of at most 128 rows (an expert's remainder past a
// multiple of 256, or a small expert) as a 128-row tile, so a near-empty second half never
// streams its own weight panel and a short remainder streams it once with half the A bytes.
template <int MODE, bool kUE, bool kW4>
__global__ __launch_bounds__(512) void gemm_fp8_kernel(Fp8GemmArgs p) {
  constexpr bool kPairs = kUE && !kW4;    // 256-row tiles (see fp8_tile_rows)
  constexpr int BMt = kPairs ? kBMp : kBMf;   // rows of the tile table
  const int NT = MODE == kGateUp ? p.N / 128 : (p.N + kBNf - 1) / kBNf;
  TileCoord tc;
  if (!map_tile(p.tile_cum, p.offsets, p.E, BMt, NT, tc)) return;
  tc.e = __builtin_amdgcn_readfirstlane(tc.e);
  tc.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
  tc.rows = __builtin_amdgcn_readfirstlane(tc.rows);
  tc.ntile = __builtin_amdgcn_readfirstlane(tc.ntile);

  __shared__ __attribute__((aligned(1024))) char ring[kW4 ? kRingF * kStageF4 : kRingBytes];
  __shared__ int row_pair[BMt];
  __shared__ float row_w[BMt];
  const int tid = threadIdx.x;
  if (MODE == kDown) {
    for (int r = tid; r < BMt; r += 512) {
      const int pair = p.sorted_pair[tc.row0 + min(r, tc.rows - 1)];
      row_pair[r] = pair;
      row_w[r] = p.topk_w ? p.topk_w[pair] : 1.0f;
    }
  }

  // Weight scales of the tile for every K block, staged in LDS before the pipeline starts (the
  // main loop issues no vector memory instructions besides its DMA): gate/up -> block ntile of
  // s_gate and of s_up; down -> the two 128-column blocks of the 256-column tile.
  // fp32 scales are kept as their bit patterns, UE8M0 scales as the e8m0 byte.
  const int KB = p.K / kBKf;
  __shared__ uint32_t wsc[2][kMaxKBlocks];
  for (int i = tid; i < (kW4 ? 0 : 2 * KB); i += 512) {
    const int which = i >= KB, kb = i - which * KB;
    const size_t blk = MODE == kGateUp ? static_cast<size_t>(tc.ntile)
                                       : static_cast<size_t>(min(tc.ntile * 2 + which, p.N / 128 - 1));
    const void* src = (MODE == kGateUp && which) ? p.s1 : p.s0;
    const size_t idx = (static_cast<size_t>(tc.e) * (p.N / 128) + blk) * KB + kb;
    wsc[which][kb] = kUE ? static_cast<uint32_t>(static_cast<const uint8_t*>(src)[idx])
                         : __float_as_uint(static_cast<const float*>(src)[idx]);
  }
  __syncthreads();

  if constexpr (kPairs) {
    if (tc.rows > kBMf) {
      fp8_tile<MODE, kUE, false, true>(p, tc, ring, &wsc[0][0], row_pair, row_w);
      return;
    }
  }
  fp8_tile<MODE, kUE, kW4, false>(p, tc, ring, &wsc[0][0], row_pair, row_w);
}

inline unsigned grid_for(int P, int E, int NT, int bm) {
  long n = static_cast<long>(max_row_tiles(P, E, bm)) * NT;
  return static_cast<unsigned>((n + 7) / 8 * 8);
}

}  // namespace

// e4m3 weights with UE8M0 scales run 256-row tiles (measured 3 % faster per DeepSeek-V3-shaped
// step than 128-row tiles); with fp32 scales the 256-row tile's per-block promotion made it 7 %
// slower, and E2M1 weights keep 128-row tiles.
int fp8_tile_rows(bool w4, bool ue8m0) { return ue8m0 && !w4 ? kBMp : kBMf; }

hipError_t launch_experts_fp8(const ExpertsLaunch& L, hipStream_t stream) {
  const int P = L.T * L.k;
  Fp8GemmArgs g{};
  g.a = static_cast<const uint8_t*>(L.a);
  g.a_s = L.a_scales;
  g.a_gather = L.a_gather;
  g.a_rows = L.a_gather ? L.T : P;
  g.sorted_pair = L.sorted_pair;
  g.k = L.k;
  g.b0 = static_cast<const uint8_t*>(L.w_gate);
  g.b1 = static_cast<const uint8_t*>(L.w_up);
  g.s0 = L.s_gate;
  g.s1 = L.s_up;
  g.K = L.d;
  g.N = L.f;
  g.offsets = L.offsets;
  g.tile_cum = L.tile_cum_a;
  g.E = L.E;
  g.hq = static_cast<uint8_t*>(L.h);
  g.hs = L.h_scales;
  const bool w4 = L.w_fp4 != 0;
  if (w4 && !L.scale_ue8m0) return hipErrorNotSupported;   // MX scales are e8m0 bytes
  const dim3 grid1(grid_for(P, L.E, L.f / 128, fp8_tile_rows(w4, L.scale_ue8m0)));
  if (L.run_gate_up) {
    if (w4)
      hipLaunchKernelGGL((gemm_fp8_kernel<kGateUp, true, true>), grid1, dim3(512), 0, stream, g);
    else if (L.scale_ue8m0)
      hipLaunchKernelGGL((gemm_fp8_kernel<kGateUp, true, false>), grid1, dim3(512), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_fp8_kernel<kGateUp, false, false>), grid1, dim3(512), 0, stream,
                         g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!L.run_down) return hipSuccess;

  Fp8GemmArgs dn{};
  dn.a = static_cast<const uint8_t*>(L.h);
  dn.a_s = L.h_scales;
  dn.a_gather = 0;
  dn.a_rows = P;
  dn.sorted_pair = L.sorted_pair;
  dn.k = L.k;
  dn.b0 = static_cast<const uint8_t*>(L.w_down);
  dn.s0 = L.s_down;
  dn.K = L.f;
  dn.N = L.d;
  dn.offsets = L.offsets;
  dn.tile_cum = L.tile_cum_b;
  dn.E = L.E;
  dn.y = L.y;
  dn.y_layout = L.y_layout;
  dn.y_bf16 = L.y_bf16;
  dn.topk_w = L.topk_w;
  const dim3 grid2(grid_for(P, L.E, (L.d + kBNf - 1) / kBNf, fp8_tile_rows(w4, L.scale_ue8m0)));
  if (w4)
    hipLaunchKernelGGL((gemm_fp8_kernel<kDown, true, true>), grid2, dim3(512), 0, stream, dn);
  else if (L.scale_ue8m0)
    hipLaunchKernelGGL((gemm_fp8_kernel<kDown, true, false>), grid2, dim3(512), 0, stream, dn);
  else
    hipLaunchKernelGGL((gemm_fp8_kernel<kDown, false, false>), grid2, dim3(512), 0, stream, dn);
  return hipGetLastError();
}

}  // namespace moe
