// bf16 grouped GEMMs on the gfx950 matrix cores (fp32 accumulation).
//
// Gate/up projection fused with SwiGLU, then the down projection with the unpermute / routing
// weight epilogue (Transformers "Experts backends" page, backends table rows grouped_mm,
// deepgemm_megamoe and sonicmoe: tokens grouped by expert, one grouped GEMM, gated MLP with
// SwiGLU). The rows of both GEMMs are the expert-sorted pairs; the gate/up GEMM reads each pair's
// token row straight from x (gather on load), so no permuted copy of x is needed.
//
// Tiling: 256 x 256 output tile per workgroup. Eight waves (two per SIMD) each own a 64 x 128
// block (gate/up: v_mfma_f32_16x16x32_bf16; down: v_mfma_f32_32x32x16_bf16); a down GEMM with a
// long K instead runs four waves (one per SIMD) of 128 x 128 whose k-steps interleave MFMAs,
// fragment reads and DMA in fenced groups. K is staged 64 at a time through 160 KB of LDS (two A
// and three B buffers) that buffer_load ... lds (global -> LDS DMA, no staging registers) fills,
// A one stage and B two stages ahead; one vmcnt wait and one barrier per stage. For the gate/up
// GEMM the 256 B-rows of a tile are 128 gate rows and the same 128 up rows; each wave holds
// matching gate and up accumulators and applies SwiGLU in registers. Results leave through LDS
// as whole 16-byte row segments.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kBM = 256;
constexpr int kBN = 256;
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
  int a_rows;                 // rows of a (bounds of the buffer descriptor)
  const int32_t* offsets;
  const int32_t* tile_cum;
  int E;
  uint16_t* h;                // gate/up output [P, N]
  void* y;                    // down output
  int y_layout, y_bf16;
  const float* topk_w;
  int cpx;                    // CUs per XCD (one workgroup per CU)
  int max_split;              // most K pieces a tail tile is cut into
  float* partial;             // [8 * cpx][kBM * kBN] fp32 partial tiles of cut tiles
};

__device__ __forceinline__ u32x2_t pack_bf16x4(float4 v) {
  u32x2_t o;
  o[0] = f32_to_bf16_bits(v.x) | (static_cast<uint32_t>(f32_to_bf16_bits(v.y)) << 16);
  o[1] = f32_to_bf16_bits(v.z) | (static_cast<uint32_t>(f32_to_bf16_bits(v.w)) << 16);
  return o;
}

// ---------------------------------------------------------------------------------------------
// Staging: K is staged 64 at a time (128-byte rows, one whole cache line per row per stage). The
// 160 KB of LDS hold two A buffers and three B buffers of 32 KB: A is fetched one stage ahead,
// the weight tile B (fewer CUs share it, so more of it misses L2) two stages ahead. Each
// wave-level DMA instruction writes 1 KB = 8 rows x 128 B;
// lane l of it fetches the global chunk that belongs at row l / 8, chunk position l % 8. The
// logical chunk c of row r sits at position c ^ ((r >> 1) & 7), so 16 consecutive rows read at
// one logical chunk hit 16 distinct 16-byte slots of a 256-byte bank line (conflict free).
// ---------------------------------------------------------------------------------------------
constexpr int kBK = 64;
constexpr int kTile = kBM * kBK * 2;     // bytes per operand per stage (32 KB)
constexpr int kLds = 5 * kTile;          // A0 A1 B0 B1 B2 (160 KB)

__device__ __forceinline__ int swz(int row, int chunk) {  // byte offset in a 256x128B tile
  return row * (kBK * 2) + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <int IPW>
struct Dma {
  i32x4_t ra, rb0, rb1;
  uint32_t aoff[IPW], boff[IPW];   // per-lane byte offsets of the thread's A and B rows
};

// MFMA block edge ME: 32 (v_mfma_f32_32x32x16_bf16, a k-step covers 16 of K) or 16
// (v_mfma_f32_16x16x32_bf16, a k-step covers 32 of K). Operand fragments: lane l holds row (or
// weight row) l % ME and 16-byte chunk l / ME of the k-step. Accumulator element e of block
// (i, j) in lane l: row acc_row<ME>(e, l), column acc_col<ME>(l) inside the block.
template <int ME> struct AccOf;
template <> struct AccOf<32> { using type = f32x16_t; static constexpr int n = 16; };
template <> struct AccOf<16> { using type = f32x4_t; static constexpr int n = 4; };
template <int ME> using acc_t = typename AccOf<ME>::type;

template <int ME>
__device__ __forceinline__ int acc_row(int e, int lane) {
  return ME == 32 ? (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3) : (lane >> 4) * 4 + e;
}
template <int ME>
__device__ __forceinline__ int acc_col(int lane) { return lane & (ME - 1); }

template <int MI, int NJ>
struct Frag {
  bf16x8_t a[MI], b[NJ];
};

// First tile column of column block j: gate/up puts the first NJ/2 blocks on gate rows and the
// rest on the matching up rows.
template <int MODE, int ME, int NJ>
__device__ __forceinline__ int col_base(int bcol0, int j) {
  return MODE == kGateUp ? (j < NJ / 2 ? bcol0 + j * ME : 128 + bcol0 + (j - NJ / 2) * ME)
                         : bcol0 + j * ME;
}

template <int MODE, int ME, int MI, int NJ>
__device__ __forceinline__ void read_frags(Frag<MI, NJ>& f, const char* As, const char* Bs,
                                           int arow0, int bcol0, int ks, int lane) {
  const int ch = (ME == 32 ? 2 : 4) * ks + lane / ME;
#pragma unroll
  for (int i = 0; i < MI; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8_t*>(As + swz(arow0 + i * ME + (lane & (ME - 1)), ch));
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8_t*>(
        Bs + swz(col_base<MODE, ME, NJ>(bcol0, j) + (lane & (ME - 1)), ch));
}

template <int ME, int MI, int NJ>
__device__ __forceinline__ void mfma_frags(acc_t<ME> (&acc)[MI][NJ], const Frag<MI, NJ>& f) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (ME == 32)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    }
}

// Instruction order of one k-step: its MFMAs with the next k-step's MI + NJ fragment reads
// (ds_read_b128) spread among them, one read after every two 16x16x32 MFMAs or after every
// 32x32x16 MFMA, the remaining MFMAs last. Left to itself the scheduler issues all reads first
// and then the MFMAs; spreading them keeps the matrix pipe fed while the reads drain
// (measured on the Mixtral-shaped prefill: gate/up -4.5 %, down unchanged).
template <int ME, int MI, int NJ>
__device__ __forceinline__ void spread_frag_reads() {
  constexpr int kPer = ME == 16 ? 2 : 1;
  static_assert(MI * NJ >= kPer * (MI + NJ), "enough MFMAs to spread the reads over");
#pragma unroll
  for (int q = 0; q < MI + NJ; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MI * NJ - kPer * (MI + NJ), 0);
}

// ---- four waves of 128x128 (one wave per SIMD) ------------------------------------------------
// With one wave per SIMD nothing else feeds the matrix pipe while a wave issues DMA or reads
// fragments, so one k-step's work is issued as groups: a few MFMAs, one fragment read of the next
// k-step, and the group's share of the stage's 16 DMA instructions (8 of A, then 8 of B), each
// group fenced so the compiler keeps the order.
template <int ME, int MI, int NJ>
struct Sched4 {
  static constexpr int kNM = MI * NJ;                 // MFMAs per k-step
  static constexpr int kNR = MI + NJ;                 // fragment reads per k-step
  static constexpr int kPer = kNM / kNR;              // MFMAs per group
  static constexpr int kKS = (kBK / 8) / (ME == 32 ? 2 : 4);   // k-steps per stage
  static constexpr int kPre = (kKS - 1) * kNR;        // groups before the stage's barrier
  static_assert(kNM % kNR == 0, "whole groups");
};

// One k-step: the MFMAs of `cur`, the reads of `nxt` (k-step ks_next of As / Bs), and, with
// kDma, DMA instructions m whose group (m * kPre / 16) falls in [g0, g0 + kNR).
template <int MODE, int ME, int MI, int NJ, bool kDma>
__device__ __forceinline__ void kstep4(acc_t<ME> (&acc)[MI][NJ], const Frag<MI, NJ>& cur,
                                       Frag<MI, NJ>& nxt, const char* As, const char* Bs,
                                       int arow0, int bcol0, int ks_next, int lane, int g0,
                                       const Dma<8>& d, uint32_t abase, uint32_t kba,
                                       uint32_t bbase, uint32_t kbb, int wave, int rows) {
  using S4 = Sched4<ME, MI, NJ>;
  const int ch = (ME == 32 ? 2 : 4) * ks_next + lane / ME;
#pragma unroll
  for (int g = 0; g < S4::kNR; ++g) {
#pragma unroll
    for (int q = 0; q < S4::kPer; ++q) {
      const int idx = g * S4::kPer + q;
      const int i = idx / NJ, j = idx % NJ;
      if constexpr (ME == 32)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
    }
    if (g < MI)
      nxt.a[g] = *reinterpret_cast<const bf16x8_t*>(As + swz(arow0 + g * ME + (lane & (ME - 1)), ch));
    else
      nxt.b[g - MI] = *reinterpret_cast<const bf16x8_t*>(
          Bs + swz(col_base<MODE, ME, NJ>(bcol0, g - MI) + (lane & (ME - 1)), ch));
    if constexpr (kDma) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        if ((m * S4::kPre) / 16 != g0 + g) continue;
        if (m < 8) {
          if ((wave * 8 + m) * 8 < rows) dma16(abase + (wave * 8 + m) * 1024, d.aoff[m], d.ra, kba);
        } else {
          dma16(bbase + (wave * 8 + m - 8) * 1024, d.boff[m - 8], wave < 2 ? d.rb0 : d.rb1, kbb);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// DMA of stage `st` of one operand into one buffer. The first DW waves issue all of it: wave
// w < DW fills rows (IPW w + i) * 8 .. +7 (i < IPW = 32 / DW); waves w >= DW issue none. A rows
// at or past the tile's valid rows are skipped (their waves skip the MFMAs); B rows 0..127 come
// from rb0, rows 128..255 from rb1. Stages past `last` (the prefetches the loop issues beyond the
// piece's end) get an offset past the buffer's range: the loads return zeros without touching
// memory, their buffers are never read, and every stage still issues the same instructions, so
// the loop's vmcnt waits stay uniform. (Buffer byte offsets stay below 2^31, so offset + 2^31
// does not wrap.)
constexpr uint32_t kPastEnd = 0x80000000u;

template <int DW>
__device__ __forceinline__ void dma_a(const char* buf, const Dma<32 / DW>& d, int st, int last,
                                      int wave, int rows) {
  constexpr int IPW = 32 / DW;
  if (wave >= DW) return;
  const uint32_t kb = st <= last ? static_cast<uint32_t>(st) * kBK * 2u : kPastEnd;
  const uint32_t base = lds_offset(buf);
#pragma unroll
  for (int i = 0; i < IPW; ++i)
    if ((wave * IPW + i) * 8 < rows) dma16(base + (wave * IPW + i) * 1024, d.aoff[i], d.ra, kb);
}

template <int DW>
__device__ __forceinline__ void dma_b(const char* buf, const Dma<32 / DW>& d, int st, int last,
                                      int wave) {
  constexpr int IPW = 32 / DW;
  if (wave >= DW) return;
  const uint32_t kb = st <= last ? static_cast<uint32_t>(st) * kBK * 2u : kPastEnd;
  const uint32_t base = lds_offset(buf);
#pragma unroll
  for (int i = 0; i < IPW; ++i)
    dma16(base + (wave * IPW + i) * 1024, d.boff[i], wave * IPW < 16 ? d.rb0 : d.rb1, kb);
}

// Partial tiles of cut tiles: fp32, row-major [256 rows][256 tile columns]. Tile column c is
// output column n0 + c for the down GEMM; for gate/up, columns 0..127 are the gate and 128..255
// the up projections of h columns n0 .. n0+127. Each store instruction writes two 128-byte row
// segments.
constexpr int kSlotFloats = kBM * kBN;

template <int MODE, int ME, int MI, int NJ>
__device__ __forceinline__ void store_partial(const acc_t<ME> (&acc)[MI][NJ], float* partial,
                                              int slot, int arow0, int bcol0, int lane) {
  float* const dst = partial + static_cast<size_t>(slot) * kSlotFloats;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = col_base<MODE, ME, NJ>(bcol0, j) + acc_col<ME>(lane);
#pragma unroll
      for (int e = 0; e < AccOf<ME>::n; ++e)
        dst[(arow0 + i * ME + acc_row<ME>(e, lane)) * kBN + col] = acc[i][j][e];
    }
}

// Row -> pair and routing weight of the down GEMM's output rows (rows past the tile's valid rows
// repeat its last row; they are never stored).
template <int kThreads>
__device__ __forceinline__ void load_row_pairs(const Bf16GemmArgs& p, const TileCoord& tc,
                                               int* row_pair, float* row_w, int tid) {
  for (int r = tid; r < kBM; r += kThreads) {
    const int rr = min(r, tc.rows - 1);
    const int pair = p.sorted_pair[tc.row0 + rr];
    row_pair[r] = pair;
    row_w[r] = p.topk_w ? p.topk_w[pair] : 1.0f;
  }
}

// LDS staging of the epilogue: gate/up h [256][136] bf16 (69632 B); down with bf16 output
// [256][264] bf16 (135168 B); down with fp32 output [64][260] fp32 per pass (66560 B).
constexpr int kStageBytes = kBM * 264 * 2;
static_assert(kStageBytes + kBM * 8 <= kLds, "row tables past the staging area");

// Epilogue of one finished 256 x 256 tile held in the accumulators: gate/up applies SwiGLU and
// stores the 256 x 128 h tile in bf16; down applies the routing weight and writes the requested
// output layout. row_pair / row_w are filled for the down GEMM.
template <int MODE, int WM, int WN, int ME>
__device__ __forceinline__ void tile_epilogue(acc_t<ME> (&acc)[kBM / WM / ME][kBN / WN / ME],
                                              const Bf16GemmArgs& p, const TileCoord& tc,
                                              char* lds, const int* row_pair,
                                              const float* row_w) {
  constexpr int kThreads = 64 * WM * WN;
  constexpr int MI = kBM / WM / ME;
  constexpr int NJ = kBN / WN / ME;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * (kBM / WM);
  const int bcol0 = MODE == kGateUp ? wn * (128 / WN) : wn * (kBN / WN);
  if (MODE == kGateUp) {
    // h tile [256 rows][128 cols] bf16, row stride 136 elements (69632 B of the ring).
    constexpr int kHS = 136;
    uint16_t* hs = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
        for (int e = 0; e < AccOf<ME>::n; ++e) {
          const int row = arow0 + i * ME + acc_row<ME>(e, lane);
          const int col = bcol0 + j * ME + acc_col<ME>(lane);
          hs[row * kHS + col] = f32_to_bf16_bits(silu_mul(acc[i][j][e], acc[i][j + NJ / 2][e]));
        }
    __syncthreads();
    const int n0 = tc.ntile * 128;
    for (int q = tid; q < kBM * 16; q += kThreads) {
      const int row = q >> 4, ch = q & 15;
      if (row < tc.rows && n0 + ch * 8 < p.N)
        *reinterpret_cast<u32x4_t*>(p.h + static_cast<size_t>(tc.row0 + row) * p.N + n0 + ch * 8) =
            *reinterpret_cast<const u32x4_t*>(hs + row * kHS + ch * 8);
    }
  } else if (p.y_bf16 && p.y_layout != MOE_Y_ACC_F32) {
    // bf16 rows (weighted for the slot layout): the whole tile staged once as [256][264] bf16,
    // every wave writing its rows, then 16-byte row segments to the output row of each pair
    // (slots) or sorted position (permuted). The 528-byte row stride puts the two 64-byte row
    // segments of one write instruction (rows r and r + 4) in different banks.
    constexpr int kYS = 264;
    uint16_t* ys = reinterpret_cast<uint16_t*>(lds);
    const bool weighted = p.y_layout == MOE_Y_SLOTS;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int e = 0; e < AccOf<ME>::n; ++e) {
        const int row = arow0 + i * ME + acc_row<ME>(e, lane);
        const float wgt = weighted ? row_w[row] : 1.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          ys[row * kYS + bcol0 + j * ME + acc_col<ME>(lane)] = f32_to_bf16_bits(acc[i][j][e] * wgt);
      }
    }
    __syncthreads();
    const int n0 = tc.ntile * kBN;
    uint16_t* const y = static_cast<uint16_t*>(p.y);
    for (int q = tid; q < kBM * (kBN / 8); q += kThreads) {
      const int row = q / (kBN / 8), ch = q % (kBN / 8);
      const int col = n0 + ch * 8;
      if (row < tc.rows && col < p.N) {
        const size_t orow = weighted ? static_cast<size_t>(row_pair[row])
                                     : static_cast<size_t>(tc.row0 + row);
        *reinterpret_cast<u32x4_t*>(y + orow * p.N + col) =
            *reinterpret_cast<const u32x4_t*>(ys + row * kYS + ch * 8);
      }
    }
  } else {
    // Passes of 64 rows staged as fp32 [64][260] (66560 B of the ring).
    constexpr int kYS = 260;
    float* ys = reinterpret_cast<float*>(lds);
    const int n0 = tc.ntile * kBN;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int rbase = arow0 + i * ME;
        if (rbase >= q * 64 && rbase < q * 64 + 64) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < AccOf<ME>::n; ++e) {
              const int row = rbase - q * 64 + acc_row<ME>(e, lane);
              const int col = bcol0 + j * ME + acc_col<ME>(lane);
              ys[row * kYS + col] = acc[i][j][e];
            }
        }
      }
      __syncthreads();
      for (int e = tid; e < 64 * 64; e += kThreads) {
        const int rl = e >> 6, c4 = (e & 63) * 4;
        const int row = q * 64 + rl;
        const int col = n0 + c4;
        if (row < tc.rows && col < p.N) {
          float4 v = *reinterpret_cast<const float4*>(ys + rl * kYS + c4);
          if (p.y_layout == MOE_Y_PERMUTED) {
            const size_t idx = static_cast<size_t>(tc.row0 + row) * p.N + col;
            if (p.y_bf16) *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.y) + idx) = pack_bf16x4(v);
            else *reinterpret_cast<float4*>(static_cast<float*>(p.y) + idx) = v;
          } else {
            const float wgt = row_w[row];
            v.x *= wgt; v.y *= wgt; v.z *= wgt; v.w *= wgt;
            const int pair = row_pair[row];
            if (p.y_layout == MOE_Y_SLOTS) {
              const size_t idx = static_cast<size_t>(pair) * p.N + col;
              if (p.y_bf16) *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.y) + idx) = pack_bf16x4(v);
              else *reinterpret_cast<float4*>(static_cast<float*>(p.y) + idx) = v;
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

template <int MODE, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(Bf16GemmArgs p) {
  constexpr int NW = WM * WN;
  constexpr int kThreads = 64 * NW;
  // Waves issuing the stage DMA. In the gate/up GEMM only one wave per SIMD does (measured 3 %
  // faster there: the SIMD's other wave keeps the MFMA pipe fed while the DMA wave waits for the
  // texture unit's queue); in the down GEMM all waves share it.
  constexpr int DW = NW == 4 ? NW : (MODE == kGateUp ? NW / 2 : NW);
  constexpr int IPW = 32 / DW;     // DMA instructions per DMA wave per operand per stage
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  // MFMA shape: 16x16x32 for gate/up, 32x32x16 for down (each measured the faster there)
  constexpr int ME = MODE == kGateUp ? 16 : 32;
  constexpr int MI = kBM / WM / ME;
  constexpr int NJ = kBN / WN / ME;
  const int NT = MODE == kGateUp ? (p.N + 127) / 128 : (p.N + kBN - 1) / kBN;
  WorkUnit wu;
  if (!map_work(p.tile_cum, p.offsets, p.E, kBM, NT, p.cpx, p.max_split, wu)) return;
  // the tile coordinates are block-uniform; say so, so descriptors and LDS bases live in SGPRs
  TileCoord tc;
  tc.e = __builtin_amdgcn_readfirstlane(wu.tc.e);
  tc.row0 = __builtin_amdgcn_readfirstlane(wu.tc.row0);
  tc.rows = __builtin_amdgcn_readfirstlane(wu.tc.rows);
  tc.ntile = __builtin_amdgcn_readfirstlane(wu.tc.ntile);
  const int split = __builtin_amdgcn_readfirstlane(wu.split);
  const int nsplit = __builtin_amdgcn_readfirstlane(wu.nsplit);

  // All of LDS: A0 A1 B0 B1 B2; after the main loop the epilogue reuses it (staging from 0,
  // the down GEMM's row -> pair / weight tables past the staging area).
  __shared__ __attribute__((aligned(1024))) char ring[kLds];
  char* const a0 = ring;
  char* const a1 = ring + kTile;
  char* const b0 = ring + 2 * kTile;
  char* const b1 = ring + 3 * kTile;
  char* const b2 = ring + 4 * kTile;
  // the down GEMM's row tables sit past the epilogue's staging area (at most kStageBytes)
  int* const row_pair = reinterpret_cast<int*>(ring + kStageBytes);
  float* const row_w = reinterpret_cast<float*>(ring + kStageBytes + kBM * sizeof(int));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * (kBM / WM);
  const int bcol0 = MODE == kGateUp ? wn * (128 / WN) : wn * (kBN / WN);

  // this piece's stages: [st0, st0 + nst) of the K / kBK stages
  const int st_all = p.K / kBK;
  const int st0 = split * st_all / nsplit;
  const int nst = (split + 1) * st_all / nsplit - st0;
  const int last = st0 + nst - 1;

  // DMA addressing: lane l of instruction i of wave w supplies row (IPW w + i) * 8 + l / 8 at
  // chunk position l % 8.
  Dma<IPW> d;
  const size_t wstride = static_cast<size_t>(p.N) * p.K;
  d.ra = make_rsrc(p.a, static_cast<uint32_t>(p.a_rows) * p.K * 2u);
  d.rb0 = make_rsrc(p.b0 + tc.e * wstride, static_cast<uint32_t>(p.N) * p.K * 2u);
  d.rb1 = MODE == kGateUp ? make_rsrc(p.b1 + tc.e * wstride, static_cast<uint32_t>(p.N) * p.K * 2u)
                          : d.rb0;
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int pos = tc.row0 + min(r, tc.rows - 1);
    const int arow = p.a_gather ? p.sorted_pair[pos] / p.k : pos;
    d.aoff[i] = static_cast<uint32_t>(arow) * p.K * 2u + c * 16;
    const int n = MODE == kGateUp ? min(tc.ntile * 128 + (r & 127), p.N - 1)
                                  : min(tc.ntile * kBN + r, p.N - 1);
    d.boff[i] = static_cast<uint32_t>(n) * p.K * 2u + c * 16;
  }

  acc_t<ME> acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < AccOf<ME>::n; ++e) acc[i][j][e] = 0.0f;

  dma_a<DW>(a0, d, st0, last, wave, tc.rows);
  dma_b<DW>(b0, d, st0, last, wave);
  dma_b<DW>(b1, d, st0 + 1, last, wave);
  wait_vmcnt<IPW>();  // all but this wave's B DMAs of stage 1
  __builtin_amdgcn_s_barrier();
  // Waves whose rows all lie past the tile's valid rows (the short last tile of an expert) skip
  // their fragment reads and MFMAs; the condition is wave-uniform.
  const bool active = arow0 < tc.rows;
  Frag<MI, NJ> fa, fb;
  if (active) read_frags<MODE, ME, MI, NJ>(fa, a0, b0, arow0, bcol0, 0, lane);

  // Stage S computes from A buffer AC and B buffer BC, with its k-step-0 fragments already in fa.
  // It first issues the DMA of A for stage S+1 into AN and of B for stage S+2 into BN2 (both
  // buffers were last read in stage S-1, which every wave finished, LDS reads included, before
  // the last barrier), then runs its k-steps but the last (4 of 16 K for ME = 32, 2 of 32 K for
  // ME = 16), reading each k-step's fragments during the previous one's MFMAs. It then waits until
  // only this wave's B DMAs of stage S+2 are in flight and its LDS reads are done; after the
  // barrier, all of stage S+1 (A in AN, B in BN1) is in LDS, and its k-step-0 fragments are read
  // while the last k-step of stage S runs.
#define MOE_STAGE(AC, BC, AN, BN1, BN2, S)                                           \
  {                                                                                  \
    dma_a<DW>(AN, d, st0 + (S) + 1, last, wave, tc.rows);                            \
    dma_b<DW>(BN2, d, st0 + (S) + 2, last, wave);                                    \
    if (active) {                                                                    \
      read_frags<MODE, ME, MI, NJ>(fb, AC, BC, arow0, bcol0, 1, lane);               \
      mfma_frags<ME, MI, NJ>(acc, fa);                                               \
      spread_frag_reads<ME, MI, NJ>();                                               \
      if constexpr (ME == 32) {                                                      \
        read_frags<MODE, ME, MI, NJ>(fa, AC, BC, arow0, bcol0, 2, lane);             \
        mfma_frags<ME, MI, NJ>(acc, fb);                                             \
        spread_frag_reads<ME, MI, NJ>();                                             \
        read_frags<MODE, ME, MI, NJ>(fb, AC, BC, arow0, bcol0, 3, lane);             \
        mfma_frags<ME, MI, NJ>(acc, fa);                                             \
        spread_frag_reads<ME, MI, NJ>();                                             \
      }                                                                              \
    }                                                                                \
    wait_vmcnt_lgkm0<IPW>();                                                         \
    __builtin_amdgcn_s_barrier();                                                    \
    if (active) {                                                                    \
      read_frags<MODE, ME, MI, NJ>(fa, AN, BN1, arow0, bcol0, 0, lane);              \
      mfma_frags<ME, MI, NJ>(acc, fb);                                               \
      spread_frag_reads<ME, MI, NJ>();                                               \
    }                                                                                \
  }
  if constexpr (NW == 4) {
    // Stage S: k-steps but the last with the DMA of A (S+1) -> AN and B (S+2) -> BN2 spread
    // through them, then the wait for stage S+1 and the barrier, then the last k-step with the
    // reads of stage S+1's first k-step. A wave whose rows lie past the tile issues its DMA only.
    using S4 = Sched4<ME, MI, NJ>;
#define MOE_STAGE4(AC, BC, AN, BN1, BN2, S)                                                     \
    {                                                                                          \
      const int sa = st0 + (S) + 1, sb = st0 + (S) + 2;                                        \
      const uint32_t kba = sa <= last ? static_cast<uint32_t>(sa) * kBK * 2u : kPastEnd;       \
      const uint32_t kbb = sb <= last ? static_cast<uint32_t>(sb) * kBK * 2u : kPastEnd;       \
      const uint32_t abase = lds_offset(AN), bbase = lds_offset(BN2);                          \
      if (active) {                                                                            \
        _Pragma("unroll") for (int ks = 0; ks < S4::kKS - 1; ++ks) {                           \
          if (ks % 2 == 0)                                                                     \
            kstep4<MODE, ME, MI, NJ, true>(acc, fa, fb, AC, BC, arow0, bcol0, ks + 1, lane,    \
                                           ks * S4::kNR, d, abase, kba, bbase, kbb, wave,      \
                                           tc.rows);                                           \
          else                                                                                 \
            kstep4<MODE, ME, MI, NJ, true>(acc, fb, fa, AC, BC, arow0, bcol0, ks + 1, lane,    \
                                           ks * S4::kNR, d, abase, kba, bbase, kbb, wave,      \
                                           tc.rows);                                           \
        }                                                                                      \
      } else {                                                                                 \
        dma_a<DW>(AN, d, sa, last, wave, tc.rows);                                             \
        dma_b<DW>(BN2, d, sb, last, wave);                                                     \
      }                                                                                        \
      wait_vmcnt_lgkm0<IPW>();                                                                 \
      __builtin_amdgcn_s_barrier();                                                            \
      if (active)                                                                              \
        kstep4<MODE, ME, MI, NJ, false>(acc, fb, fa, AN, BN1, arow0, bcol0, 0, lane, 0, d,     \
                                        0u, 0u, 0u, 0u, wave, tc.rows);                        \
    }
    for (int s = 0; s < nst; s += 6) {
      MOE_STAGE4(a0, b0, a1, b1, b2, s)
      if (s + 1 < nst) MOE_STAGE4(a1, b1, a0, b2, b0, s + 1)
      if (s + 2 < nst) MOE_STAGE4(a0, b2, a1, b0, b1, s + 2)
      if (s + 3 < nst) MOE_STAGE4(a1, b0, a0, b1, b2, s + 3)
      if (s + 4 < nst) MOE_STAGE4(a0, b1, a1, b2, b0, s + 4)
      if (s + 5 < nst) MOE_STAGE4(a1, b2, a0, b0, b1, s + 5)
    }
#undef MOE_STAGE4
  } else {
  // buffers of stage s: A a[s % 2], B b[s % 3]; the pattern repeats every 6 stages
  for (int s = 0; s < nst; s += 6) {
    MOE_STAGE(a0, b0, a1, b1, b2, s)
    if (s + 1 < nst) MOE_STAGE(a1, b1, a0, b2, b0, s + 1)
    if (s + 2 < nst) MOE_STAGE(a0, b2, a1, b0, b1, s + 2)
    if (s + 3 < nst) MOE_STAGE(a1, b0, a0, b1, b2, s + 3)
    if (s + 4 < nst) MOE_STAGE(a0, b1, a1, b2, b0, s + 4)
    if (s + 5 < nst) MOE_STAGE(a1, b2, a0, b0, b1, s + 5)
  }
  }
#undef MOE_STAGE
  wait_vmcnt<0>();  // the past-the-end prefetches (no memory traffic)
  __syncthreads();

  if (nsplit > 1) {
    // a piece of a cut tile: store the partial in register order and leave the rest to the fix-up
    store_partial<MODE, ME, MI, NJ>(acc, p.partial, wu.part_slot, arow0, bcol0, lane);
    return;
  }
  if (MODE == kDown) {
    load_row_pairs<kThreads>(p, tc, row_pair, row_w, tid);
    __syncthreads();
  }
  tile_epilogue<MODE, WM, WN, ME>(acc, p, tc, ring, row_pair, row_w);
}


// Fix-up of the cut tiles, element-wise: kFixBlocks blocks of 256 threads per cut-tile slot, each
// covering 8 tile rows. A thread adds the pieces' partials in piece order (fp32) for 4 columns
// and applies the same epilogue as the GEMM: gate/up -> SwiGLU -> bf16 h; down -> routing weight
// -> requested layout.
constexpr int kFixRows = 8;
constexpr int kFixBlocks = kBM / kFixRows;

template <int MODE>
__global__ __launch_bounds__(256) void fixup_bf16_kernel(Bf16GemmArgs p) {
  const int NT = MODE == kGateUp ? (p.N + 127) / 128 : (p.N + kBN - 1) / kBN;
  TileCoord tc;
  int nsplit, slot0;
  if (!map_cut_tile(p.tile_cum, p.offsets, p.E, kBM, NT, p.cpx, p.max_split,
                    blockIdx.x / kFixBlocks, tc, nsplit, slot0))
    return;
  const int tid = threadIdx.x;
  const float* const src = p.partial + static_cast<size_t>(slot0) * kSlotFloats;
  if (MODE == kGateUp) {
    // 8 rows x 128 h columns: thread -> row tid / 32, h columns 4 (tid % 32) .. +3
    const int row = (blockIdx.x % kFixBlocks) * kFixRows + tid / 32;
    const int c = (tid % 32) * 4;
    const int n = tc.ntile * 128 + c;
    if (row >= tc.rows || n >= p.N) return;
    const float* q = src + row * kBN + c;
    f32x4_t g = *reinterpret_cast<const f32x4_t*>(q);
    f32x4_t u = *reinterpret_cast<const f32x4_t*>(q + 128);
    for (int t = 1; t < nsplit; ++t) {
      g += *reinterpret_cast<const f32x4_t*>(q + static_cast<size_t>(t) * kSlotFloats);
      u += *reinterpret_cast<const f32x4_t*>(q + static_cast<size_t>(t) * kSlotFloats + 128);
    }
    const float4 h = make_float4(silu_mul(g[0], u[0]), silu_mul(g[1], u[1]),
                                 silu_mul(g[2], u[2]), silu_mul(g[3], u[3]));
    *reinterpret_cast<u32x2_t*>(p.h + static_cast<size_t>(tc.row0 + row) * p.N + n) =
        pack_bf16x4(h);
  } else {
    // 8 rows x 256 output columns in two passes of 4 rows: thread -> column 4 (tid % 64) .. +3
    const int c = (tid % 64) * 4;
    const int col = tc.ntile * kBN + c;
    if (col >= p.N) return;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int row = (blockIdx.x % kFixBlocks) * kFixRows + pass * 4 + tid / 64;
      if (row >= tc.rows) break;
      const float* q = src + row * kBN + c;
      f32x4_t a = *reinterpret_cast<const f32x4_t*>(q);
      for (int t = 1; t < nsplit; ++t)
        a += *reinterpret_cast<const f32x4_t*>(q + static_cast<size_t>(t) * kSlotFloats);
      float4 v = make_float4(a[0], a[1], a[2], a[3]);
      const int pos = tc.row0 + row;
      if (p.y_layout == MOE_Y_PERMUTED) {
        const size_t idx = static_cast<size_t>(pos) * p.N + col;
        if (p.y_bf16) *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.y) + idx) = pack_bf16x4(v);
        else *reinterpret_cast<float4*>(static_cast<float*>(p.y) + idx) = v;
      } else {
        const int pair = p.sorted_pair[pos];
        const float wgt = p.topk_w ? p.topk_w[pair] : 1.0f;
        v.x *= wgt; v.y *= wgt; v.z *= wgt; v.w *= wgt;
        if (p.y_layout == MOE_Y_SLOTS) {
          const size_t idx = static_cast<size_t>(pair) * p.N + col;
          if (p.y_bf16) *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.y) + idx) = pack_bf16x4(v);
          else *reinterpret_cast<float4*>(static_cast<float*>(p.y) + idx) = v;
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
}

inline long max_tiles(int P, int E, int NT) {
  return static_cast<long>(max_row_tiles(P, E, kBM)) * NT;
}

// K pieces a tail tile may be cut into: at least 8 stages (512 of K) per piece, at most 8 pieces.
inline int max_split_for(int K) { return std::max(1, std::min(8, K / kBK / 8)); }

// Tiles are cut only on XCDs with at most kCutMaxRounds whole rounds. An XCD holds at least
// (total - 49) / 8 tiles, and total >= NT * ceil(P / kBM); when even that bound leaves every XCD
// more rounds, no tile can be cut and neither cutting nor the fix-up launch is needed.
inline bool may_cut(int P, int NT, int cpx) {
  const long min_tiles = static_cast<long>(NT) * ((P + kBM - 1) / kBM);
  return (min_tiles - 49) / 8 < static_cast<long>(kCutMaxRounds + 1) * cpx;
}

}  // namespace

int bf16_tile_rows_gateup() { return kBM; }
int bf16_tile_rows_down() { return kBM; }

// Wave layout: WM x WN waves, each owning (256/WM) x (256/WN); the gate/up GEMM and short-K down
// GEMMs take 4 x 2, down GEMMs with K >= MOE_BF16_DOWN4_MIN_K (4096) take 2 x 2 (measured faster there).
#ifndef MOE_BF16_WAVES
#define MOE_BF16_WAVES 4, 2
#endif
#ifndef MOE_BF16_DOWN4_MIN_K
#define MOE_BF16_DOWN4_MIN_K 4096
#endif

// The GEMM, then (when tail tiles may be cut) the fix-up of the cut tiles.
template <int MODE, int WM, int WN>
hipError_t launch_gemm(const Bf16GemmArgs& g, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, WM, WN>), dim3(grid), dim3(64 * WM * WN), 0, stream,
                     g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.max_split < 2) return e;
  hipLaunchKernelGGL((fixup_bf16_kernel<MODE>), dim3(8 * g.cpx * kFixBlocks), dim3(256), 0, stream,
                     g);
  return hipGetLastError();
}

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
  g.a_rows = L.a_gather ? L.T : P;
  g.offsets = L.offsets;
  g.tile_cum = L.tile_cum_a;
  g.E = L.E;
  g.h = static_cast<uint16_t*>(L.h);
  g.cpx = L.cpx;
  g.max_split =
      L.split_partial && may_cut(P, (L.f + 127) / 128, L.cpx) ? max_split_for(L.d) : 1;
  g.partial = L.split_partial;
  if (L.run_gate_up) {
    const hipError_t e = launch_gemm<kGateUp, MOE_BF16_WAVES>(
        g, work_grid(max_tiles(P, L.E, (L.f + 127) / 128), L.cpx), stream);
    if (e != hipSuccess) return e;
  }
  if (!L.run_down) return hipSuccess;

  Bf16GemmArgs dn{};
  dn.a = static_cast<const uint16_t*>(L.h);
  dn.a_gather = 0;
  dn.sorted_pair = L.sorted_pair;
  dn.k = L.k;
  dn.b0 = static_cast<const uint16_t*>(L.w_down);
  dn.K = L.f;
  dn.N = L.d;
  dn.a_rows = P;
  dn.offsets = L.offsets;
  dn.tile_cum = L.tile_cum_b;
  dn.E = L.E;
  dn.y = L.y;
  dn.y_layout = L.y_layout;
  dn.y_bf16 = L.y_bf16;
  dn.topk_w = L.topk_w;
  dn.cpx = L.cpx;
  dn.max_split =
      L.split_partial && may_cut(P, (L.d + kBN - 1) / kBN, L.cpx) ? max_split_for(L.f) : 1;
  dn.partial = L.split_partial;
  const unsigned grid2 = work_grid(max_tiles(P, L.E, (L.d + kBN - 1) / kBN), L.cpx);
  if (L.f >= MOE_BF16_DOWN4_MIN_K) return launch_gemm<kDown, 2, 2>(dn, grid2, stream);
  return launch_gemm<kDown, MOE_BF16_WAVES>(dn, grid2, stream);
}

}  // namespace moe
