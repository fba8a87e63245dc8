// Internal helpers shared by the HIP sources of libmoe (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kFp8Group = 128;   // activation group width and weight block edge

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;
// Raw 16-byte vector (a native vector type, so copies stay in registers).
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// ---- scalar formats -------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  // gfx950 converts in hardware (v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN)
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// UE8M0 scale byte b (value 2^(b - 127)) of a group with absolute maximum amax: the smallest e
// with 448 * 2^e >= amax, e = 0 for amax = 0, clamped to 0..254. With amax = fr * 2^ex,
// fr in [0.5, 1) (frexp, exact also for subnormals) and 448 = 0.875 * 2^9, the condition reads
// 2^(e + 9 - ex) >= fr / 0.875, whose least solution is e = ex - 9, plus one when fr > 0.875.
__device__ __forceinline__ int ue8m0_byte(float amax) {
  if (!(amax > 0.0f)) return 127;
  const int ex = __builtin_amdgcn_frexp_expf(amax);
  const float fr = __builtin_amdgcn_frexp_mantf(amax);
  const int e = ex - 9 + (fr > 0.875f ? 1 : 0);
  return min(254, max(0, e + 127));
}

// OCP E2M1 (FP4) code of v (|v| rounded to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to
// the even code, beyond 6 saturating): each threshold adds one code step; at a midpoint the
// comparison is strict when the lower code is even and inclusive when it is odd.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return c | (signbit(v) ? 8u : 0u);
}

// MX scale byte for E2M1 blocks: the smallest e with 6 * 2^e >= amax (0 -> byte 127), clamped to
// 0..254. With amax = fr * 2^ex, fr in [0.5, 1), and 6 = 0.75 * 2^3: e = ex - 3, plus one when
// fr > 0.75.
__device__ __forceinline__ int mx4_byte(float amax) {
  if (!(amax > 0.0f)) return 127;
  const int ex = __builtin_amdgcn_frexp_expf(amax);
  const float fr = __builtin_amdgcn_frexp_mantf(amax);
  const int e = ex - 3 + (fr > 0.75f ? 1 : 0);
  return min(254, max(0, e + 127));
}

// OCP E4M3FN encode: round to nearest even, saturate to +-448 (0x7E / 0xFE); zero keeps its sign.
// Normal range: round the fp32 mantissa from 23 to 3 bits with the add-half-minus-one-plus-lsb
// trick, then rebias the exponent (fp32 bias 127 -> e4m3 bias 7). Below 2^-6 the e4m3 grid is the
// uniform subnormal step 2^-9, so the code is rint(|v| * 2^9).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a >= 0x43e00000u) return sign | 0x7eu;                 // |v| >= 448 (and inf/nan)
  if (a < 0x3c800000u) {                                     // |v| < 2^-6
    float m = rintf(__uint_as_float(a) * 512.0f);
    return sign | static_cast<uint32_t>(m);
  }
  uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t ex = (c >> 3) & 0xfu, man = c & 0x7u;
  float v = ex == 0 ? static_cast<float>(man) * 0x1p-9f
                    : __uint_as_float(((ex + 120u) << 23) | (man << 20));
  return (c & 0x80u) ? -v : v;
}

// ---- wave helpers -------------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// A 32-bit value from another lane of the same 16-lane row by a DPP move (no LDS round trip).
// Controls used here: lane ^ 1 and lane ^ 2 (quad permutes [1,0,3,2] and [2,3,0,1]), lane i <->
// 7 - i within eight (row half mirror) and lane i <-> 15 - i within sixteen (row mirror). Applied
// in that order to a commutative reduction they leave every lane of a 2, 4, 8 or 16-lane group
// with the group's result: each step pairs a lane with one of the other block of the next size.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(v)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  // the hardware reciprocal (1 ulp) instead of an IEEE division: the result is rounded to bf16
  // or quantised afterwards, far coarser than either
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---- global -> LDS DMA ---------------------------------------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = N and expcnt / lgkmcnt left at their maximum (no wait)
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  // s_waitcnt with vmcnt = N, lgkmcnt = 0 (this wave's LDS reads done), expcnt not waited on
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

// Buffer resource for raw byte addressing of [base, base + bytes) (out-of-range reads return 0).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = static_cast<int>(a & 0xffffffffu);
  r[1] = static_cast<int>(a >> 32);   // stride 0
  r[2] = static_cast<int>(bytes);
  r[3] = 0x00020000;                  // raw buffer, 32-bit data format
  return r;
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<size_t>((const __attribute__((address_space(3))) char*)(p)));
}

// One wave-wide 16-byte-per-lane DMA from global memory straight into LDS: lane l's 16 bytes land
// at lds + 16 l. Issued as inline asm so the compiler does not add LDS-DMA waits of its own; the
// GEMM loop places explicit vmcnt waits before its barriers instead (there are no other vector
// memory instructions in that loop).
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4_t rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// Same as dma16 with 4 bytes per lane (lane l's dword lands at lds + 4 l); inactive lanes skip.
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, i32x4_t rsrc, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// ---- grouped-GEMM tile schedule ----------------------------------------------------------------
//
// The rows of a grouped GEMM are the P pairs in expert-sorted order; expert e owns rows
// [offsets[e], offsets[e+1]). A row tile never straddles two experts, so expert e contributes
// ceil(M_e / BM) row tiles. tile_cum[e] = number of row tiles of experts < e (tile_cum[E] = total).
// Logical tiles are numbered expert-major, then output-column tile, then row tile, so that the
// row tiles sharing one weight panel are adjacent and run together.

struct TileCoord {
  int e;       // expert
  int row0;    // first sorted row of the tile
  int rows;    // valid rows in the tile (1..BM)
  int ntile;   // output-column tile index
};

// Resolves logical tile `logical` (< tile_cum[E] * NT) to its expert, rows and column tile.
__device__ __forceinline__ void decode_tile(const int32_t* __restrict__ tile_cum,
                                            const int32_t* __restrict__ offsets, int E, int BM,
                                            int NT, int logical, TileCoord& tc) {
  // largest e with tile_cum[e] * NT <= logical (experts with no rows have equal tile_cum entries)
  int lo = 0, hi = E;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (tile_cum[mid] * NT <= logical) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int nrt = tile_cum[e + 1] - tile_cum[e];
  const int rem = logical - tile_cum[e] * NT;
  const int ntile = rem / nrt;
  const int rt = rem - ntile * nrt;
  const int start = offsets[e] + rt * BM;
  tc.e = e;
  tc.row0 = start;
  tc.rows = min(BM, offsets[e + 1] - start);
  tc.ntile = ntile;
}

// Maps a hardware block index to a tile; returns false for blocks beyond the real tile count.
// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD b % 8); each XCD is
// handed one contiguous range of logical tiles so that blocks sharing weight panels and input rows
// share that XCD's L2.
__device__ __forceinline__ bool map_tile(const int32_t* __restrict__ tile_cum,
                                         const int32_t* __restrict__ offsets, int E, int BM,
                                         int NT, TileCoord& tc) {
  const int total = tile_cum[E] * NT;
  const int chunk = (total + 7) / 8;
  const int b = blockIdx.x;
  const int slot = b >> 3;
  if (slot >= chunk) return false;
  const int logical = (b & 7) * chunk + slot;
  if (logical >= total) return false;
  decode_tile(tile_cum, offsets, E, BM, NT, logical, tc);
  return true;
}

// Split of the last, partial round. With one workgroup per CU and `cpx` CUs per XCD, an XCD
// holding n tiles runs floor(n / cpx) whole rounds; the tail = n mod cpx tiles of its last round
// would leave cpx - tail CUs idle, so each tail tile is cut into S = min(max_split, cpx / tail)
// contiguous K ranges run by S workgroups. Every piece stores its fp32 partial tile; a second
// kernel adds the S partials of each cut tile in piece order and runs the tile's epilogue.
// Tiles are cut only when the XCD has at most kCutMaxRounds whole rounds: over more rounds the
// CUs finish their tiles at scattered times and the last round is no longer an idle step.
constexpr int kCutMaxRounds = 4;
struct XcdShare {
  int base;   // first logical tile of the XCD
  int full;   // tiles run whole (a multiple of cpx)
  int tail;   // tiles of the last round
  int S;      // pieces per tail tile (1 = not cut)
};

__device__ __forceinline__ XcdShare xcd_share(int total, int x, int cpx, int max_split) {
  XcdShare r;
  const int chunk = (total + 7) / 8;
  r.base = x * chunk;
  const int n = max(0, min(chunk, total - r.base));
  r.full = n / cpx * cpx;
  r.tail = n - r.full;
  r.S = r.tail > 0 && r.full <= kCutMaxRounds * cpx ? max(1, min(max_split, cpx / r.tail)) : 1;
  return r;
}

struct WorkUnit {
  TileCoord tc;
  int split;       // piece index (0 for an uncut tile)
  int nsplit;      // pieces of this tile (1 = uncut)
  int part_slot;   // partial-tile slot of this piece, < 8 * cpx (pieces of a tile are adjacent)
};

__device__ __forceinline__ bool map_work(const int32_t* __restrict__ tile_cum,
                                         const int32_t* __restrict__ offsets, int E, int BM,
                                         int NT, int cpx, int max_split, WorkUnit& w) {
  const int b = blockIdx.x;
  const int x = b & 7, s = b >> 3;
  const XcdShare sh = xcd_share(tile_cum[E] * NT, x, cpx, max_split);
  int logical;
  if (s < sh.full) {
    logical = sh.base + s;
    w.split = 0;
    w.nsplit = 1;
    w.part_slot = 0;
  } else {
    const int u = s - sh.full;
    if (u >= sh.tail * sh.S) return false;
    logical = sh.base + sh.full + u / sh.S;
    w.split = sh.S > 1 ? u % sh.S : 0;
    w.nsplit = sh.S;
    w.part_slot = x * cpx + u;
  }
  decode_tile(tile_cum, offsets, E, BM, NT, logical, w.tc);
  return true;
}

// The cut tile handled by fix-up block c (< 8 * cpx): tail tile c % cpx of XCD c / cpx. Returns
// false when that tile does not exist or was not cut; slot0 is its first partial slot.
__device__ __forceinline__ bool map_cut_tile(const int32_t* __restrict__ tile_cum,
                                             const int32_t* __restrict__ offsets, int E, int BM,
                                             int NT, int cpx, int max_split, int c, TileCoord& tc,
                                             int& nsplit, int& slot0) {
  const int x = c / cpx, t = c % cpx;
  const XcdShare sh = xcd_share(tile_cum[E] * NT, x, cpx, max_split);
  if (t >= sh.tail || sh.S < 2) return false;
  nsplit = sh.S;
  slot0 = x * cpx + t * sh.S;
  decode_tile(tile_cum, offsets, E, BM, NT, sh.base + sh.full + t, tc);
  return true;
}

// ---- helpers of the fused small-batch path ----------------------------------------------------

// The pairs (flat index t * k + j) routed to expert e, in ascending order, found by one workgroup
// of NT threads in ids[0 .. P): those of rank skip .. skip + CAP - 1 written to list (LDS), their
// total number M returned to every thread. wsum: LDS scratch of NT / 64 ints. Ends with a
// barrier, so list is ready for the whole group.
template <int NT, int CAP>
__device__ int expert_pair_list(const int32_t* __restrict__ ids, int P, int e, int32_t* list,
                                int* wsum, int skip = 0) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  int total = 0;
  for (int base = 0; base < P; base += NT) {
    const int i = base + static_cast<int>(threadIdx.x);
    const bool hit = i < P && ids[i] == e;
    const uint64_t m = __ballot(hit);
    if (lane == 0) wsum[w] = __popcll(m);
    __syncthreads();
    int off = total, tot = 0;
#pragma unroll
    for (int v = 0; v < NT / kWave; ++v) {
      off += v < w ? wsum[v] : 0;
      tot += wsum[v];
    }
    const int at = off + __popcll(m & ((1ull << lane) - 1ull));
    if (hit && at >= skip && at < skip + CAP) list[at - skip] = i;
    total += tot;
    __syncthreads();
  }
  return total;
}

// One 128-wide fp8 group held by 16 consecutive lanes, 8 values each (lane & 15 = position): the
// group's amax over the 16 lanes, then the e4m3 codes of this lane's 8 values (lo: values 0..3,
// hi: 4..7) by the fp32 rule (s = amax / 448, code = e4m3(v / s), s = 1 for a zero group) or the
// UE8M0 rule (byte b, code = e4m3(v * 2^(127 - b))). Returns the scale's value (UE8M0: 2^(b - 127));
// *byte gets b. Every lane of the 16 must call it.
template <bool kUE>
__device__ __forceinline__ float quant_group16(const float (&v)[8], uint32_t& lo, uint32_t& hi,
                                               int* byte) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, dpp_f32<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_f32<kDppXor2>(amax));
  amax = fmaxf(amax, dpp_f32<kDppHalfMirror>(amax));
  amax = fmaxf(amax, dpp_f32<kDppMirror>(amax));
  lo = hi = 0;
  if constexpr (kUE) {
    const int b = ue8m0_byte(amax);
    const float inv = ldexpf(1.0f, 127 - b);
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3_encode(v[i] * inv) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3_encode(v[4 + i] * inv) << (8 * i);
    *byte = b;
    return ldexpf(1.0f, b - 127);
  } else {
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3_encode(v[i] / s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3_encode(v[4 + i] / s) << (8 * i);
    *byte = 0;
    return s;
  }
}

// Blocks to launch for map_work: per XCD at most chunk whole tiles plus cpx tail pieces.
inline unsigned work_grid(long max_tiles, int cpx) {
  return static_cast<unsigned>(((max_tiles + 7) / 8 + cpx) * 8);
}

// Upper bound on the number of row tiles: sum_e ceil(M_e/BM) <= floor(P/BM) + min(E, P).
inline int max_row_tiles(int P, int E, int BM) { return P / BM + (E < P ? E : P); }

}  // namespace moe
