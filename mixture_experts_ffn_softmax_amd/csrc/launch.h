// Kernel launchers of libmoe (internal). Arguments are validated by the C ABI layer before any of
// these is called; every launcher only enqueues work on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

hipError_t launch_router_logits(const void* x, moe_dtype x_dtype, const float* wr, int T, int d,
                                int E, float* logits, hipStream_t stream);
hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                               hipStream_t stream);

size_t permute_workspace_bytes(int P, int E);
hipError_t launch_permute(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, void* workspace,
                          hipStream_t stream);
hipError_t launch_gather_rows(const void* x, size_t row_bytes, const int32_t* sorted_pair, int P,
                              int k, void* x_perm, hipStream_t stream);

hipError_t launch_quantize_act(const void* x, moe_dtype x_dtype, int M, int K,
                               const int32_t* row_index, uint8_t* q, void* scales, bool ue8m0,
                               hipStream_t stream);
hipError_t launch_quantize_weight(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                                  uint8_t* q, void* scales, bool ue8m0, hipStream_t stream);
// FP4 E2M1 weights with MX scales: nblocks 32-element blocks (rows * K / 32)
hipError_t launch_quantize_weight_mx4(const void* w, moe_dtype w_dtype, size_t nblocks,
                                      uint8_t* q, uint8_t* scales, hipStream_t stream);
// packed E2M1 [rows, K/2] (rows % 16 == 0, K % 128 == 0) -> matrix-fragment order
hipError_t launch_tile_weight_fp4(const uint8_t* q, size_t rows, int K, uint8_t* out,
                                  hipStream_t stream);
// e8m0 bytes -> fp32 values 2^(b - 127)
hipError_t launch_e8m0_expand(const uint8_t* b, size_t n, float* out, hipStream_t stream);

hipError_t launch_combine(const void* y, moe_dtype y_dtype, moe_y_layout layout,
                          const int32_t* pair_pos, const float* topk_w, int T, int k, int d,
                          void* out, moe_dtype out_dtype, hipStream_t stream);

hipError_t launch_tile_table(const int32_t* offsets, int E, int bm_a, int bm_b, int32_t* cum_a,
                             int32_t* cum_b, hipStream_t stream);

// Cut tail tiles of the bf16 GEMMs: partial-tile slots per GEMM (8 XCDs x at most 32 CUs each),
// and the CUs per XCD the tile schedule assumes.
constexpr int kSplitSlots = 256;
int cus_per_xcd();

// Everything one experts forward needs, resolved by the ABI layer.
struct ExpertsLaunch {
  int T, d, f, E, k;
  const void* a;              // x [T, d] (a_gather = 1: row of pair = sorted_pair[pos] / k) or
  int a_gather;               // x_perm [P, d] in sorted order (a_gather = 0)
  const float* a_scales;      // fp8: [T, d/128] (gather) or [P, d/128], fp32 values (powers of
                              // two with UE8M0 weight scales)
  const int32_t* sorted_pair;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* s_gate;         // fp8 block scales: fp32, or e8m0 bytes when scale_ue8m0
  const void* s_up;
  const void* s_down;
  int scale_ue8m0;            // fp8: UE8M0 scales, applied by the block-scaled MFMA
  int w_fp4;                  // weights packed E2M1 with MX scales [E, rows, cols/32]
  const int32_t* offsets;
  const int32_t* tile_cum_a;  // row tiles of the gate/up GEMM
  const int32_t* tile_cum_b;  // row tiles of the down GEMM
  const float* topk_w;
  int y_layout;
  int y_bf16;
  void* y;
  void* h;                    // workspace: hidden activations [P, f]
  float* h_scales;            // fp8: [P, f/128] fp32 (powers of two when scale_ue8m0)
  float* h32;                 // fp8 decode: h [P, f] fp32 before its quantisation
  uint8_t* h_scale_bytes;     // fp8 decode with UE8M0 scales: [P, f/128] e8m0 bytes
  int cpx;                    // CUs per XCD (<= kSplitSlots / 8)
  float* split_partial;       // bf16 GEMMs: [kSplitSlots][256 * 256] fp32, or null (no cutting;
                              // the two GEMMs use it one after the other)
  int run_gate_up, run_down;  // which projections this call enqueues (the other one is skipped)
  // fp8 small-batch kernels with UE8M0 scales read the activation scales as e8m0 bytes:
  // a_scale_bytes [T, d/128] (or [P, d/128]) for x, h_scale_bytes for h
  const void* a_scale_bytes;
  // Fused small-batch path (decode kernels only): pair_ids non-null. Each workgroup finds its
  // expert's pairs in the routing ids [T * k] itself (no offsets or sorted_pair); h, its scales
  // and the slots y [P, d] are indexed by pair.
  const int32_t* pair_ids;
};

// pairs a fused small-batch launch may carry (one pair per thread of a 256-thread workgroup)
constexpr int kFusedMaxPairs = 256;

// Fused small-batch path, launch 1: per token router logits (or given logits), top-k, and with
// xq non-null e4m3 codes xq [T, d] + scales xs [T, d/128] (fp32, or e8m0 bytes with ue).
// x and wr 16-byte aligned, d % 128 == 0, E <= kMaxExperts.
hipError_t launch_fused_route(const void* x, moe_dtype x_dtype, const float* logits,
                              const float* wr, float* logits_out, int T, int d, int E, int k,
                              int32_t* ids, float* w, uint8_t* xq, void* xs, bool ue,
                              hipStream_t stream);

int f32_tile_rows();
hipError_t launch_experts_f32(const ExpertsLaunch& L, hipStream_t stream);

int bf16_tile_rows_gateup();
int bf16_tile_rows_down();
hipError_t launch_experts_bf16(const ExpertsLaunch& L, hipStream_t stream);

hipError_t launch_experts_bf16_decode(const ExpertsLaunch& L, hipStream_t stream);

int fp8_tile_rows(bool w4, bool ue8m0);   // rows of the fp8 GEMMs' tile tables
hipError_t launch_experts_fp8(const ExpertsLaunch& L, hipStream_t stream);
hipError_t launch_experts_fp8_decode(const ExpertsLaunch& L, hipStream_t stream);

}  // namespace moe
