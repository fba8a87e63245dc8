// C ABI of libmoe: argument validation, workspace layout and kernel dispatch.
// Every check runs on the host before anything is enqueued; on error nothing is launched and no
// output is touched.
#include <limits.h>

#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool is_float_type(moe_dtype t) { return t == MOE_F32 || t == MOE_BF16; }

inline size_t elem_size(moe_dtype t) { return t == MOE_F32 ? 4 : t == MOE_BF16 ? 2 : 1; }

inline moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

moe_status check_topology(int T, int E, int k) {
  if (T < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
  if (E > kMaxExperts || k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(T) * k > INT_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Small-batch (weight streaming) kernels take over while the mean number of rows per expert,
// P / E, is small; past it the tiled grouped GEMMs are faster. Both paths timed on MI355X at the
// Mixtral-shaped (E = 8) and DeepSeek-V3-shaped (E = 256) layers for T = 8 .. 512:
//   bf16: small-batch faster up to 12 rows per expert (Mixtral T = 48: 0.566 vs 0.574 ms), the
//         tiled GEMM from 16 (T = 64: 0.579 vs 0.622 ms);
//   e4m3 / E2M1: small-batch faster up to 16 rows per expert on the Mixtral shape (fp32 scales,
//         UE8M0 and E2M1; tiled from 32) and on the DeepSeek-V3 shape with E2M1 weights (1.28 vs
//         1.50 ms at 16 rows); on the DeepSeek-V3 shape with e4m3 weights the tiled GEMM is up to
//         5 % faster from 4 (UE8M0) or 16 (fp32 scales) rows, the largest loss of this rule.
constexpr int kSmallRowsBf16 = 12;
constexpr int kSmallRowsLowp = 16;

// 8-bit activation codes with e4m3 or E2M1 weights (block scales, fp8 quantisation of x and h)
inline bool is_low_precision(moe_dtype w) { return w == MOE_FP8_E4M3 || w == MOE_FP4_E2M1; }

inline bool uses_decode(moe_dtype act, moe_dtype w, long long P, int E, int d, int f) {
  return act == MOE_BF16 && w == MOE_BF16 && P <= static_cast<long long>(kSmallRowsBf16) * E &&
         d % 128 == 0 && f % 128 == 0;
}

// fp8 layers with few rows per expert take the weight-streaming fp8 kernels.
inline bool uses_fp8_decode(moe_dtype act, moe_dtype w, long long P, int E) {
  return act == MOE_FP8_E4M3 && is_low_precision(w) &&
         P <= static_cast<long long>(kSmallRowsLowp) * E;
}

// bf16 tiled GEMMs cut their tail tiles; they need partial-tile slots and counters.
inline bool uses_split(moe_dtype act, moe_dtype w, long long P, int E, int d, int f) {
  return act == MOE_BF16 && w == MOE_BF16 && !uses_decode(act, w, P, E, d, f);
}

struct ExpertsLayout {
  size_t cum_a, cum_b, h, h_scales, x_scales, h32, h_scale_bytes, split_partial, total;
};

ExpertsLayout experts_layout(int T, int d, int f, int E, int k, moe_dtype act, moe_dtype w) {
  ExpertsLayout L{};
  const size_t P = static_cast<size_t>(T) * k;
  size_t off = 0;
  L.cum_a = off;
  off = align_up(off + (E + 1) * sizeof(int32_t));
  L.cum_b = off;
  off = align_up(off + (E + 1) * sizeof(int32_t));
  L.h = off;
  const size_t h_elem = is_low_precision(w) ? 1 : (act == MOE_F32 ? 4 : 2);
  off = align_up(off + P * f * h_elem);
  L.h_scales = off;
  if (is_low_precision(w)) off = align_up(off + P * (f / kFp8Group) * sizeof(float));
  // fp8 with UE8M0 scales: x_scales expanded from e8m0 bytes to fp32 values
  L.x_scales = off;
  if (is_low_precision(w))
    off = align_up(off + static_cast<size_t>(T) * (d / kFp8Group) * sizeof(float));
  // fp8 decode: fp32 h before its quantisation, and its e8m0 scale bytes
  L.h32 = L.h_scale_bytes = 0;
  if (uses_fp8_decode(act, w, static_cast<long long>(P), E)) {
    L.h32 = off;
    off = align_up(off + P * f * sizeof(float));
    L.h_scale_bytes = off;
    off = align_up(off + P * (f / kFp8Group));
  }
  L.split_partial = 0;
  if (uses_split(act, w, static_cast<long long>(P), E, d, f)) {
    L.split_partial = off;
    off = align_up(off + static_cast<size_t>(kSplitSlots) * 256 * 256 * sizeof(float));
  }
  L.total = off;
  return L;
}

__global__ void zero_f32_kernel(float* p, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i < n; i += static_cast<size_t>(gridDim.x) * blockDim.x) p[i] = 0.0f;
}

}  // namespace

namespace moe {

// CUs per XCD of the current device (its 8 XCDs share the CUs evenly), cached per device and
// capped so the split-tile slots stay within kSplitSlots.
int cus_per_xcd() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int c = std::max(1, std::min(kSplitSlots / 8, cus / 8));
  if (dev < 64) cache[dev].store(c, std::memory_order_relaxed);
  return c;
}

}  // namespace moe

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    default: return "MOE_ERR_UNKNOWN";
  }
}

moe_status moe_route(const float* logits, const void* x, moe_dtype x_dtype,
                     const float* w_router, int T, int d, int E, int k, float* logits_out,
                     int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  moe_status st = check_topology(T, E, k);
  if (st != MOE_OK) return st;
  if (!topk_ids || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (!logits) {
    if (!x || !w_router || !logits_out || d < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (!is_float_type(x_dtype)) return MOE_ERR_UNSUPPORTED;
    if (static_cast<long long>(T) * d > INT_MAX / 2) return MOE_ERR_UNSUPPORTED;
    if (T < 256 && d % 8 == 0 && aligned(x, 16) && aligned(w_router, 16))
      // few tokens: one workgroup per token computes its logits and its top-k in one launch
      // (the same arithmetic as the two separate kernels)
      return dev(launch_fused_route(x, x_dtype, nullptr, w_router, logits_out, T, d, E, k,
                                    topk_ids, topk_w, nullptr, nullptr, false, stream));
    hipError_t e = launch_router_logits(x, x_dtype, w_router, T, d, E, logits_out, stream);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    logits = logits_out;
  } else if (logits_out && logits_out != logits) {
    hipError_t e = hipMemcpyAsync(logits_out, logits, sizeof(float) * static_cast<size_t>(T) * E,
                                  hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  }
  return dev(launch_topk_softmax(logits, T, E, k, topk_ids, topk_w, stream));
}

size_t moe_permute_workspace_size(int T, int k, int E) {
  if (check_topology(T, E, k) != MOE_OK) return 0;
  return align_up(permute_workspace_bytes(T * k, E));
}

moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, const void* x,
                       moe_dtype x_dtype, const float* x_scales, int d, void* x_perm,
                       float* x_perm_scales, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  moe_status st = check_topology(T, E, k);
  if (st != MOE_OK) return st;
  if (!topk_ids || !counts || !offsets || !sorted_pair || !pair_pos) return MOE_ERR_INVALID_ARGUMENT;
  const bool gather = x != nullptr || x_perm != nullptr;
  if (gather) {
    if (!x || !x_perm || d < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16 && x_dtype != MOE_FP8_E4M3)
      return MOE_ERR_INVALID_ARGUMENT;
    if (x_dtype == MOE_FP8_E4M3) {
      if (d % kFp8Group) return MOE_ERR_UNSUPPORTED;
      if (!x_scales || !x_perm_scales) return MOE_ERR_INVALID_ARGUMENT;
    }
  }
  if (!workspace || workspace_bytes < moe_permute_workspace_size(T, k, E))
    return workspace ? MOE_ERR_WORKSPACE_TOO_SMALL : MOE_ERR_INVALID_ARGUMENT;
  const int P = T * k;
  hipError_t e = launch_permute(topk_ids, P, E, counts, offsets, sorted_pair, pair_pos, workspace,
                                stream);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  if (gather) {
    e = launch_gather_rows(x, static_cast<size_t>(d) * elem_size(x_dtype), sorted_pair, P, k,
                           x_perm, stream);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    if (x_dtype == MOE_FP8_E4M3) {
      e = launch_gather_rows(x_scales, static_cast<size_t>(d / kFp8Group) * sizeof(float),
                             sorted_pair, P, k, x_perm_scales, stream);
      if (e != hipSuccess) return MOE_ERR_DEVICE;
    }
  }
  return MOE_OK;
}

moe_status fp8_quantize_act(const void* x, moe_dtype x_dtype, int M, int K, int group,
                            const int32_t* row_index, uint8_t* q, float* scales,
                            hipStream_t stream) {
  if (!x || !q || !scales || M < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!is_float_type(x_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  if (group != kFp8Group || K % kFp8Group) return MOE_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 8)) return MOE_ERR_UNSUPPORTED;
  return dev(launch_quantize_act(x, x_dtype, M, K, row_index, q, scales, false, stream));
}

moe_status fp8_quantize_act_ue8m0(const void* x, moe_dtype x_dtype, int M, int K, int group,
                                  const int32_t* row_index, uint8_t* q, uint8_t* scales,
                                  hipStream_t stream) {
  if (!x || !q || !scales || M < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!is_float_type(x_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  if (group != kFp8Group || K % kFp8Group) return MOE_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 8)) return MOE_ERR_UNSUPPORTED;
  return dev(launch_quantize_act(x, x_dtype, M, K, row_index, q, scales, true, stream));
}

moe_status fp8_quantize_weight(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                               int block, uint8_t* q, float* scales, hipStream_t stream) {
  if (!w || !q || !scales || batch < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!is_float_type(w_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  if (block != kFp8Group || N % kFp8Group || K % kFp8Group) return MOE_ERR_UNSUPPORTED;
  if (!aligned(q, 4)) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(batch) * (N / kFp8Group) * (K / kFp8Group) > INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  return dev(launch_quantize_weight(w, w_dtype, batch, N, K, q, scales, false, stream));
}

moe_status fp8_quantize_weight_ue8m0(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                                     int block, uint8_t* q, uint8_t* scales, hipStream_t stream) {
  if (!w || !q || !scales || batch < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!is_float_type(w_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  if (block != kFp8Group || N % kFp8Group || K % kFp8Group) return MOE_ERR_UNSUPPORTED;
  if (!aligned(q, 4)) return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(batch) * (N / kFp8Group) * (K / kFp8Group) > INT_MAX)
    return MOE_ERR_UNSUPPORTED;
  return dev(launch_quantize_weight(w, w_dtype, batch, N, K, q, scales, true, stream));
}

moe_status fp4_tile_weight(const uint8_t* q, int batch, int N, int K, uint8_t* q_tiled,
                           hipStream_t stream) {
  if (!q || !q_tiled || batch < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (N % 16 || K % 128) return MOE_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(q_tiled, 16)) return MOE_ERR_UNSUPPORTED;
  const size_t bytes = static_cast<size_t>(batch) * N * (K / 2);
  const uintptr_t a = reinterpret_cast<uintptr_t>(q), b = reinterpret_cast<uintptr_t>(q_tiled);
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARGUMENT;   // no overlap
  if (bytes / 16 > (static_cast<size_t>(INT_MAX) << 6)) return MOE_ERR_UNSUPPORTED;
  return dev(launch_tile_weight_fp4(q, static_cast<size_t>(batch) * N, K, q_tiled, stream));
}

moe_status fp4_quantize_weight_mx(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                                  uint8_t* q, uint8_t* scales, hipStream_t stream) {
  if (!w || !q || !scales || batch < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!is_float_type(w_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  if (K % 32) return MOE_ERR_UNSUPPORTED;
  if (!aligned(q, 16)) return MOE_ERR_UNSUPPORTED;
  const size_t nblocks = static_cast<size_t>(batch) * N * (K / 32);
  if (nblocks > (static_cast<size_t>(INT_MAX) << 6)) return MOE_ERR_UNSUPPORTED;
  return dev(launch_quantize_weight_mx4(w, w_dtype, nblocks, q, scales, stream));
}

int moe_experts_small_batch(int T, int d, int f, int E, int k, moe_dtype act_dtype,
                            moe_dtype w_dtype) {
  if (check_topology(T, E, k) != MOE_OK || d < 1 || f < 1) return -1;
  const long long P = static_cast<long long>(T) * k;
  const bool bf16 = act_dtype == MOE_BF16 && w_dtype == MOE_BF16;
  const bool fp8 = act_dtype == MOE_FP8_E4M3 && is_low_precision(w_dtype);
  const bool f32 = act_dtype == MOE_F32 && w_dtype == MOE_F32;
  if (!bf16 && !fp8 && !f32) return -1;
  return (bf16 && uses_decode(act_dtype, w_dtype, P, E, d, f)) ||
                 (fp8 && uses_fp8_decode(act_dtype, w_dtype, P, E))
             ? 1
             : 0;
}

size_t moe_experts_workspace_size(int T, int d, int f, int E, int k, moe_dtype act_dtype,
                                  moe_dtype w_dtype) {
  if (check_topology(T, E, k) != MOE_OK || d < 1 || f < 1) return 0;
  return experts_layout(T, d, f, E, k, act_dtype, w_dtype).total;
}

moe_status moe_experts_forward(const moe_experts_args* a, hipStream_t stream) {
  if (!a) return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_topology(a->T, a->E, a->k);
  if (st != MOE_OK) return st;
  if (a->d < 1 || a->f < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!a->x || !a->w_gate || !a->w_up || !a->w_down || !a->offsets || !a->sorted_pair || !a->y)
    return MOE_ERR_INVALID_ARGUMENT;
  if (a->y_layout != MOE_Y_PERMUTED && a->y_layout != MOE_Y_SLOTS && a->y_layout != MOE_Y_ACC_F32)
    return MOE_ERR_INVALID_ARGUMENT;
  if (a->y_layout != MOE_Y_PERMUTED && !a->topk_w) return MOE_ERR_INVALID_ARGUMENT;
  if (a->phase != MOE_PHASE_ALL && a->phase != MOE_PHASE_GATE_UP && a->phase != MOE_PHASE_DOWN)
    return MOE_ERR_INVALID_ARGUMENT;
  const bool run_gate_up = a->phase != MOE_PHASE_DOWN;
  const bool run_down = a->phase != MOE_PHASE_GATE_UP;
  if (!is_float_type(a->y_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  const moe_dtype act = a->act_dtype, w = a->w_dtype;
  const bool f32 = act == MOE_F32 && w == MOE_F32;
  const bool bf16 = act == MOE_BF16 && w == MOE_BF16;
  const bool w4 = act == MOE_FP8_E4M3 && w == MOE_FP4_E2M1;
  const bool fp8 = (act == MOE_FP8_E4M3 && w == MOE_FP8_E4M3) || w4;
  if (!f32 && !bf16 && !fp8) return MOE_ERR_UNSUPPORTED;
  if (f32 && a->y_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (bf16 && (a->d % 64 || a->f % 64)) return MOE_ERR_UNSUPPORTED;
  if (a->scale_fmt != MOE_SCALE_F32 && a->scale_fmt != MOE_SCALE_UE8M0)
    return MOE_ERR_INVALID_ARGUMENT;
  const bool ue8m0 = a->scale_fmt == MOE_SCALE_UE8M0;
  if (ue8m0 && !fp8) return MOE_ERR_INVALID_ARGUMENT;  // scales exist only on the fp8 path
  if (fp8) {
    if (a->d % kFp8Group || a->f % kFp8Group) return MOE_ERR_UNSUPPORTED;
    if (a->d > 32768 || a->f > 32768) return MOE_ERR_UNSUPPORTED;
    if (!a->x_scales || !a->s_gate || !a->s_up || !a->s_down) return MOE_ERR_INVALID_ARGUMENT;
  }
  // the matrix-core paths read x and the weights with 16-byte loads and LDS DMA, and store y
  // with 8- and 16-byte stores; fp32 block scales are read as dwords
  if (!f32 && (!aligned(a->x, 16) || !aligned(a->w_gate, 16) || !aligned(a->w_up, 16) ||
               !aligned(a->w_down, 16) || !aligned(a->y, 16)))
    return MOE_ERR_UNSUPPORTED;
  if (fp8 && !ue8m0 && (!aligned(a->x_scales, 4) || !aligned(a->s_gate, 4) ||
                        !aligned(a->s_up, 4) || !aligned(a->s_down, 4)))
    return MOE_ERR_UNSUPPORTED;
  const long long P = static_cast<long long>(a->T) * a->k;
  // E2M1 weights: MX scales are e8m0 bytes
  if (w4 && !ue8m0) return MOE_ERR_UNSUPPORTED;
  if (w4 && (!aligned(a->s_gate, 4) || !aligned(a->s_up, 4) || !aligned(a->s_down, 4)))
    return MOE_ERR_UNSUPPORTED;   // MX scale rows are read as dwords
  // 32-bit element offsets inside the kernels
  if (static_cast<long long>(a->T) * a->d > INT_MAX / 2 || P * a->f > INT_MAX / 2 ||
      P * a->d > INT_MAX / 2 || static_cast<long long>(a->f) * a->d > INT_MAX / 4)
    return MOE_ERR_UNSUPPORTED;
  const ExpertsLayout L = experts_layout(a->T, a->d, a->f, a->E, a->k, act, w);
  if (!a->workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (a->workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;

  char* ws = static_cast<char*>(a->workspace);
  ExpertsLaunch X{};
  X.T = a->T;
  X.d = a->d;
  X.f = a->f;
  X.E = a->E;
  X.k = a->k;
  X.a = a->x;
  X.a_gather = 1;
  X.a_scales = static_cast<const float*>(a->x_scales);
  X.sorted_pair = a->sorted_pair;
  X.w_gate = a->w_gate;
  X.w_up = a->w_up;
  X.w_down = a->w_down;
  X.s_gate = a->s_gate;
  X.s_up = a->s_up;
  X.s_down = a->s_down;
  X.scale_ue8m0 = ue8m0 ? 1 : 0;
  X.w_fp4 = w4 ? 1 : 0;
  X.offsets = a->offsets;
  X.tile_cum_a = reinterpret_cast<int32_t*>(ws + L.cum_a);
  X.tile_cum_b = reinterpret_cast<int32_t*>(ws + L.cum_b);
  X.topk_w = a->topk_w;
  X.y_layout = a->y_layout;
  X.y_bf16 = a->y_dtype == MOE_BF16;
  X.y = a->y;
  X.h = ws + L.h;
  X.h_scales = reinterpret_cast<float*>(ws + L.h_scales);
  const bool fp8_decode = fp8 && uses_fp8_decode(act, w, P, a->E);
  X.h32 = fp8_decode ? reinterpret_cast<float*>(ws + L.h32) : nullptr;
  X.h_scale_bytes = fp8_decode ? reinterpret_cast<uint8_t*>(ws + L.h_scale_bytes) : nullptr;
  X.cpx = cus_per_xcd();
  const bool split = uses_split(act, w, P, a->E, a->d, a->f);
  X.split_partial = split ? reinterpret_cast<float*>(ws + L.split_partial) : nullptr;
  X.run_gate_up = run_gate_up ? 1 : 0;
  X.run_down = run_down ? 1 : 0;

  const bool decode = uses_decode(act, w, P, a->E, a->d, a->f);
  int bm_a, bm_b;
  if (f32) { bm_a = bm_b = f32_tile_rows(); }
  else if (fp8_decode) { bm_a = bm_b = 0; }  // no tile table
  else if (fp8) { bm_a = bm_b = fp8_tile_rows(w4, ue8m0); }
  else if (decode) { bm_a = bm_b = 0; }  // no tile table
  else { bm_a = bf16_tile_rows_gateup(); bm_b = bf16_tile_rows_down(); }

  hipError_t e = hipSuccess;
  // the gate/up phase writes the tile tables of both GEMMs (a down-only call reads them from the
  // workspace, as it reads h)
  if (run_gate_up && !decode && !fp8_decode) {  // decode kernels map (expert, row panel) directly
    e = launch_tile_table(a->offsets, a->E, bm_a, bm_b, const_cast<int32_t*>(X.tile_cum_a),
                          const_cast<int32_t*>(X.tile_cum_b), stream);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  }
  if (run_down && a->y_layout == MOE_Y_ACC_F32) {
    const size_t n = static_cast<size_t>(a->T) * a->d;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 65536))),
                       dim3(256), 0, stream, static_cast<float*>(a->y), n);
    if ((e = hipGetLastError()) != hipSuccess) return MOE_ERR_DEVICE;
  }
  if (ue8m0) X.a_scale_bytes = a->x_scales;   // the small-batch kernels read the bytes
  if (run_gate_up && ue8m0 && !fp8_decode) {
    // the tiled GEMMs read activation scales as fp32 values; e8m0 bytes expand exactly
    float* xs = reinterpret_cast<float*>(ws + L.x_scales);
    e = launch_e8m0_expand(static_cast<const uint8_t*>(a->x_scales),
                           static_cast<size_t>(a->T) * (a->d / kFp8Group), xs, stream);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    X.a_scales = xs;
  }
  if (f32) e = launch_experts_f32(X, stream);
  else if (fp8_decode) e = launch_experts_fp8_decode(X, stream);
  else if (fp8) e = launch_experts_fp8(X, stream);
  else if (decode) e = launch_experts_bf16_decode(X, stream);
  else e = launch_experts_bf16(X, stream);
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  return dev(e);
}

}  // extern "C"

namespace {

struct FusedLayout {
  size_t xq, xs, h, h32, hs, slots, total;
};

// Workspace of the fused path: x codes and scales (fp8 / FP4), h (bf16; or fp32 before its
// quantisation, e4m3 codes and scales), and the slots [P, d] in the output type.
FusedLayout fused_layout(int T, int d, int f, int k, moe_dtype w, moe_dtype out) {
  FusedLayout L{};
  const size_t P = static_cast<size_t>(T) * k;
  size_t off = 0;
  if (is_low_precision(w)) {
    L.xq = off;
    off = align_up(off + static_cast<size_t>(T) * d);
    L.xs = off;
    off = align_up(off + static_cast<size_t>(T) * (d / kFp8Group) * sizeof(float));
    L.h32 = off;
    off = align_up(off + P * f * sizeof(float));
    L.h = off;   // e4m3 codes
    off = align_up(off + P * f);
    L.hs = off;
    off = align_up(off + P * (f / kFp8Group) * sizeof(float));
  } else {
    L.h = off;
    off = align_up(off + P * f * 2);
  }
  L.slots = off;
  off = align_up(off + P * d * (out == MOE_F32 ? 4 : 2));
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t moe_fused_workspace_size(int T, int d, int f, int E, int k, moe_dtype w_dtype,
                                moe_dtype out_dtype) {
  if (check_topology(T, E, k) != MOE_OK || d < 1 || f < 1) return 0;
  if (static_cast<long long>(T) * k > kFusedMaxPairs || d % kFp8Group || f % kFp8Group) return 0;
  return fused_layout(T, d, f, k, w_dtype, out_dtype).total;
}

}  // extern "C"

namespace {

// Host-side checks of a fused call (everything but the workspace); on success *L is its layout.
moe_status fused_validate(const moe_fused_args* a, FusedLayout* L) {
  if (!a) return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_topology(a->T, a->E, a->k);
  if (st != MOE_OK) return st;
  if (a->d < 1 || a->f < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (!a->x || !a->w_gate || !a->w_up || !a->w_down || !a->out || !a->topk_ids || !a->topk_w)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!a->logits && !a->w_router) return MOE_ERR_INVALID_ARGUMENT;
  if (a->out_dtype != MOE_BF16 && a->out_dtype != MOE_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (a->x_dtype != MOE_BF16 && a->x_dtype != MOE_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (a->scale_fmt != MOE_SCALE_F32 && a->scale_fmt != MOE_SCALE_UE8M0)
    return MOE_ERR_INVALID_ARGUMENT;
  const moe_dtype w = a->w_dtype;
  const bool lowp = is_low_precision(w);
  const bool ue8m0 = a->scale_fmt == MOE_SCALE_UE8M0;
  if (w != MOE_BF16 && !lowp) return MOE_ERR_UNSUPPORTED;
  if (w == MOE_BF16 && (a->x_dtype != MOE_BF16 || ue8m0)) return MOE_ERR_UNSUPPORTED;
  if (w == MOE_FP4_E2M1 && !ue8m0) return MOE_ERR_UNSUPPORTED;
  if (lowp && (!a->s_gate || !a->s_up || !a->s_down)) return MOE_ERR_INVALID_ARGUMENT;
  if (w == MOE_FP4_E2M1 &&
      (!aligned(a->s_gate, 4) || !aligned(a->s_up, 4) || !aligned(a->s_down, 4)))
    return MOE_ERR_UNSUPPORTED;
  const long long P = static_cast<long long>(a->T) * a->k;
  if (P > kFusedMaxPairs) return MOE_ERR_UNSUPPORTED;
  if (a->d % kFp8Group || a->f % kFp8Group) return MOE_ERR_UNSUPPORTED;
  if (a->d > 32768 || a->f > 32768) return MOE_ERR_UNSUPPORTED;
  if (!aligned(a->x, 16) || (!a->logits && !aligned(a->w_router, 16))) return MOE_ERR_UNSUPPORTED;
  if (!aligned(a->w_gate, 16) || !aligned(a->w_up, 16) || !aligned(a->w_down, 16))
    return MOE_ERR_UNSUPPORTED;
  if (lowp && !ue8m0 && (!aligned(a->s_gate, 4) || !aligned(a->s_up, 4) || !aligned(a->s_down, 4)))
    return MOE_ERR_UNSUPPORTED;
  if (static_cast<long long>(a->f) * a->d > INT_MAX / 4) return MOE_ERR_UNSUPPORTED;
  *L = fused_layout(a->T, a->d, a->f, a->k, w, a->out_dtype);
  return MOE_OK;
}

// Enqueues a validated fused call with its workspace at ws (at least L.total bytes).
moe_status fused_launch(const moe_fused_args* a, const FusedLayout& L, char* ws,
                        hipStream_t stream) {
  const moe_dtype w = a->w_dtype;
  const bool lowp = is_low_precision(w);
  const bool ue8m0 = a->scale_fmt == MOE_SCALE_UE8M0;
  uint8_t* xq = lowp ? reinterpret_cast<uint8_t*>(ws + L.xq) : nullptr;
  void* xs = lowp ? static_cast<void*>(ws + L.xs) : nullptr;
  hipError_t e = launch_fused_route(a->x, a->x_dtype, a->logits, a->w_router, a->logits_out, a->T,
                                    a->d, a->E, a->k, a->topk_ids, a->topk_w, xq, xs, ue8m0,
                                    stream);
  if (e != hipSuccess) return MOE_ERR_DEVICE;

  ExpertsLaunch X{};
  X.T = a->T;
  X.d = a->d;
  X.f = a->f;
  X.E = a->E;
  X.k = a->k;
  X.a = lowp ? static_cast<const void*>(xq) : a->x;
  X.a_gather = 1;
  X.a_scales = static_cast<const float*>(xs);
  X.a_scale_bytes = xs;
  X.w_gate = a->w_gate;
  X.w_up = a->w_up;
  X.w_down = a->w_down;
  X.s_gate = a->s_gate;
  X.s_up = a->s_up;
  X.s_down = a->s_down;
  X.scale_ue8m0 = ue8m0 ? 1 : 0;
  X.w_fp4 = w == MOE_FP4_E2M1 ? 1 : 0;
  X.topk_w = a->topk_w;
  X.y_layout = MOE_Y_SLOTS;
  X.y_bf16 = a->out_dtype == MOE_BF16;
  X.y = ws + L.slots;
  X.h = ws + L.h;
  X.h32 = lowp ? reinterpret_cast<float*>(ws + L.h32) : nullptr;
  X.h_scales = lowp ? reinterpret_cast<float*>(ws + L.hs) : nullptr;
  X.h_scale_bytes = lowp ? reinterpret_cast<uint8_t*>(ws + L.hs) : nullptr;
  X.pair_ids = a->topk_ids;
  X.cpx = cus_per_xcd();
  X.run_gate_up = X.run_down = 1;
  e = lowp ? launch_experts_fp8_decode(X, stream) : launch_experts_bf16_decode(X, stream);
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  return dev(launch_combine(ws + L.slots, a->out_dtype, MOE_Y_SLOTS, nullptr, nullptr, a->T, a->k,
                            a->d, a->out, a->out_dtype, stream));
}

// ---- the allocation-free variant ----------------------------------------------------------------
//
// Device memory of moe_fused_forward_noalloc, used in place of a caller's workspace: a fixed
// array in the library's device code, one per GPU the library runs on, alive until the process
// ends. Host code never passes the array's name to a kernel or copy (on the host it is only a
// stand-in for the symbol); it uses the device address hipGetSymbolAddress returns for the
// current device, looked up once per device.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::atomic<char*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;

// This device's scratch address (device = the current one); hipGetSymbolAddress runs once per
// device, with that device current, under the mutex.
hipError_t device_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<char*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_fused_forward(const moe_fused_args* a, hipStream_t stream) {
  FusedLayout L{};
  const moe_status st = fused_validate(a, &L);
  if (st != MOE_OK) return st;
  if (!a->workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (a->workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return fused_launch(a, L, static_cast<char*>(a->workspace), stream);
}

moe_status moe_fused_forward_noalloc(const moe_fused_args* a, hipStream_t stream) {
  FusedLayout L{};
  const moe_status st = fused_validate(a, &L);
  if (st != MOE_OK) return st;
  if (L.total > kScratchBytes) return MOE_ERR_UNSUPPORTED;   // beyond the fixed scratch array
  char* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) return MOE_ERR_DEVICE;
  return fused_launch(a, L, ws, stream);
}

moe_status moe_combine(const void* y, moe_dtype y_dtype, moe_y_layout layout,
                       const int32_t* pair_pos, const float* topk_w, int T, int k, int d,
                       void* out, moe_dtype out_dtype, hipStream_t stream) {
  if (!y || !out || T < 1 || k < 1 || d < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (layout != MOE_Y_PERMUTED && layout != MOE_Y_SLOTS && layout != MOE_Y_ACC_F32)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!is_float_type(y_dtype) || !is_float_type(out_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  if (layout == MOE_Y_ACC_F32 && y_dtype != MOE_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (layout == MOE_Y_PERMUTED && (!pair_pos || !topk_w)) return MOE_ERR_INVALID_ARGUMENT;
  if (static_cast<long long>(T) * k * d > (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  return dev(launch_combine(y, y_dtype, layout, pair_pos, topk_w, T, k, d, out, out_dtype, stream));
}

}  // extern "C"
