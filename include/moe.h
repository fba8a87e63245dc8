/*
 * moe.h - C ABI of the MI355X (gfx950) sparse mixture-of-experts experts forward pass.
 *
 * The layer (Transformers docs page "Experts backends", introduction): for every token the router
 * picks k experts, the token's hidden state is projected through those experts' parameters, and
 * the expert outputs are summed with the routing weights. The router (lira-now explainer "Mixture
 * of Experts (MoE): a practical explanation", section 5, router step by step): logits over E
 * experts -> softmax -> top-k -> renormalise the k selected probabilities. Each expert is a gated
 * MLP (same Transformers page, backends table rows deepgemm_megamoe and sonicmoe):
 *     y = W_down (silu(W_gate x) * (W_up x)),   silu(z) = z / (1 + exp(-z)).
 * Tokens are grouped by selected expert so that one grouped GEMM serves every expert (same table,
 * row grouped_mm). The optional fine-grained FP8 path follows the Transformers page "Fine-grained
 * FP8" (introduction): e4m3 weights with one fp32 scale per 128x128 block, e4m3 activations with a
 * dynamic fp32 scale per token per 128 input channels.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named x, logits, w_*, s_*, ids, counts, offsets, sorted_pair, pair_pos, y, out,
 *    workspace are DEVICE pointers owned by the caller. The library never allocates, frees or
 *    synchronises; all work is enqueued on `stream` (NULL = the null stream) and completes
 *    asynchronously in stream order.
 *  - Row-major, contiguous tensors. Weights use the nn.Linear layout (out_features x in_features),
 *    so a projection is x W^T: W_gate, W_up are [E, f, d] and W_down is [E, d, f].
 *  - T tokens, d hidden size, f expert intermediate size, E experts, k experts per token,
 *    P = T*k (token, slot) pairs, pair index p = t*k + j.
 *  - Arguments are checked on the host before anything is enqueued. On any error nothing is
 *    enqueued and no output is written; the status says why. A failed launch returns
 *    MOE_ERR_DEVICE. Faults inside kernels surface at the caller's next synchronisation.
 *  - The library is stateless and re-entrant; calls on different streams may overlap as long as
 *    their buffers do not.
 *  - Limits: 1 <= k <= E <= 1024, k <= 32, T >= 1, T*k < 2^31, d and f >= 1.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* bad sizes, k > E, null required pointer, unknown enum */
  MOE_ERR_UNSUPPORTED = 2,        /* valid request without a kernel (e.g. fp8 dims not /128) */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_DEVICE = 4,             /* a HIP launch or API call failed */
  MOE_STATUS_RANGE_MIN_ = -0x7FFFFFFF - 1, /* range markers, not values: see below */
  MOE_STATUS_RANGE_MAX_ = 0x7FFFFFFF
} moe_status;

typedef enum {
  MOE_F32 = 0,       /* IEEE binary32 */
  MOE_BF16 = 1,      /* bfloat16 */
  MOE_FP8_E4M3 = 2,  /* OCP E4M3FN: bias 7, max 448, no infinities */
  MOE_FP4_E2M1 = 3,  /* OCP E2M1 (0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte: element 2j in the
                        low nibble of byte j; expert weights only, with MX scales (below) */
  MOE_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  MOE_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} moe_dtype;

/* Format of fp8 block scales (Transformers "Fine-grained FP8" page, section "UE8M0 scale
 * format": checkpoints that store weight scales as packed float8_e8m0fnu instead of float32). */
typedef enum {
  MOE_SCALE_F32 = 0,   /* one fp32 value per block */
  MOE_SCALE_UE8M0 = 1, /* one byte b per block, value 2^(b - 127) (255 = NaN, never produced) */
  MOE_SCALE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  MOE_SCALE_RANGE_MAX_ = 0x7FFFFFFF
} moe_scale_fmt;

/* Layout of the expert outputs that moe_experts_forward writes and moe_combine reads. */
typedef enum {
  MOE_Y_PERMUTED = 0, /* y [P, d]: unweighted expert outputs, rows in sorted-pair order */
  MOE_Y_SLOTS = 1,    /* y [T, k, d]: y[t][j] = w[t][j] * expert_{ids[t][j]}(x[t]) (fused
                         unpermute + weighting in the down-projection epilogue) */
  MOE_Y_ACC_F32 = 2,  /* y [T, d] fp32: the weighted sum accumulated with atomic adds (zeroed by
                         moe_experts_forward); summation order, and so rounding, is not fixed
                         when k > 2 */
  MOE_Y_RANGE_MIN_ = -0x7FFFFFFF - 1,
  MOE_Y_RANGE_MAX_ = 0x7FFFFFFF
} moe_y_layout;

/* Every enum above and below carries a *_RANGE_MIN_ / *_RANGE_MAX_ pair that is not a value:
 * it makes every int32 a representable value of the enum type (and keeps the type 4 bytes), so an
 * out-of-range value from a C caller or a foreign-function binding is read without undefined
 * behaviour and rejected with MOE_ERR_INVALID_ARGUMENT (moe_status_string: "MOE_ERR_UNKNOWN"). */

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* ------------------------------------------------------------------------------------------
 * moe_route - router: softmax over E expert logits, top-k, renormalise.
 * (lira-now explainer, section 5, steps 2-5 and its pseudocode; gyaansetu explainer, top-k
 * routing.)
 *
 *  logits      [T, E] fp32, or NULL to compute logits = x . w_router^T here in fp32.
 *  x           [T, d] of x_dtype (MOE_F32 or MOE_BF16); used only when logits == NULL.
 *  w_router    [E, d] fp32; used only when logits == NULL.
 *  logits_out  [T, E] fp32: receives the logits that the selection used. Required when
 *              logits == NULL (the computed logits live there); nullable otherwise.
 *  topk_ids    [T, k] int32 out: expert ids by descending logit; equal logits go to the lower
 *              expert index (+0 and -0 are equal). (Selecting on logits picks the same set as
 *              selecting on softmax probabilities, since softmax is strictly increasing.) NaN
 *              logits are outside the contract: they are ordered by their bits (above +inf
 *              with the sign bit clear, below -inf with it set) and make weights NaN.
 *  topk_w      [T, k] fp32 out: w[t][j] = exp(l_j - l_max) / sum_{j'<k} exp(l_j' - l_max), the
 *              selected softmax probabilities renormalised to sum to 1.
 * ------------------------------------------------------------------------------------------ */
moe_status moe_route(const float* logits, const void* x, moe_dtype x_dtype,
                     const float* w_router, int T, int d, int E, int k, float* logits_out,
                     int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * moe_permute - group the P = T*k (token, slot) pairs by expert.
 * (Transformers "Experts backends" page, backends table row grouped_mm: tokens are sorted by
 * their selected expert so one grouped GEMM projects them all.)
 *
 *  topk_ids     [T, k] int32 in [0, E). The ids live on the device and are not read by the
 *               host: an id outside [0, E) is a caller error that the kernels contain rather
 *               than report. Such a pair is left out of counts and sorted_pair, its pair_pos
 *               entry is -1, offsets[E] becomes the number of in-range pairs (so offsets[E] < P
 *               flags the error), rows [offsets[E], P) of sorted_pair and x_perm are left
 *               unwritten, and no memory outside the buffers named here is touched. moe_combine
 *               (MOE_Y_PERMUTED) skips pairs whose pair_pos lies outside [0, P); moe_experts
 *               must not be given such a permutation.
 *  counts       [E] int32 out: pairs per expert.
 *  offsets      [E+1] int32 out: exclusive prefix sum of counts; offsets[E] = P.
 *  sorted_pair  [P] int32 out: pair indices p = t*k + j, expert by expert, ascending p within an
 *               expert (a stable sort, so the result is deterministic).
 *  pair_pos     [P] int32 out: inverse of sorted_pair (pair p sits at row pair_pos[p]).
 *  x, x_perm    optional gather (both NULL to skip): x_perm[r] = x[sorted_pair[r] / k], rows of d
 *               elements of x_dtype (MOE_F32, MOE_BF16 or MOE_FP8_E4M3); a row whose
 *               sorted_pair entry lies outside [0, P) is skipped.
 *  x_scales     FP8 only, [T, d/128] fp32; x_perm_scales [P, d/128] receives the gathered rows.
 *  workspace    device scratch of at least moe_permute_workspace_size(T, k, E) bytes.
 * ------------------------------------------------------------------------------------------ */
moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, const void* x,
                       moe_dtype x_dtype, const float* x_scales, int d, void* x_perm,
                       float* x_perm_scales, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

size_t moe_permute_workspace_size(int T, int k, int E);

/* ------------------------------------------------------------------------------------------
 * fp8_quantize_act - dynamic per-token, per-group activation quantisation to e4m3.
 * (Transformers "Fine-grained FP8" page, introduction: activations are quantised per group per
 * token, the group matching the weights' 128 input channels, with scales computed at run time.)
 *
 *  x          [rows_in, K] of x_dtype (MOE_F32 or MOE_BF16).
 *  row_index  nullable [M] int32: output row i quantises input row row_index[i] (gather while
 *             quantising); NULL means output row i = input row i (rows_in = M).
 *  q          [M, K] e4m3 codes out; scales [M, K/group] fp32 out.
 *  Per group: s = amax/448 in fp32 (s = 1 if the group is all zero), q = e4m3(v / s) with IEEE
 *  fp32 division, round-to-nearest-even, saturating at +-448. group must be 128; K % 128 == 0.
 * ------------------------------------------------------------------------------------------ */
moe_status fp8_quantize_act(const void* x, moe_dtype x_dtype, int M, int K, int group,
                            const int32_t* row_index, uint8_t* q, float* scales,
                            hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp8_quantize_act_ue8m0 - the same with UE8M0 scales (Transformers "Fine-grained FP8" page,
 * section "UE8M0 scale format": power-of-two scales stored as e8m0 bytes).
 *
 *  Arguments as fp8_quantize_act; scales [M, K/group] uint8 e8m0 bytes out.
 *  Per group: b is the byte of the smallest power of two 2^e with 448 * 2^e >= amax (b = 127 for
 *  an all-zero group; b clamped to 0..254), q = e4m3(v * 2^-e), round-to-nearest-even (the
 *  scaling is exact and no value exceeds 448). Errors as fp8_quantize_act.
 * ------------------------------------------------------------------------------------------ */
moe_status fp8_quantize_act_ue8m0(const void* x, moe_dtype x_dtype, int M, int K, int group,
                                  const int32_t* row_index, uint8_t* q, uint8_t* scales,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp8_quantize_weight - offline 128x128 block quantisation of expert weights to e4m3.
 * (Transformers "Fine-grained FP8" page, introduction: weights are quantised to 8 bits per
 * two-dimensional block, weight_block_size = (128, 128).)
 *
 *  w       [batch, N, K] of w_dtype (MOE_F32 or MOE_BF16), e.g. batch = E experts.
 *  q       [batch, N, K] e4m3 codes out; scales [batch, N/128, K/128] fp32 out.
 *  Same rounding rule as fp8_quantize_act with the block's absmax. N % 128 == K % 128 == 0.
 * ------------------------------------------------------------------------------------------ */
moe_status fp8_quantize_weight(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                               int block, uint8_t* q, float* scales, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp8_quantize_weight_ue8m0 - 128x128 block quantisation with UE8M0 scales (Transformers
 * "Fine-grained FP8" page, section "UE8M0 scale format").
 *
 *  Arguments as fp8_quantize_weight; scales [batch, N/128, K/128] uint8 e8m0 bytes out, chosen
 *  by the fp8_quantize_act_ue8m0 rule with the block's absmax. Errors as fp8_quantize_weight.
 * ------------------------------------------------------------------------------------------ */
moe_status fp8_quantize_weight_ue8m0(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                                     int block, uint8_t* q, uint8_t* scales, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp4_quantize_weight_mx - expert weights to FP4 E2M1 with MX block scales (Transformers
 * "Experts backends" page, notes on FP8 and FP4 quantised experts packed as int8 with UE8M0 or
 * float32 scales; "Fine-grained FP8" page, section "UE8M0 scale format": FP4 experts with UE8M0
 * weight scales).
 *
 *  w       [batch, N, K] of w_dtype (MOE_F32 or MOE_BF16).
 *  q       [batch, N, K/2] packed E2M1 out; scales [batch, N, K/32] e8m0 bytes out: one per row
 *          per 32 consecutive input channels.
 *  Per block: b is the byte of the smallest power of two 2^e with 6 * 2^e >= amax (127 for an
 *  all-zero block, clamped to 0..254), codes E2M1(v * 2^-e) to nearest, ties to the even code.
 *  K % 32 == 0 (MOE_ERR_UNSUPPORTED otherwise); bad pointers or sizes: MOE_ERR_INVALID_ARGUMENT.
 * ------------------------------------------------------------------------------------------ */
moe_status fp4_quantize_weight_mx(const void* w, moe_dtype w_dtype, int batch, int N, int K,
                                  uint8_t* q, uint8_t* scales, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * fp4_tile_weight - packed E2M1 weights from row order to the matrix-fragment order that
 * moe_experts_forward streams (a byte permutation; the layout of the block-scaled matrix
 * instruction with an FP4 operand, as measured on gfx950).
 *
 *  q        [batch, N, K/2] packed E2M1 rows (as fp4_quantize_weight_mx writes them).
 *  q_tiled  out, same size, must not overlap q: for each b, each 16-row group n16 = n / 16 and
 *           each 128-wide K block c, 1024 bytes at ((b * N/16 + n16) * K/128 + c) * 1024; in it,
 *           16 bytes per lane l = r + 16 g (r, g < 16, 4): row 16 n16 + r, K = 128 c + 32 g ..
 *           128 c + 32 g + 31, packed as in q.
 *  N % 16 == 0, K % 128 == 0, both pointers 16-byte aligned (MOE_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------------------------ */
moe_status fp4_tile_weight(const uint8_t* q, int batch, int N, int K, uint8_t* q_tiled,
                           hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * moe_experts_forward - both grouped projections of every selected expert.
 * (Transformers "Experts backends" page: introduction and backends table rows grouped_mm,
 * deepgemm_megamoe, sonicmoe; the decode-time switch to a small-batch kernel; AWS fused-MoE news
 * page, sections on swap-AB: small token counts put the large weight dimension on the matrix
 * unit's fixed-size side.)
 *
 * Gate and up projections run as one grouped GEMM whose epilogue applies SwiGLU and writes the
 * hidden activation h [P, f] to the workspace (bf16; e4m3 + per-128 scales on the fp8 path).
 * The down projection runs as a second grouped GEMM whose epilogue writes y in a->y_layout.
 * Small batches (few rows per expert, see moe_experts_small_batch) use weight-streaming kernels
 * with the weight rows on the MFMA M side.
 * a->phase selects both projections (MOE_PHASE_ALL) or one of them (see moe_experts_phase); an
 * unknown value is MOE_ERR_INVALID_ARGUMENT.
 *
 * Supported dtype combinations (act_dtype / w_dtype / y_dtype):
 *    F32 / F32 / F32                 fp32 everywhere
 *    BF16 / BF16 / BF16 or F32       bf16 MFMA, fp32 accumulation
 *    FP8_E4M3 / FP8_E4M3 / BF16 or F32
 *        x = e4m3 codes [T, d] with x_scales [T, d/128] (from fp8_quantize_act); weights e4m3
 *        with block scales; fp32 accumulation with per-128-K scale promotion; h is re-quantised
 *        per pair per 128 channels. d % 128 == f % 128 == 0.
 *        With scale_fmt = MOE_SCALE_UE8M0 every scale (x_scales from fp8_quantize_act_ue8m0,
 *        s_gate / s_up / s_down from fp8_quantize_weight_ue8m0) is an e8m0 byte; the matrix unit
 *        applies them as its per-row / per-column block scales (no promotion step) and h is
 *        re-quantised with UE8M0 scales. scale_fmt other than MOE_SCALE_F32 on a non-fp8 path,
 *        or an unknown value, is MOE_ERR_INVALID_ARGUMENT.
 *    FP8_E4M3 / FP4_E2M1 / BF16 or F32, scale_fmt = MOE_SCALE_UE8M0 (MOE_SCALE_F32 is
 *        MOE_ERR_UNSUPPORTED)
 *        weights packed E2M1 [E, f, d/2] and [E, d, f/2] in matrix-fragment order (from
 *        fp4_quantize_weight_mx, then fp4_tile_weight) with MX scales (row order, as the
 *        quantiser writes them) s_gate / s_up [E, f, d/32] and s_down [E, d, f/32]; x and h
 *        e4m3 with UE8M0 per-128 scales. d % 128 == f % 128 == 0; the three MX scale arrays
 *        4-byte aligned (MOE_ERR_UNSUPPORTED otherwise).
 * Alignment on every path but F32 / F32 / F32: x, w_gate, w_up, w_down and y 16-byte aligned,
 * fp32 scale arrays 4-byte aligned (MOE_ERR_UNSUPPORTED otherwise). Contiguous tensors from a
 * device allocator, and their slices along the expert or token dimension, satisfy this.
 * ------------------------------------------------------------------------------------------ */
/* Which projections one moe_experts_forward call runs. A MOE_PHASE_GATE_UP call followed, in
 * stream order, by a MOE_PHASE_DOWN call with the same arguments and the same workspace (whose h
 * the first call wrote) computes exactly what one MOE_PHASE_ALL call computes; a caller can put
 * its own work on the stream between the two (e.g. event records to time each projection). */
typedef enum {
  MOE_PHASE_ALL = 0,      /* gate/up + SwiGLU, then down */
  MOE_PHASE_GATE_UP = 1,  /* gate/up + SwiGLU only: h in the workspace */
  MOE_PHASE_DOWN = 2,     /* down only, from the h of a previous MOE_PHASE_GATE_UP call */
  MOE_PHASE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  MOE_PHASE_RANGE_MAX_ = 0x7FFFFFFF
} moe_experts_phase;

typedef struct {
  int T, d, f, E, k;
  moe_dtype act_dtype;           /* dtype of x */
  moe_dtype w_dtype;             /* dtype of the expert weights */
  moe_dtype y_dtype;             /* element type of y for MOE_Y_PERMUTED / MOE_Y_SLOTS */
  moe_y_layout y_layout;
  const void* x;                 /* [T, d] token activations */
  const void* x_scales;          /* FP8: [T, d/128], fp32 or e8m0 bytes (scale_fmt) */
  const void* w_gate;            /* [E, f, d] */
  const void* w_up;              /* [E, f, d] */
  const void* w_down;            /* [E, d, f] */
  const void* s_gate;            /* FP8: [E, f/128, d/128], fp32 or e8m0 bytes (scale_fmt) */
  const void* s_up;              /* FP8: [E, f/128, d/128] */
  const void* s_down;            /* FP8: [E, d/128, f/128] */
  const int32_t* offsets;        /* [E+1] from moe_permute */
  const int32_t* sorted_pair;    /* [P] from moe_permute */
  const float* topk_w;           /* [T, k] routing weights (MOE_Y_SLOTS, MOE_Y_ACC_F32) */
  void* y;                       /* output, see moe_y_layout */
  void* workspace;               /* >= moe_experts_workspace_size(...) bytes */
  size_t workspace_bytes;
  moe_scale_fmt scale_fmt;       /* FP8 block-scale format (MOE_SCALE_F32 elsewhere) */
  moe_experts_phase phase;       /* which projection(s) this call runs (MOE_PHASE_ALL = both) */
} moe_experts_args;

moe_status moe_experts_forward(const moe_experts_args* a, hipStream_t stream);

size_t moe_experts_workspace_size(int T, int d, int f, int E, int k, moe_dtype act_dtype,
                                  moe_dtype w_dtype);

/* Which kernels moe_experts_forward runs for these sizes (the Transformers "Experts backends"
 * page, decode-time switch: a kernel made for small batches below some size; the AWS fused-MoE
 * news page, swap-AB for small token counts): 1 = the small-batch weight-streaming kernels (weight
 * rows on the matrix unit's M side), 0 = the tiled grouped GEMMs, -1 = no kernel for this dtype
 * combination or invalid sizes. The switch is on the mean number of rows per expert: small-batch
 * while T*k <= 12 E (bf16) or T*k <= 16 E (e4m3 / E2M1 weights; bf16 also needs d % 128 == 0 and
 * f % 128 == 0); fp32 layers always take the tiled kernels. */
int moe_experts_small_batch(int T, int d, int f, int E, int k, moe_dtype act_dtype,
                            moe_dtype w_dtype);

/* ------------------------------------------------------------------------------------------
 * moe_combine - weighted sum of each token's k expert outputs.
 * (Transformers "Experts backends" page, introduction; lira-now explainer, section 4 (router +
 * combine) and section 5 step 6: y = sum_i w_i * expert_i(x).)
 *
 *  MOE_Y_PERMUTED: out[t] = sum_{j<k} topk_w[t][j] * y[pair_pos[t*k+j]]   (y [P, d])
 *  MOE_Y_SLOTS:    out[t] = sum_{j<k} y[t][j]                             (y [T, k, d])
 *  MOE_Y_ACC_F32:  out[t] = y[t]                                          (y [T, d] fp32)
 *  Sums run in fp32 in the order j = 0..k-1; one rounding to out_dtype (MOE_F32 or MOE_BF16).
 *  pair_pos and topk_w are read only for MOE_Y_PERMUTED; a pair whose pair_pos lies outside
 *  [0, T*k) (moe_permute's mark for an out-of-range expert id) adds nothing.
 * ------------------------------------------------------------------------------------------ */
moe_status moe_combine(const void* y, moe_dtype y_dtype, moe_y_layout layout,
                       const int32_t* pair_pos, const float* topk_w, int T, int k, int d,
                       void* out, moe_dtype out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * moe_fused_forward - the whole layer for small batches (decode) in one call: one routing kernel
 * (router logits or given logits, top-k with renormalised weights, and for fp8 / FP4 experts the
 * activation quantisation), the two expert projections (for fp8 / FP4 with the h quantiser between
 * them) and the combine. After the single fused MoE kernel of the AWS fused-MoE news page, as far
 * as it pays here: no permutation is materialised (each expert's workgroups find its pairs in
 * topk_ids), and the steps that need every workgroup's results (h quantisation, combine) stay
 * launches of their own, since a hand-off inside a launch costs each workgroup an L2 write-back
 * and invalidation on gfx950. Computes what moe_route + moe_permute (+ fp8_quantize_act) +
 * moe_experts_forward (slots) + moe_combine compute: routing ids and weights bit-identical to that
 * sequence, and the output too wherever the sequence runs the same small-batch kernels
 * (moe_experts_small_batch(...) == 1; beyond that batch size it runs the tiled GEMMs, whose
 * intermediate rounding differs).
 *
 *  T*k <= 256 pairs (MOE_ERR_UNSUPPORTED otherwise); d % 128 == f % 128 == 0; E <= 1024, k <= E.
 *  x [T, d] (MOE_BF16, or MOE_F32 with fp8 / FP4 experts), 16-byte aligned.
 *  logits [T, E] fp32 router logits, or NULL: computed as x . w_router^T (w_router [E, d] fp32,
 *    16-byte aligned), and written to logits_out [T, E] when that is non-NULL.
 *  w_dtype / scale_fmt and the weight and scale arrays: as for moe_experts_forward, alignment
 *    included (MOE_BF16 with
 *    bf16 x; MOE_FP8_E4M3 with fp32 or UE8M0 block scales; MOE_FP4_E2M1 in fragment order with MX
 *    scales, UE8M0 only); fp8 / FP4 quantise x per token per 128 channels here.
 *  out [T, d] (out_dtype MOE_BF16 or MOE_F32); topk_ids / topk_w [T, k] out (required).
 *  workspace: >= moe_fused_workspace_size(...) bytes, caller-owned, any contents; calls that share
 *    a workspace must not overlap on the device. Device errors: MOE_ERR_DEVICE.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  int T, d, f, E, k;
  moe_dtype x_dtype;
  moe_dtype w_dtype;
  moe_scale_fmt scale_fmt;
  const void* x;                 /* [T, d] */
  const float* logits;           /* [T, E] or NULL (router GEMM) */
  const float* w_router;         /* [E, d] fp32, used when logits == NULL */
  float* logits_out;             /* nullable [T, E] */
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* s_gate;
  const void* s_up;
  const void* s_down;
  void* out;                     /* [T, d] */
  moe_dtype out_dtype;
  int32_t* topk_ids;             /* [T, k] out */
  float* topk_w;                 /* [T, k] out */
  void* workspace;
  size_t workspace_bytes;
} moe_fused_args;

moe_status moe_fused_forward(const moe_fused_args* a, hipStream_t stream);

/* Bytes of workspace moe_fused_forward needs (0 for unsupported sizes). */
size_t moe_fused_workspace_size(int T, int d, int f, int E, int k, moe_dtype w_dtype,
                                moe_dtype out_dtype);

/* ------------------------------------------------------------------------------------------
 * moe_fused_forward_noalloc - moe_fused_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Computes exactly what moe_fused_forward computes (same kernels, bit-identical outputs), but
 * instead of a caller's workspace it uses a fixed device array inside the library, one per GPU,
 * of MOE_NOALLOC_SCRATCH_BYTES bytes, which the GPU holds until the process ends; a->workspace
 * and a->workspace_bytes are ignored. The call allocates and frees nothing. The caller still
 * passes x, the weights and the outputs.
 *  - Limit: moe_fused_workspace_size(...) of the call must be <= MOE_NOALLOC_SCRATCH_BYTES
 *    (e.g. the Mixtral-shaped decode layer, d = 4096, f = 14336, with bf16, e4m3 or FP4 experts at
 *    every batch the fused path takes, T*k <= 256); larger requests return MOE_ERR_UNSUPPORTED
 *    and enqueue nothing. Other errors as moe_fused_forward.
 *  - The first call on a device looks up that device's array (the device current at the call,
 *    which must be the stream's device); a failed lookup returns MOE_ERR_DEVICE.
 *  - Every call on one GPU shares that GPU's array and leaves its contents behind; nothing in the
 *    fused path reads the array before writing it. Calls that overlap on one GPU (different
 *    streams or host threads without ordering between them) race on the array: order them.
 * ------------------------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

moe_status moe_fused_forward_noalloc(const moe_fused_args* a, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
