/*
 * moe.h -- C ABI of the MI355X (gfx950) fused Mixture-of-Experts forward.
 *
 * The forward pass routes tokens to experts, sorts the routes into
 * per-expert tile-padded order, runs a gather grouped GEMM1 (gate/up
 * projection) on block-scaled 4-bit weights with a fused SwiGLU epilogue
 * (and, per mode, a requantisation of its output), a grouped GEMM2 (down
 * projection), and a routing-weighted top-k finalize into [M, H].  It is
 * the problem stated by "flashinfer.fused_moe.cute_dsl_fused_moe" (FlashInfer
 * API reference; signature and Parameters), with the routing plan of
 * "vllm.models.flint.ops.moe_cute" (grouped_moe), the route-order
 * finalize and `accumulate` of "flashinfer.fused_moe.alphamoe_nvfp4_routed_moe"
 * (summary, Parameters) and the MXFP8 x MXFP4 mode of FlashInfer pull request
 * 4440 ("feat(moe): MXFP8 x MXFP4 CuTe-DSL fused MoE for SM100, plus
 * large-batch routing locality", description).
 *
 * Conventions shared by every entry point
 *  - Pointers named as device pointers point to device memory of the
 *    current HIP device; all are caller-owned.  The library never
 *    allocates, frees or reads back device memory and never synchronises the
 *    host; every call only enqueues work on `stream` (a hipStream_t, NULL
 *    for the default stream), so calls can be captured into a HIP graph.
 *  - The library has no mutable global state apart from the scratch array
 *    of moe_forward_noalloc; concurrent calls of the other entry points on
 *    different streams are safe when their buffers do not overlap.
 *  - Arguments are checked on the host before anything is enqueued.  On a
 *    non-MOE_OK return nothing has been enqueued, except MOE_ERR_DEVICE,
 *    which reports a failed launch.
 *  - Data values are not validated: an expert id outside
 *    [local_expert_offset, local_expert_offset + num_local_experts) is a
 *    route of another GPU's share and is dropped, whatever its value.
 *  - bf16 values are passed as uint16_t bit patterns; E4M3 ("fn"), E8M0
 *    and packed E2M1 values as uint8_t codes.  Packed E2M1 holds element
 *    2i in the low nibble and element 2i+1 in the high nibble of byte i.
 *  - All tensors are row-major and contiguous unless a stride is given.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1, /* NULL where required, non-NULL where forbidden, bad sizes */
  MOE_ERR_UNSUPPORTED = 2,      /* a valid request this build does not implement (the message names it) */
  MOE_ERR_WORKSPACE = 3,        /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_DEVICE = 4,           /* a HIP launch failed */
  MOE_ERR_SCRATCH_TOO_SMALL = 5 /* moe_forward_noalloc: the pass needs more than MOE_NOALLOC_SCRATCH_BYTES */
} moe_status_t;

/* Quantisation modes ("quant_mode" of cute_dsl_fused_moe, Parameters):
 *  W4A16     : x bf16 [M,H]; weights NVFP4 = packed E2M1 + linear E4M3
 *              block-16 scales + a per-expert fp32 scale; FC1 output bf16.
 *  W4A4      : x NVFP4 (packed E2M1 [M,H/2] + E4M3 [M,H/16]); weights as
 *              W4A16; the FC1 output is requantised to NVFP4 with the
 *              global scale fc2_input_scale.
 *  MXFP8_MXFP4 ("w4a8"): x MXFP8 (E4M3 [M,H] + E8M0 block-32 [M,H/32]);
 *              weights MXFP4 = packed E2M1 + E8M0 block-32 scales; FC1
 *              output requantised to MXFP8; w*_alpha still multiply. */
typedef enum { MOE_QUANT_W4A16 = 0, MOE_QUANT_W4A4 = 1, MOE_QUANT_MXFP8_MXFP4 = 2 } moe_quant_mode_t;

/* Finalize ("use_fused_finalize" of cute_dsl_fused_moe):
 *  DETERMINISTIC: GEMM2 writes unweighted bf16 rows y2 [route_slots, H] in
 *                 permuted order; moe_finalize then reduces each token's
 *                 routes in route order (bitwise reproducible).
 *  ATOMIC       : the GEMM2 epilogue adds w * routed_scaling_factor * y2
 *                 into `out` with packed-bf16 atomics (not reproducible
 *                 bit for bit, and each add rounds to bf16; no y2 buffer).
 *                 The default of the pages' API (use_fused_finalize);
 *                 here DETERMINISTIC is the default, the zero value.
 *                 Faster at decode sizes; at large batches the atomics
 *                 contend and it is slower. */
typedef enum { MOE_FINALIZE_DETERMINISTIC = 0, MOE_FINALIZE_ATOMIC = 1 } moe_finalize_mode_t;

/* How moe_sort parallelises.  Both give the identical plan.
 *  AUTO  : one workgroup for small route counts, spans above.
 *  SINGLE: one workgroup walks every route.
 *  SPAN  : each workgroup owns one contiguous span of routes (histogram,
 *          cross-span scan, stable scatter inside the span) -- the
 *          contiguous-window ordering of FlashInfer pull request 4440. */
typedef enum { MOE_ROUTE_ORDER_AUTO = 0, MOE_ROUTE_ORDER_SINGLE = 1, MOE_ROUTE_ORDER_SPAN = 2 } moe_route_order_t;

/* Which launch sequence moe_forward takes for a W4A16 batch at tile 16.
 *  AUTO  : the two-launch decode path when it applies (see moe_forward) and
 *          the batch is expected to give each local expert at most 1.25
 *          routes (4 * M * top_k <= 5 * num_experts): it streams an expert's
 *          weights once per route row, so beyond that the tiled path, which
 *          streams them once per expert, is faster;
 *  DECODE: the two-launch decode path whenever it applies;
 *  TILED : never the decode path. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_DECODE = 1, MOE_PATH_TILED = 2 } moe_path_t;

/* Routing plan (the moe_sort outputs of "vllm.models.flint.ops.moe_cute",
 * grouped_moe).  Route r = t * top_k + j.  Inside each local expert the
 * routes take consecutive slots in ascending r; each expert's range is
 * padded to a multiple of `tile` and the ranges follow expert order.
 * Device arrays (carved from a caller workspace by moe_plan_init):
 *   expanded_to_permuted [M*top_k]  slot of route r, -1 if not local
 *   permuted_to_expanded [route_slots] route in slot s, -1 for padding
 *   tile_to_expert       [max_tiles] local expert of tile i, -1 unused
 *   tile_to_mn_limit     [max_tiles] exclusive end slot of tile i's valid
 *                                    rows, -1 unused
 *   num_tiles            [1]         tiles in use
 *   expert_offsets       [E_l+1]     first slot of each expert; [E_l] = used slots
 *   expert_counts        [E_l]       local routes per expert
 * route_slots = round_up(M*top_k + min(E_l, M*top_k)*(tile-1), tile) is an
 * upper bound that needs no host read-back; max_tiles = route_slots/tile. */
typedef struct moe_plan {
  int32_t* expanded_to_permuted;
  int32_t* permuted_to_expanded;
  int32_t* tile_to_expert;
  int32_t* tile_to_mn_limit;
  int32_t* num_tiles;
  int32_t* expert_offsets;
  int32_t* expert_counts;
  int32_t* scratch; /* sort scratch (span histograms) */
  int64_t route_slots;
  int32_t max_tiles;
  int32_t tile;
  int32_t M;
  int32_t top_k;
  int32_t num_local_experts;
  int32_t max_spans; /* span workgroups the scratch is sized for */
} moe_plan_t;

/* Static text for a status code. */
const char* moe_status_string(moe_status_t status);

/* Slot capacity of a plan: the number of permuted rows the grouped GEMMs
 * are sized for, the counterpart of get_max_num_permuted_tokens(num_tokens,
 * top_k, num_local_experts, route_tile) in "vllm.models.flint.ops.moe_cute"
 * (grouped_moe; the page names the function and does not print it).  It is
 * round_up(M*top_k + min(E_l, M*top_k)*(tile-1), tile): every local route
 * plus at most tile-1 padding rows for each expert that has a route, which
 * bounds the padded total for any routing without reading it back.
 * Returns 0 for M < 0, top_k < 1, num_local_experts < 1 or tile < 1. */
int64_t moe_route_slots(int M, int top_k, int num_local_experts, int tile);

/* Bytes of device workspace a plan needs, 256-byte aligned pieces: the
 * counterpart of allocate_moe_sort_buffers in "vllm.models.flint.ops.moe_cute"
 * (grouped_moe), caller-owned as the routing workspace of
 * "flashinfer.fused_moe.alphamoe_nvfp4_routed_moe" (Parameters).  0 for
 * arguments moe_plan_init would reject. */
size_t moe_plan_workspace_size(int M, int top_k, int num_local_experts, int tile);

/* Carve a plan out of `workspace` (device memory, >= moe_plan_workspace_size
 * bytes, 256-byte aligned).  Host-only; enqueues nothing.  tile must be a
 * power of two in [16, 256]; M >= 0, top_k in [1, 64], num_local_experts in
 * [1, 512] (MOE_ERR_INVALID_ARGUMENT, or MOE_ERR_UNSUPPORTED for a tile or
 * expert count outside these limits; MOE_ERR_WORKSPACE for a missing,
 * unaligned or short workspace). */
moe_status_t moe_plan_init(moe_plan_t* plan, void* workspace, size_t workspace_bytes, int M, int top_k,
                           int num_local_experts, int tile);

/* moe_sort: build the routing plan from topk_ids (device int32 [M, top_k],
 * global expert ids): the moe_sort step of "vllm.models.flint.ops.moe_cute"
 * (grouped_moe: tile_idx_to_expert_idx, tile_idx_to_mn_limit,
 * expanded_idx_to_permuted_idx, permuted_idx_to_expanded_idx,
 * total_num_padded_tokens), restricted to this GPU's experts as
 * num_local_experts / local_expert_offset of
 * "flashinfer.fused_moe.cute_dsl_fused_moe" (Parameters) state.  Routes with
 * local_expert_offset <= id < local_expert_offset + num_local_experts belong
 * to this GPU; others are dropped.  The order inside an expert is ascending
 * route index (the pages' order is atomic arrival; this one is stable, so
 * the plan is bit-exact and reproducible), and SPAN gives the same plan as
 * SINGLE through the contiguous per-workgroup route spans of FlashInfer pull
 * request 4440 (description, item 2).  Requires local_expert_offset >= 0 and
 * local_expert_offset + num_local_experts <= num_experts; M, top_k and
 * num_local_experts must equal the plan's (MOE_ERR_INVALID_ARGUMENT). */
moe_status_t moe_sort(const int32_t* topk_ids, int M, int top_k, int num_experts, int num_local_experts,
                      int local_expert_offset, moe_route_order_t route_order, const moe_plan_t* plan,
                      moe_stream_t stream);

/* moe_grouped_gemm1_swiglu: for every valid slot s (route r, token
 * t = r / top_k, local expert e), gather x[t], multiply by W1[e]^T in fp32,
 * scale by w1_alpha[e] in fp32 and apply
 *   y1 = min(g, limit) * sigmoid(swiglu_alpha * min(g, limit)) *
 *        (clamp(u, -limit, limit) + swiglu_beta)
 * to gate g (W1 rows [0, I)) and up u (rows [I, 2I)), rounded once to bf16
 * ("vllm.models.flint.ops.moe_cute" docstring; SwiGLU parameters of
 * cute_dsl_fused_moe).  Then store y1 per mode:
 *   W4A16      : y1 bf16 [route_slots, I]; y1_sf NULL
 *   W4A4       : packed E2M1 [route_slots, I/2] + E4M3 y1_sf [route_slots, I/16],
 *                quantised with global scale *fc2_input_scale
 *   MXFP8_MXFP4: E4M3 [route_slots, I] + E8M0 y1_sf [route_slots, I/32]
 * Inputs (device): x as in moe_quant_mode_t with row stride x_row_stride in
 * x's storage units (bf16 elements, or bytes; 0 = contiguous rows; shorter
 * than a row: MOE_ERR_INVALID_ARGUMENT; not a multiple of 16 bytes:
 * MOE_ERR_UNSUPPORTED); x_sf contiguous, NULL in W4A16.  w1 packed E2M1 [E_l, 2I, H/2]; w1_sf E4M3 [E_l, 2I, H/16] (NVFP4)
 * or E8M0 [E_l, 2I, H/32] (MX); w1_alpha fp32 [E_l].  fc2_input_scale: a
 * device fp32 scalar, required in W4A4 and NULL otherwise.  H and I must be
 * multiples of the scale block (16 NVFP4, 32 MX; else
 * MOE_ERR_INVALID_ARGUMENT) and of 32 (else MOE_ERR_UNSUPPORTED); tiles that
 * N = I or K = H does not fill are masked, following the partial-N-tile
 * support of FlashInfer pull request 4440 (description, item 1).
 * Padding rows of y1 are not written. */
moe_status_t moe_grouped_gemm1_swiglu(moe_quant_mode_t mode, const void* x, const uint8_t* x_sf,
                                      int64_t x_row_stride, const moe_plan_t* plan, const uint8_t* w1,
                                      const uint8_t* w1_sf, const float* w1_alpha, int H, int I,
                                      float swiglu_alpha, float swiglu_beta, float swiglu_limit,
                                      const float* fc2_input_scale, void* y1, uint8_t* y1_sf,
                                      moe_stream_t stream);

/* FC1 activations ("flashinfer.fused_moe.cute_dsl_fused_moe", Parameters
 * activation_type, situ_beta, situ_linear_beta). */
typedef enum moe_activation {
  MOE_ACT_SWIGLU = 0,      /* gated SwiGLU with swiglu_alpha / beta / limit; SiTU when situ_beta > 0 */
  MOE_ACT_GEGLU_TANH = 1,  /* gated GeGLU, tanh-approximate GELU of the gate */
  MOE_ACT_RELU2 = 2        /* non-gated ReLU^2: W1 holds I rows, y1[j] = max(h_j, 0)^2 */
} moe_activation_t;

/* moe_grouped_gemm1_act: moe_grouped_gemm1_swiglu with the FC1 activation
 * chosen by `activation`, and two optional scales of the accumulator:
 *   w1_alpha_up: device fp32 [E_l], the up half's own per-expert scale
 *     (gate rows take w1_alpha; "flashinfer.fused_moe.
 *     alphamoe_nvfp4_routed_moe", Parameters output1_scale_gate_scalar and
 *     output1_scale_scalar).  NULL: w1_alpha for both halves.
 *   per_token_scale: device fp32 [M], W4A4 only: the token's input row scale
 *     ("flashinfer.fused_moe.cute_dsl_fused_moe", Parameters
 *     per_token_scale), applied after the expert scale:
 *     g = fp32(fp32(acc_g) * w1_alpha[e]) * per_token_scale[t], likewise u.
 *     NULL: none.  Non-NULL outside W4A4: MOE_ERR_INVALID_ARGUMENT.
 *   fc1_bias: device fp32 [E_l, 2I] (gate rows, then up rows), added to g and
 *     u after the scales, before the activation ("flashinfer.fused_moe.
 *     cutlass_fused_moe", Parameters fc1_expert_biases).  NULL: none.
 * The activations (same Parameters of cute_dsl_fused_moe):
 *   MOE_ACT_SWIGLU, situ_beta == 0: the SwiGLU above.
 *   MOE_ACT_SWIGLU, situ_beta  > 0: SiTU,
 *       y1 = situ_beta * tanh(g / situ_beta) * sigmoid(g) * u',
 *       u' = situ_linear_beta * tanh(u / situ_linear_beta) if situ_linear_beta > 0, else u.
 *   MOE_ACT_GEGLU_TANH: y1 = g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3))) * u.
 *   MOE_ACT_RELU2 (non-gated): w1 is [E_l, I, H/2] codes + [E_l, I, H/16 or
 *       H/32] scales, one row per y1 column; y1[j] = max(h_j, 0)^2 with h_j
 *       row j's accumulator scaled like a gate value (w1_alpha, per-token
 *       scale, fc1_bias [E_l, I]).  w1_alpha_up must be NULL.
 * Everything else (inputs, layouts, requantisation, rounding once to bf16)
 * is as in moe_grouped_gemm1_swiglu.  MOE_ERR_INVALID_ARGUMENT: an unknown
 * activation; situ_beta or situ_linear_beta negative or not finite;
 * situ_linear_beta > 0 without situ_beta > 0; GeGLU or SiTU together with
 * non-default SwiGLU parameters (1, 0, FLT_MAX), GeGLU or ReLU^2 with SiTU
 * parameters, ReLU^2 with w1_alpha_up. */
moe_status_t moe_grouped_gemm1_act(moe_quant_mode_t mode, const void* x, const uint8_t* x_sf,
                                   int64_t x_row_stride, const moe_plan_t* plan, const uint8_t* w1,
                                   const uint8_t* w1_sf, const float* w1_alpha, const float* w1_alpha_up, int H,
                                   int I, int activation, float swiglu_alpha, float swiglu_beta,
                                   float swiglu_limit, float situ_beta, float situ_linear_beta,
                                   const float* fc2_input_scale, const float* per_token_scale,
                                   const float* fc1_bias, void* y1, uint8_t* y1_sf, moe_stream_t stream);

/* moe_grouped_gemm2: for every valid slot s of local expert e, multiply the
 * stored FC1 output (decoded as moe_grouped_gemm1_swiglu wrote it; in W4A4
 * fc2_input_scale is part of w2_alpha) by W2[e]^T in fp32 and scale by
 * w2_alpha[e] in fp32.
 *   finalize DETERMINISTIC (y2 != NULL, out == NULL): y2[s] = bf16(result),
 *     bf16 [route_slots, H], unweighted ("grouped_moe" returns permuted
 *     unweighted bf16 rows).
 *   finalize ATOMIC (y2 == NULL, out != NULL): out[t] += bf16(w[r] *
 *     routed_scaling_factor * result) with packed-bf16 atomics; topk_weights
 *     fp32 [M, top_k] required; `out` must hold its seed (zeros, or the
 *     previous output when accumulating).
 * w2 packed E2M1 [E_l, H, I/2]; w2_sf E4M3 [E_l, H, I/16] or E8M0
 * [E_l, H, I/32]; w2_alpha fp32 [E_l].  Padding rows of y2 are not written.
 * y2 must be 16-byte aligned and out 4-byte aligned (else
 * MOE_ERR_UNSUPPORTED). */
moe_status_t moe_grouped_gemm2(moe_quant_mode_t mode, const void* y1, const uint8_t* y1_sf,
                               const moe_plan_t* plan, const uint8_t* w2, const uint8_t* w2_sf,
                               const float* w2_alpha, int H, int I, uint16_t* y2, const float* topk_weights,
                               float routed_scaling_factor, uint16_t* out, moe_stream_t stream);

/* moe_grouped_gemm2_bias: moe_grouped_gemm2 with a per-expert GEMM2 bias
 * fc2_bias, device fp32 [E_l, H], added to alpha2 * result before y2's bf16
 * rounding (and before the routing weight in atomic mode)
 * ("flashinfer.fused_moe.cutlass_fused_moe", Parameters fc2_expert_biases;
 * the page calls it the GEMM1 bias, read as GEMM2's).  NULL: none. */
moe_status_t moe_grouped_gemm2_bias(moe_quant_mode_t mode, const void* y1, const uint8_t* y1_sf,
                                    const moe_plan_t* plan, const uint8_t* w2, const uint8_t* w2_sf,
                                    const float* w2_alpha, const float* fc2_bias, int H, int I, uint16_t* y2,
                                    const float* topk_weights, float routed_scaling_factor, uint16_t* out,
                                    moe_stream_t stream);

/* moe_finalize: deterministic weighted top-k reduction
 * ("flashinfer.fused_moe.alphamoe_nvfp4_routed_moe", summary and
 * `accumulate`; the caller-side reduction of "grouped_moe"):
 *   acc = accumulate ? out[t,h] : 0                         (fp32)
 *   for j = 0 .. top_k-1 with a local route r = t*top_k + j:
 *     acc = acc + fp32(topk_weights[r] * routed_scaling_factor) * y2[slot(r), h]
 *   out[t,h] = bf16(acc)
 * with separate fp32 multiplies and adds.  accumulate = 0 overwrites `out`
 * and equals accumulating onto a zero output bit for bit.  A token with no
 * local route gets 0 (or keeps its value when accumulating).  y2 bf16
 * [route_slots, H]; topk_weights fp32 [M, top_k]; out bf16 [M, H].  y2 and
 * out 16-byte aligned, H a multiple of 8 (else MOE_ERR_UNSUPPORTED). */
moe_status_t moe_finalize(const uint16_t* y2, const moe_plan_t* plan, const float* topk_weights, int H,
                          float routed_scaling_factor, int accumulate, uint16_t* out, moe_stream_t stream);

/* Options of moe_forward.  moe_opts_init() fills the defaults. */
typedef struct moe_opts {
  float swiglu_alpha;            /* default 1.0 */
  float swiglu_beta;             /* default 0.0 */
  float swiglu_limit;            /* default FLT_MAX (no clamp) */
  const float* fc2_input_scale;  /* device fp32 scalar: W4A4 only, else NULL */
  float routed_scaling_factor;   /* default 1.0 */
  int accumulate;                /* 0: overwrite out; 1: add into out */
  int finalize_mode;             /* moe_finalize_mode_t, default DETERMINISTIC */
  int route_order;               /* moe_route_order_t, default AUTO */
  int tile;                      /* route tile; 0 = moe_default_tile() */
  int64_t x_row_stride;          /* 0 = contiguous rows */
  void* workspace;               /* device, >= moe_workspace_size() bytes, 256-byte aligned;
                                    any initial contents (see moe_workspace_size) */
  size_t workspace_bytes;
  void** phase_events;           /* optional: MOE_NUM_PHASE_EVENTS hipEvent_t recorded on the
                                    stream before sort, after sort, after GEMM1, after GEMM2,
                                    after finalize (timing); NULL = none */
  int activation;                /* moe_activation_t, default MOE_ACT_SWIGLU (rules as in
                                    moe_grouped_gemm1_act) */
  float situ_beta;               /* default 0 (SwiGLU); > 0 selects SiTU */
  float situ_linear_beta;        /* default 0 (no up-branch clamp) */
  const float* w1_alpha_up;      /* device fp32 [E_l]: the up half's scale; NULL = w1_alpha */
  const float* per_token_scale;  /* device fp32 [M], W4A4 only: GEMM1 input row scale; NULL = none */
  const float* fc1_bias;         /* device fp32 [E_l, 2I]: GEMM1 bias (moe_grouped_gemm1_act); NULL = none */
  const float* fc2_bias;         /* device fp32 [E_l, H]: GEMM2 bias (moe_grouped_gemm2_bias); NULL = none */
  int path;                      /* moe_path_t, default AUTO */
} moe_opts_t;

#define MOE_NUM_PHASE_EVENTS 5

void moe_opts_init(moe_opts_t* opts);

/* The route tile moe_forward uses when opts->tile == 0 (the route_tile of
 * "vllm.models.flint.ops.moe_cute", grouped_moe, which the page's caller
 * picks per batch).  It estimates the routes per local expert as
 * M * top_k / num_experts (the local share of the routes spread over the
 * local experts) and returns 16 up to 16 routes, then by mode (the
 * fastest kernel measured at each size):
 *   W4A16      : 32 up to 32 routes (the expert-streaming kernel), else 128
 *                (the wide-tile kernel);
 *   W4A4       : 32 up to 48 routes, else 64 (the expert-streaming kernel
 *                at every larger size);
 *   MXFP8_MXFP4: 32 up to 48, 64 up to 96, 128 up to 384, else 256, the
 *                tile of the large-batch benchmark in FlashInfer pull
 *                request 4440. */
int moe_default_tile(int M, int top_k, int num_experts, int num_local_experts, moe_quant_mode_t mode);

/* Bytes of device workspace moe_forward needs: the caller-owned buffers of
 * "flashinfer.fused_moe.alphamoe_nvfp4_routed_moe" (Parameters: routing
 * workspace, permuted intermediates) in one allocation.  It holds, in
 * 256-byte aligned pieces: a counter block of the decode path (one done
 * count per 64 output columns, cleared by the forward's own GEMM1 launch),
 * the routing plan (moe_forward_plan), y1 (+ y1_sf) and, in deterministic
 * mode or on the decode path, y2.  The workspace needs no initial contents;
 * every piece is written before it is read within one call.  Two
 * moe_forward calls in flight at once must not share a workspace.  Returns
 * 0 for arguments moe_forward would reject as invalid. */
size_t moe_workspace_size(int M, int H, int I, int top_k, int num_local_experts, int tile,
                          moe_quant_mode_t mode, int finalize_mode);

/* The routing plan inside a moe_forward workspace: after a moe_forward on
 * that workspace has run with the same M, top_k, num_local_experts and tile
 * (the tile it used: opts->tile, or moe_default_tile), `plan` points at the
 * plan that forward built and used (every array of moe_plan_t, as moe_sort
 * writes them), also on the decode path, which builds it inside GEMM1.
 * Host-only, enqueues nothing.  MOE_ERR_WORKSPACE if the workspace is NULL
 * or too small for the plan; otherwise as moe_plan_init. */
moe_status_t moe_forward_plan(moe_plan_t* plan, void* workspace, size_t workspace_bytes, int M, int top_k,
                              int num_local_experts, int tile);

/* moe_forward: the whole pass, argument order as the
 * cute_dsl_fused_moe signature (x, x_sf, token_selected_experts,
 * token_final_scales, w1, w1_sf, w1_alpha, w2, w2_sf, w2_alpha,
 * num_experts, top_k, num_local_experts, local_expert_offset, quant_mode)
 * followed by the output, the shapes, the options and the stream.
 *   out: bf16 [M, H], overwritten (accumulate = 0) or added to; 16-byte
 *        aligned (else MOE_ERR_UNSUPPORTED).
 * Enqueues moe_sort, moe_grouped_gemm1_swiglu, moe_grouped_gemm2 and (in
 * deterministic mode) moe_finalize; in atomic mode with accumulate = 0 the
 * output is zero-filled first by a kernel.  Decode-sized W4A16 batches
 * (tile 16, M * top_k <= 1024, H and I multiples of 512, I <= 8192,
 * 4-byte aligned w1_sf and w2_sf, and the routing plan plus one bf16 row
 * of H within 64 KiB of LDS; opts->path selects when, see moe_path_t) take
 * two launches
 * instead: GEMM1 with the routing plan, then GEMM2, which finalizes too:
 * in deterministic mode the last workgroup per 64 output columns applies
 * the route-order finalize to them; in atomic mode every route row is
 * added into out with packed-bf16 atomics (GEMM1 clears out first unless
 * accumulating).
 * `out` is this GPU's share: the sum over its local routes only. */
moe_status_t moe_forward(const void* x, const uint8_t* x_sf, const int32_t* topk_ids, const float* topk_weights,
                         const uint8_t* w1, const uint8_t* w1_sf, const float* w1_alpha, const uint8_t* w2,
                         const uint8_t* w2_sf, const float* w2_alpha, int num_experts, int top_k,
                         int num_local_experts, int local_expert_offset, moe_quant_mode_t quant_mode,
                         uint16_t* out, int M, int H, int I, const moe_opts_t* opts, moe_stream_t stream);

/* moe_forward_noalloc: moe_forward for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments and results as moe_forward, but
 * the workspace is a fixed array inside the library: opts->workspace must
 * be NULL and opts->workspace_bytes 0 (else MOE_ERR_INVALID_ARGUMENT).
 * The array holds MOE_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the
 * library runs on, from the first call on that device until the process
 * ends; a pass whose moe_workspace_size() (at opts->tile, or
 * moe_default_tile) is larger returns MOE_ERR_SCRATCH_TOO_SMALL and enqueues
 * nothing.  The call allocates and frees nothing (its first call on a
 * device looks up the array's address there, a host-side query).  All calls
 * on one GPU share that GPU's array: two calls whose work overlaps on the
 * device (different streams, or host threads without ordering) race on it
 * and give undefined results; calls on one stream are ordered and safe. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_forward_noalloc(const void* x, const uint8_t* x_sf, const int32_t* topk_ids,
                                 const float* topk_weights, const uint8_t* w1, const uint8_t* w1_sf,
                                 const float* w1_alpha, const uint8_t* w2, const uint8_t* w2_sf,
                                 const float* w2_alpha, int num_experts, int top_k, int num_local_experts,
                                 int local_expert_offset, moe_quant_mode_t quant_mode, uint16_t* out, int M, int H,
                                 int I, const moe_opts_t* opts, moe_stream_t stream);

/* ---- Input preparation (model-load / activation quantisers) ----------- */

/* gscale[b] = amax(|x[b, :]|) / (6 * 448) for `batches` contiguous batches
 * of batch_elems bf16 values (the NVFP4 per-tensor or per-expert global
 * scale).  gscale: device fp32 [batches]. */
moe_status_t moe_nvfp4_global_scale(const uint16_t* x, int64_t batches, int64_t batch_elems, float* gscale,
                                    moe_stream_t stream);

/* moe_fc2_input_scale: the W4A4 calibration of fc2_input_scale
 * ("flashinfer.fused_moe.cute_dsl_fused_moe", Parameters fc2_input_scale:
 * the global scale of GEMM2's NVFP4 input).  Runs GEMM1 of the W4A4 mode on
 * the plan (the arguments as moe_grouped_gemm1_act, without y1) and writes
 *   *fc2_input_scale = max |y1| / (6 * 448)   (fp32, correctly rounded)
 * over every valid route and column, y1 taken after its bf16 rounding and
 * before any requantisation: the same formula as the NVFP4 global scale of
 * moe_nvfp4_global_scale.  fc2_input_scale is a device fp32 scalar; it is
 * also the pass's accumulator, so it must not be read until the pass ends.
 * Then w2_alpha of the W4A4 forward folds it in (see moe_quant_mode_t).
 * M = 0 gives 0. */
moe_status_t moe_fc2_input_scale(const void* x, const uint8_t* x_sf, int64_t x_row_stride, const moe_plan_t* plan,
                                 const uint8_t* w1, const uint8_t* w1_sf, const float* w1_alpha,
                                 const float* w1_alpha_up, int H, int I, int activation, float swiglu_alpha,
                                 float swiglu_beta, float swiglu_limit, float situ_beta, float situ_linear_beta,
                                 const float* per_token_scale, const float* fc1_bias, float* fc2_input_scale,
                                 moe_stream_t stream);

/* NVFP4 quantisation of bf16 [batches, rows, cols] (cols % 16 == 0), batch
 * b with global scale gscale[b] (device fp32): block scale
 * E4M3(blockamax / (6 * gscale)), codes E2M1(v / (decode(scale) * gscale)),
 * round-to-nearest-even, saturating, decided in fp32.  q packed
 * [batches, rows, cols/2], sf [batches, rows, cols/16]. */
moe_status_t moe_quantize_nvfp4(const uint16_t* x, int64_t batches, int64_t rows, int64_t cols,
                                const float* gscale, uint8_t* q, uint8_t* sf, moe_stream_t stream);

/* MX quantisation (OCP MX v1.0) of bf16 [rows, cols] (cols % 32 == 0):
 * E8M0 block-32 scale 2^(floor(log2 blockamax) - emax), elements
 * round-to-nearest-even and saturated.  elem 0: E4M3 (q [rows, cols]),
 * elem 1: E2M1 (q packed [rows, cols/2]); sf [rows, cols/32]. */
moe_status_t moe_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* sf,
                             moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
