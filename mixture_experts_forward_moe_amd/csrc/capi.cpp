// capi.cpp -- the C ABI (include/moe.h): host-side argument checks, plan
// carving, workspace sizing and the launch sequence of moe_forward.  Every
// check runs before anything is enqueued; nothing here allocates device
// memory or synchronises the host.
#include <float.h>
#include <cmath>
#include <hip/hip_runtime.h>
#include <string.h>

#include "internal.h"

using namespace moe;

namespace {

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

// Plan layout inside a workspace: e2p, p2e, tile_expert, tile_limit,
// num_tiles, offsets, counts, scratch -- each piece 256-byte aligned.
struct PlanLayout {
  size_t e2p, p2e, te, tl, nt, off, cnt, scratch, total;
  int64_t slots;
  int max_tiles, max_spans;
};

PlanLayout plan_layout(int M, int top_k, int El, int tile) {
  PlanLayout L;
  const int64_t R = (int64_t)M * top_k;
  L.slots = moe_route_slots(M, top_k, El, tile);
  L.max_tiles = (int)(L.slots / tile);
  L.max_spans = sort_max_spans(R);
  size_t o = 0;
  L.e2p = o; o = align256(o + sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
  L.p2e = o; o = align256(o + sizeof(int32_t) * (size_t)(L.slots > 0 ? L.slots : 1));
  L.te = o; o = align256(o + sizeof(int32_t) * (size_t)(L.max_tiles > 0 ? L.max_tiles : 1));
  L.tl = o; o = align256(o + sizeof(int32_t) * (size_t)(L.max_tiles > 0 ? L.max_tiles : 1));
  L.nt = o; o = align256(o + sizeof(int32_t));
  L.off = o; o = align256(o + sizeof(int32_t) * (size_t)(El + 1));
  L.cnt = o; o = align256(o + sizeof(int32_t) * (size_t)El);
  L.scratch = o; o = align256(o + sizeof(int32_t) * (size_t)L.max_spans * El);
  L.total = o;
  return L;
}

bool plan_args_ok(int M, int top_k, int El, int tile) {
  return M >= 0 && top_k >= 1 && top_k <= 64 && El >= 1 && El <= MAX_LOCAL_EXPERTS && pow2_in(tile, 16, 256);
}

moe_status_t dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

bool plan_ok(const moe_plan_t* p) {
  return p && p->expanded_to_permuted && p->permuted_to_expanded && p->tile_to_expert && p->tile_to_mn_limit &&
         p->num_tiles && p->expert_offsets && p->expert_counts && p->scratch &&
         plan_args_ok(p->M, p->top_k, p->num_local_experts, p->tile) &&
         p->route_slots == moe_route_slots(p->M, p->top_k, p->num_local_experts, p->tile);
}

bool mode_ok(int mode) { return mode == MOE_QUANT_W4A16 || mode == MOE_QUANT_W4A4 || mode == MOE_QUANT_MXFP8_MXFP4; }

// shapes the kernels take: H and I multiples of the scale block (16 for
// NVFP4, 32 for MX) are valid; the kernels need multiples of 32 (a packed
// 16-byte load of codes spans 32 elements), with partial tiles masked.  The
// non-gated ReLU^2 writes y1 columns [0, I/2) and [I/2, I) from separate row
// blocks, so with MXFP8 y1 blocks of 32 it needs I a multiple of 64.
moe_status_t shape_check(int H, int I, int mode, int activation = MOE_ACT_SWIGLU) {
  if (H <= 0 || I <= 0) return MOE_ERR_INVALID_ARGUMENT;
  const int blk = (mode == MOE_QUANT_MXFP8_MXFP4) ? 32 : 16;
  if (H % blk != 0 || I % blk != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 32 != 0 || I % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (activation == MOE_ACT_RELU2 && mode == MOE_QUANT_MXFP8_MXFP4 && I % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The FC1 activation's kernel arguments from the ABI's parameters (rules in
// moe.h, moe_grouped_gemm1_act).
moe_status_t make_act(int activation, float alpha, float beta, float limit, float situ_beta, float situ_lin,
                      GateAct* out) {
  if (activation != MOE_ACT_SWIGLU && activation != MOE_ACT_GEGLU_TANH && activation != MOE_ACT_RELU2)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!(limit > 0.0f)) return MOE_ERR_INVALID_ARGUMENT;
  if (!(situ_beta >= 0.0f) || !std::isfinite(situ_beta)) return MOE_ERR_INVALID_ARGUMENT;
  if (!(situ_lin >= 0.0f) || !std::isfinite(situ_lin)) return MOE_ERR_INVALID_ARGUMENT;
  if (situ_lin > 0.0f && !(situ_beta > 0.0f)) return MOE_ERR_INVALID_ARGUMENT;
  const bool swiglu_default = alpha == 1.0f && beta == 0.0f && limit == FLT_MAX;
  GateAct a = {ACT_SWIGLU, alpha, beta, limit, situ_beta, situ_lin};
  if (activation == MOE_ACT_GEGLU_TANH || activation == MOE_ACT_RELU2) {
    if (!swiglu_default || situ_beta > 0.0f) return MOE_ERR_INVALID_ARGUMENT;
    a.kind = activation == MOE_ACT_RELU2 ? ACT_RELU2 : ACT_GEGLU_TANH;
  } else if (situ_beta > 0.0f) {
    if (!swiglu_default) return MOE_ERR_INVALID_ARGUMENT;
    a.kind = ACT_SITU;
  }
  *out = a;
  return MOE_OK;
}

size_t y1_bytes(int mode, int64_t slots, int I) {
  if (mode == MOE_QUANT_W4A16) return (size_t)slots * I * 2;
  if (mode == MOE_QUANT_W4A4) return (size_t)slots * (I / 2);
  return (size_t)slots * I;
}
size_t y1_sf_bytes(int mode, int64_t slots, int I) {
  if (mode == MOE_QUANT_W4A16) return 0;
  if (mode == MOE_QUANT_W4A4) return (size_t)slots * (I / 16);
  return (size_t)slots * (I / 32);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or option (H and I must be multiples of 32, I of 64 for ReLU^2 "
                                     "in the MX mode; tile a power of two in [16, 256]; at most 512 local experts)";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_DEVICE: return "HIP launch failed";
    case MOE_ERR_SCRATCH_TOO_SMALL:
      return "the pass needs more workspace than the no-allocation scratch array holds (MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int64_t moe_route_slots(int M, int top_k, int num_local_experts, int tile) {
  if (M < 0 || top_k < 1 || num_local_experts < 1 || tile < 1) return 0;
  const int64_t R = (int64_t)M * top_k;
  const int64_t busy = R < num_local_experts ? R : num_local_experts;
  const int64_t need = R + busy * (tile - 1);
  return (need + tile - 1) / tile * tile;
}

size_t moe_plan_workspace_size(int M, int top_k, int num_local_experts, int tile) {
  if (!plan_args_ok(M, top_k, num_local_experts, tile)) return 0;
  return plan_layout(M, top_k, num_local_experts, tile).total;
}

moe_status_t moe_plan_init(moe_plan_t* plan, void* workspace, size_t workspace_bytes, int M, int top_k,
                           int num_local_experts, int tile) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  if (M < 0 || top_k < 1 || top_k > 64 || num_local_experts < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (num_local_experts > MAX_LOCAL_EXPERTS || !pow2_in(tile, 16, 256)) return MOE_ERR_UNSUPPORTED;
  PlanLayout L = plan_layout(M, top_k, num_local_experts, tile);
  if (!workspace || ((uintptr_t)workspace & 255) != 0 || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  uint8_t* b = (uint8_t*)workspace;
  plan->expanded_to_permuted = (int32_t*)(b + L.e2p);
  plan->permuted_to_expanded = (int32_t*)(b + L.p2e);
  plan->tile_to_expert = (int32_t*)(b + L.te);
  plan->tile_to_mn_limit = (int32_t*)(b + L.tl);
  plan->num_tiles = (int32_t*)(b + L.nt);
  plan->expert_offsets = (int32_t*)(b + L.off);
  plan->expert_counts = (int32_t*)(b + L.cnt);
  plan->scratch = (int32_t*)(b + L.scratch);
  plan->route_slots = L.slots;
  plan->max_tiles = L.max_tiles;
  plan->tile = tile;
  plan->M = M;
  plan->top_k = top_k;
  plan->num_local_experts = num_local_experts;
  plan->max_spans = L.max_spans;
  return MOE_OK;
}

moe_status_t moe_sort(const int32_t* topk_ids, int M, int top_k, int num_experts, int num_local_experts,
                      int local_expert_offset, moe_route_order_t route_order, const moe_plan_t* plan,
                      moe_stream_t stream) {
  if (!plan_ok(plan)) return MOE_ERR_INVALID_ARGUMENT;
  if (M != plan->M || top_k != plan->top_k || num_local_experts != plan->num_local_experts)
    return MOE_ERR_INVALID_ARGUMENT;
  if (M > 0 && !topk_ids) return MOE_ERR_INVALID_ARGUMENT;
  if (local_expert_offset < 0 || num_experts < 1 || (int64_t)local_expert_offset + num_local_experts > num_experts)
    return MOE_ERR_INVALID_ARGUMENT;
  if (route_order != MOE_ROUTE_ORDER_AUTO && route_order != MOE_ROUTE_ORDER_SINGLE &&
      route_order != MOE_ROUTE_ORDER_SPAN)
    return MOE_ERR_INVALID_ARGUMENT;
  return dev(launch_sort(topk_ids, M, top_k, local_expert_offset, route_order, plan, (hipStream_t)stream));
}

moe_status_t moe_grouped_gemm1_act(moe_quant_mode_t mode, const void* x, const uint8_t* x_sf,
                                   int64_t x_row_stride, const moe_plan_t* plan, const uint8_t* w1,
                                   const uint8_t* w1_sf, const float* w1_alpha, const float* w1_alpha_up, int H,
                                   int I, int activation, float swiglu_alpha, float swiglu_beta,
                                   float swiglu_limit, float situ_beta, float situ_linear_beta,
                                   const float* fc2_input_scale, const float* per_token_scale,
                                   const float* fc1_bias, void* y1, uint8_t* y1_sf, moe_stream_t stream) {
  if (!mode_ok(mode) || !plan_ok(plan)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t s = shape_check(H, I, mode, activation);
  if (s != MOE_OK) return s;
  if (!w1 || !w1_sf || !w1_alpha || !y1) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->M > 0 && !x) return MOE_ERR_INVALID_ARGUMENT;
  if ((mode == MOE_QUANT_W4A16) != (x_sf == NULL)) return MOE_ERR_INVALID_ARGUMENT;   // x_sf None iff w4a16
  if ((mode == MOE_QUANT_W4A4) != (fc2_input_scale != NULL)) return MOE_ERR_INVALID_ARGUMENT;
  if (per_token_scale && mode != MOE_QUANT_W4A4) return MOE_ERR_INVALID_ARGUMENT;
  if ((mode == MOE_QUANT_W4A16) != (y1_sf == NULL)) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t row_units = (mode == MOE_QUANT_W4A4) ? H / 2 : H;
  if (x_row_stride != 0 && x_row_stride < row_units) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t stride = x_row_stride ? x_row_stride : row_units;
  if ((stride * (mode == MOE_QUANT_W4A16 ? 2 : 1)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  Gemm1Params p = {};
  s = make_act(activation, swiglu_alpha, swiglu_beta, swiglu_limit, situ_beta, situ_linear_beta, &p.act);
  if (s != MOE_OK) return s;
  if (p.act.kind == ACT_RELU2 && w1_alpha_up) return MOE_ERR_INVALID_ARGUMENT;  // no up half
  p.mode = mode;
  p.x = x;
  p.x_sf = x_sf;
  p.x_row_stride = stride;
  p.plan = plan;
  p.w1 = w1;
  p.w1_sf = w1_sf;
  p.w1_alpha = w1_alpha;
  p.w1_alpha_up = w1_alpha_up;
  p.H = H;
  p.I = I;
  p.fc2_input_scale = fc2_input_scale;
  p.per_token_scale = per_token_scale;
  p.fc1_bias = fc1_bias;
  p.y1 = y1;
  p.y1_sf = y1_sf;
  if (plan->M == 0) return MOE_OK;
  return dev(launch_gemm1(p, (hipStream_t)stream));
}

moe_status_t moe_grouped_gemm1_swiglu(moe_quant_mode_t mode, const void* x, const uint8_t* x_sf,
                                      int64_t x_row_stride, const moe_plan_t* plan, const uint8_t* w1,
                                      const uint8_t* w1_sf, const float* w1_alpha, int H, int I,
                                      float swiglu_alpha, float swiglu_beta, float swiglu_limit,
                                      const float* fc2_input_scale, void* y1, uint8_t* y1_sf,
                                      moe_stream_t stream) {
  return moe_grouped_gemm1_act(mode, x, x_sf, x_row_stride, plan, w1, w1_sf, w1_alpha, NULL, H, I,
                               MOE_ACT_SWIGLU, swiglu_alpha, swiglu_beta, swiglu_limit, 0.0f, 0.0f,
                               fc2_input_scale, NULL, NULL, y1, y1_sf, stream);
}

moe_status_t moe_grouped_gemm2_bias(moe_quant_mode_t mode, const void* y1, const uint8_t* y1_sf,
                                    const moe_plan_t* plan, const uint8_t* w2, const uint8_t* w2_sf,
                                    const float* w2_alpha, const float* fc2_bias, int H, int I, uint16_t* y2,
                                    const float* topk_weights, float routed_scaling_factor, uint16_t* out,
                                    moe_stream_t stream) {
  if (!mode_ok(mode) || !plan_ok(plan)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t s = shape_check(H, I, mode);
  if (s != MOE_OK) return s;
  if (!y1 || !w2 || !w2_sf || !w2_alpha) return MOE_ERR_INVALID_ARGUMENT;
  if ((mode == MOE_QUANT_W4A16) != (y1_sf == NULL)) return MOE_ERR_INVALID_ARGUMENT;
  if ((y2 == NULL) == (out == NULL)) return MOE_ERR_INVALID_ARGUMENT;  // exactly one finalize mode
  if (out && !topk_weights) return MOE_ERR_INVALID_ARGUMENT;
  // packed-bf16 atomics into out; 16-byte stores of y2 rows
  if ((out && ((uintptr_t)out & 3) != 0) || (y2 && ((uintptr_t)y2 & 15) != 0)) return MOE_ERR_UNSUPPORTED;
  Gemm2Params p = {};
  p.mode = mode;
  p.y1 = y1;
  p.y1_sf = y1_sf;
  p.plan = plan;
  p.w2 = w2;
  p.w2_sf = w2_sf;
  p.w2_alpha = w2_alpha;
  p.fc2_bias = fc2_bias;
  p.H = H;
  p.I = I;
  p.y2 = y2;
  p.topk_weights = topk_weights;
  p.routed_scaling_factor = routed_scaling_factor;
  p.out = out;
  if (plan->M == 0) return MOE_OK;
  return dev(launch_gemm2(p, (hipStream_t)stream));
}

moe_status_t moe_grouped_gemm2(moe_quant_mode_t mode, const void* y1, const uint8_t* y1_sf,
                               const moe_plan_t* plan, const uint8_t* w2, const uint8_t* w2_sf,
                               const float* w2_alpha, int H, int I, uint16_t* y2, const float* topk_weights,
                               float routed_scaling_factor, uint16_t* out, moe_stream_t stream) {
  return moe_grouped_gemm2_bias(mode, y1, y1_sf, plan, w2, w2_sf, w2_alpha, NULL, H, I, y2, topk_weights,
                                routed_scaling_factor, out, stream);
}

moe_status_t moe_finalize(const uint16_t* y2, const moe_plan_t* plan, const float* topk_weights, int H,
                          float routed_scaling_factor, int accumulate, uint16_t* out, moe_stream_t stream) {
  if (!plan_ok(plan) || H <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (plan->M > 0 && (!y2 || !topk_weights || !out)) return MOE_ERR_INVALID_ARGUMENT;
  if (plan->M == 0) return MOE_OK;
  if (((uintptr_t)y2 & 15) != 0 || ((uintptr_t)out & 15) != 0) return MOE_ERR_UNSUPPORTED;  // 16-byte accesses
  return dev(launch_finalize(y2, plan->expanded_to_permuted, topk_weights, plan->M, plan->top_k, H,
                             routed_scaling_factor, accumulate ? 1 : 0, out, (hipStream_t)stream));
}

void moe_opts_init(moe_opts_t* o) {
  if (!o) return;
  memset(o, 0, sizeof(*o));
  o->swiglu_alpha = 1.0f;
  o->swiglu_beta = 0.0f;
  o->swiglu_limit = FLT_MAX;
  o->fc2_input_scale = NULL;
  o->routed_scaling_factor = 1.0f;
  o->accumulate = 0;
  o->finalize_mode = MOE_FINALIZE_DETERMINISTIC;
  o->route_order = MOE_ROUTE_ORDER_AUTO;
  o->tile = 0;
  o->x_row_stride = 0;
  o->path = MOE_PATH_AUTO;
}

int moe_default_tile(int M, int top_k, int num_experts, int num_local_experts, moe_quant_mode_t mode) {
  // routes per local expert, expected: of the M * top_k routes, those that
  // land on this GPU's num_local_experts of num_experts
  const int El = num_local_experts > 0 ? num_local_experts : 1;
  const int E = num_experts > El ? num_experts : El;
  const double per_expert = (double)M * top_k / E;
  if (per_expert <= 16) return 16;
  // W4A16: the expert-streaming kernel (32-row passes) while one pass covers
  // an expert, the wide-tile kernel beyond
  if (mode == MOE_QUANT_W4A16) return per_expert <= 32 ? 32 : 128;
  // W4A4: the expert-streaming kernel at every larger size (it stays ahead
  // of the 128-slot tiles at least to 256 routes per expert)
  if (mode == MOE_QUANT_W4A4) return per_expert <= 48 ? 32 : 64;
  if (per_expert <= 48) return 32;
  if (per_expert <= 96) return 64;
  // the MX mode's large-batch kernel works on 256-slot tiles (the tile of
  // the large-batch benchmark of pull request 4440)
  if (per_expert > 384) return 256;
  return 128;
}

size_t moe_workspace_size(int M, int H, int I, int top_k, int num_local_experts, int tile, moe_quant_mode_t mode,
                          int finalize_mode) {
  if (!plan_args_ok(M, top_k, num_local_experts, tile) || !mode_ok(mode) || H <= 0 || I <= 0) return 0;
  PlanLayout L = plan_layout(M, top_k, num_local_experts, tile);
  // the decode path's counter block first, then the plan (moe_forward_plan)
  size_t total = DEC_COUNTER_BYTES + L.total;
  total = align256(total + y1_bytes(mode, L.slots, I));
  total = align256(total + y1_sf_bytes(mode, L.slots, I));
  const bool dec = tile == 16 && decode_supported(mode, M, top_k, num_local_experts, H, I);
  if (finalize_mode == MOE_FINALIZE_DETERMINISTIC || dec) total = align256(total + (size_t)L.slots * H * 2);
  return total;
}

moe_status_t moe_forward_plan(moe_plan_t* plan, void* workspace, size_t workspace_bytes, int M, int top_k,
                              int num_local_experts, int tile) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < DEC_COUNTER_BYTES) return MOE_ERR_WORKSPACE;
  return moe_plan_init(plan, (uint8_t*)workspace + DEC_COUNTER_BYTES, workspace_bytes - DEC_COUNTER_BYTES, M, top_k,
                       num_local_experts, tile);
}

namespace {
struct MarkCtx {
  hipEvent_t* ev;
  hipStream_t st;
  hipError_t err;
};
void mark_phase(void* ctx, int i) {
  MarkCtx* c = (MarkCtx*)ctx;
  if (c->ev && c->ev[i] && c->err == hipSuccess) c->err = hipEventRecord(c->ev[i], c->st);
}
}  // namespace

moe_status_t moe_forward(const void* x, const uint8_t* x_sf, const int32_t* topk_ids, const float* topk_weights,
                         const uint8_t* w1, const uint8_t* w1_sf, const float* w1_alpha, const uint8_t* w2,
                         const uint8_t* w2_sf, const float* w2_alpha, int num_experts, int top_k,
                         int num_local_experts, int local_expert_offset, moe_quant_mode_t quant_mode,
                         uint16_t* out, int M, int H, int I, const moe_opts_t* opts, moe_stream_t stream) {
  if (!opts || !mode_ok(quant_mode)) return MOE_ERR_INVALID_ARGUMENT;
  if (M < 0 || top_k < 1 || top_k > 64 || num_local_experts < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (local_expert_offset < 0 || (int64_t)local_expert_offset + num_local_experts > num_experts)
    return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t s = shape_check(H, I, quant_mode, opts->activation);
  if (s != MOE_OK) return s;
  if (opts->finalize_mode != MOE_FINALIZE_DETERMINISTIC && opts->finalize_mode != MOE_FINALIZE_ATOMIC)
    return MOE_ERR_INVALID_ARGUMENT;
  if (opts->path != MOE_PATH_AUTO && opts->path != MOE_PATH_DECODE && opts->path != MOE_PATH_TILED)
    return MOE_ERR_INVALID_ARGUMENT;
  if (M > 0 && (!x || !topk_ids || !topk_weights || !out)) return MOE_ERR_INVALID_ARGUMENT;
  if (M > 0 && ((uintptr_t)out & 15) != 0) return MOE_ERR_UNSUPPORTED;  // 16-byte accesses and bf16-pair atomics
  if (!w1 || !w1_sf || !w1_alpha || !w2 || !w2_sf || !w2_alpha) return MOE_ERR_INVALID_ARGUMENT;
  if ((quant_mode == MOE_QUANT_W4A16) != (x_sf == NULL)) return MOE_ERR_INVALID_ARGUMENT;
  if ((quant_mode == MOE_QUANT_W4A4) != (opts->fc2_input_scale != NULL)) return MOE_ERR_INVALID_ARGUMENT;
  if (opts->per_token_scale && quant_mode != MOE_QUANT_W4A4) return MOE_ERR_INVALID_ARGUMENT;
  if (num_local_experts > MAX_LOCAL_EXPERTS) return MOE_ERR_UNSUPPORTED;
  GateAct act;
  s = make_act(opts->activation, opts->swiglu_alpha, opts->swiglu_beta, opts->swiglu_limit, opts->situ_beta,
               opts->situ_linear_beta, &act);
  if (s != MOE_OK) return s;
  if (act.kind == ACT_RELU2 && opts->w1_alpha_up) return MOE_ERR_INVALID_ARGUMENT;  // no up half
  const int tile = opts->tile ? opts->tile : moe_default_tile(M, top_k, num_experts, num_local_experts, quant_mode);
  if (!pow2_in(tile, 16, 256)) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_workspace_size(M, H, I, top_k, num_local_experts, tile, quant_mode, opts->finalize_mode);
  if (!opts->workspace || opts->workspace_bytes < need || ((uintptr_t)opts->workspace & 255) != 0)
    return MOE_ERR_WORKSPACE;

  moe_plan_t plan;
  PlanLayout L = plan_layout(M, top_k, num_local_experts, tile);
  int* counters = (int*)opts->workspace;
  s = moe_forward_plan(&plan, opts->workspace, opts->workspace_bytes, M, top_k, num_local_experts, tile);
  if (s != MOE_OK) return s;
  uint8_t* base = (uint8_t*)opts->workspace + DEC_COUNTER_BYTES + L.total;
  void* y1 = base;
  base += align256(y1_bytes(quant_mode, L.slots, I));
  uint8_t* y1_sf = (quant_mode == MOE_QUANT_W4A16) ? NULL : base;
  base += align256(y1_sf_bytes(quant_mode, L.slots, I));
  // (the decode kernels read scale pairs as aligned 32-bit words)
  // the decode path streams each expert's weights once per route row: by
  // default it is taken only while the batch is expected to give a local
  // expert at most 1.25 routes
  const bool dec_wanted = opts->path == MOE_PATH_DECODE ||
                          (opts->path == MOE_PATH_AUTO && 4 * (int64_t)M * top_k <= 5 * (int64_t)num_experts);
  const bool dec = dec_wanted && tile == 16 && decode_supported(quant_mode, M, top_k, num_local_experts, H, I) &&
                   opts->x_row_stride % 8 == 0 && ((uintptr_t)w1_sf & 3) == 0 && ((uintptr_t)w2_sf & 3) == 0;
  uint16_t* y2 = (opts->finalize_mode == MOE_FINALIZE_DETERMINISTIC || dec) ? (uint16_t*)base : NULL;

  hipStream_t st = (hipStream_t)stream;
  hipEvent_t* ev = (hipEvent_t*)opts->phase_events;
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], st) : hipSuccess; };
  if (mark(0) != hipSuccess) return MOE_ERR_DEVICE;
  if (M == 0) {
    if (!opts->accumulate && out) { /* nothing to write: M == 0 */ }
    for (int i = 1; i < MOE_NUM_PHASE_EVENTS; i++)
      if (mark(i) != hipSuccess) return MOE_ERR_DEVICE;
    return MOE_OK;
  }
  if (dec) {
    // decode-sized batch: GEMM1 (with the routing plan), then GEMM2 with the finalize
    DecodeParams d = {};
    d.topk_ids = topk_ids;
    d.local_expert_offset = local_expert_offset;
    d.x = x;
    d.x_row_stride = opts->x_row_stride ? opts->x_row_stride : H;
    d.w1 = w1;
    d.w1_sf = w1_sf;
    d.w1_alpha = w1_alpha;
    d.w1_alpha_up = opts->w1_alpha_up;
    d.fc1_bias = opts->fc1_bias;
    d.fc2_bias = opts->fc2_bias;
    d.w2 = w2;
    d.w2_sf = w2_sf;
    d.w2_alpha = w2_alpha;
    d.H = H;
    d.I = I;
    d.act = act;
    d.y1 = (uint16_t*)y1;
    d.y2 = y2;
    d.counters = counters;
    d.topk_weights = topk_weights;
    d.routed_scaling_factor = opts->routed_scaling_factor;
    d.accumulate = opts->accumulate;
    d.atomic = opts->finalize_mode == MOE_FINALIZE_ATOMIC;
    d.out = out;
    d.plan = &plan;
    MarkCtx mc = {ev, st, hipSuccess};
    d.mark = mark_phase;
    d.mark_ctx = &mc;
    if (launch_decode(d, st) != hipSuccess || mc.err != hipSuccess) return MOE_ERR_DEVICE;
    if (mark(4) != hipSuccess) return MOE_ERR_DEVICE;
    return MOE_OK;
  }
  s = moe_sort(topk_ids, M, top_k, num_experts, num_local_experts, local_expert_offset,
               (moe_route_order_t)opts->route_order, &plan, stream);
  if (s != MOE_OK) return s;
  if (mark(1) != hipSuccess) return MOE_ERR_DEVICE;
  if (opts->finalize_mode == MOE_FINALIZE_ATOMIC && !opts->accumulate) {
    if (launch_zero_fill(out, (size_t)M * H * 2, st) != hipSuccess) return MOE_ERR_DEVICE;
  }
  s = moe_grouped_gemm1_act(quant_mode, x, x_sf, opts->x_row_stride, &plan, w1, w1_sf, w1_alpha,
                            opts->w1_alpha_up, H, I, opts->activation, opts->swiglu_alpha, opts->swiglu_beta,
                            opts->swiglu_limit, opts->situ_beta, opts->situ_linear_beta, opts->fc2_input_scale,
                            opts->per_token_scale, opts->fc1_bias, y1, y1_sf, stream);
  if (s != MOE_OK) return s;
  if (mark(2) != hipSuccess) return MOE_ERR_DEVICE;
  if (opts->finalize_mode == MOE_FINALIZE_DETERMINISTIC) {
    s = moe_grouped_gemm2_bias(quant_mode, y1, y1_sf, &plan, w2, w2_sf, w2_alpha, opts->fc2_bias, H, I, y2,
                               NULL, opts->routed_scaling_factor, NULL, stream);
    if (s != MOE_OK) return s;
    if (mark(3) != hipSuccess) return MOE_ERR_DEVICE;
    s = moe_finalize(y2, &plan, topk_weights, H, opts->routed_scaling_factor, opts->accumulate, out, stream);
    if (s != MOE_OK) return s;
  } else {
    s = moe_grouped_gemm2_bias(quant_mode, y1, y1_sf, &plan, w2, w2_sf, w2_alpha, opts->fc2_bias, H, I, NULL,
                               topk_weights, opts->routed_scaling_factor, out, stream);
    if (s != MOE_OK) return s;
    if (mark(3) != hipSuccess) return MOE_ERR_DEVICE;
  }
  if (mark(4) != hipSuccess) return MOE_ERR_DEVICE;
  return MOE_OK;
}

moe_status_t moe_fc2_input_scale(const void* x, const uint8_t* x_sf, int64_t x_row_stride, const moe_plan_t* plan,
                                 const uint8_t* w1, const uint8_t* w1_sf, const float* w1_alpha,
                                 const float* w1_alpha_up, int H, int I, int activation, float swiglu_alpha,
                                 float swiglu_beta, float swiglu_limit, float situ_beta, float situ_linear_beta,
                                 const float* per_token_scale, const float* fc1_bias, float* fc2_input_scale,
                                 moe_stream_t stream) {
  if (!plan_ok(plan) || !fc2_input_scale) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t s = shape_check(H, I, MOE_QUANT_W4A4, activation);
  if (s != MOE_OK) return s;
  if (!w1 || !w1_sf || !w1_alpha || !x_sf || (plan->M > 0 && !x)) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t row_units = H / 2;
  if (x_row_stride != 0 && x_row_stride < row_units) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t stride = x_row_stride ? x_row_stride : row_units;
  if (stride % 16 != 0) return MOE_ERR_UNSUPPORTED;
  Gemm1Params p = {};
  s = make_act(activation, swiglu_alpha, swiglu_beta, swiglu_limit, situ_beta, situ_linear_beta, &p.act);
  if (s != MOE_OK) return s;
  if (p.act.kind == ACT_RELU2 && w1_alpha_up) return MOE_ERR_INVALID_ARGUMENT;
  p.mode = MOE_QUANT_W4A4;
  p.x = x;
  p.x_sf = x_sf;
  p.x_row_stride = stride;
  p.plan = plan;
  p.w1 = w1;
  p.w1_sf = w1_sf;
  p.w1_alpha = w1_alpha;
  p.w1_alpha_up = w1_alpha_up;
  p.H = H;
  p.I = I;
  p.per_token_scale = per_token_scale;
  p.fc1_bias = fc1_bias;
  hipStream_t st = (hipStream_t)stream;
  unsigned* bits = reinterpret_cast<unsigned*>(fc2_input_scale);
  if (launch_zero_fill(bits, sizeof(float), st) != hipSuccess) return MOE_ERR_DEVICE;
  if (plan->M > 0 && launch_gemm1_amax(p, bits, st) != hipSuccess) return MOE_ERR_DEVICE;
  return dev(launch_gscale_finish(fc2_input_scale, 1, st));
}

moe_status_t moe_nvfp4_global_scale(const uint16_t* x, int64_t batches, int64_t batch_elems, float* gscale,
                                    moe_stream_t stream) {
  if (batches < 0 || batch_elems < 0 || (batches > 0 && (!x || !gscale))) return MOE_ERR_INVALID_ARGUMENT;
  if (batch_elems % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (batches == 0) return MOE_OK;
  return dev(launch_nvfp4_global_scale(x, batches, batch_elems, gscale, (hipStream_t)stream));
}

moe_status_t moe_quantize_nvfp4(const uint16_t* x, int64_t batches, int64_t rows, int64_t cols,
                                const float* gscale, uint8_t* q, uint8_t* sf, moe_stream_t stream) {
  if (batches < 0 || rows < 0 || cols < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (cols % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (batches * rows * cols > 0 && (!x || !gscale || !q || !sf)) return MOE_ERR_INVALID_ARGUMENT;
  return dev(launch_quantize_nvfp4(x, batches, rows, cols, gscale, q, sf, (hipStream_t)stream));
}

moe_status_t moe_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* sf,
                             moe_stream_t stream) {
  if (rows < 0 || cols < 0 || (elem != 0 && elem != 1)) return MOE_ERR_INVALID_ARGUMENT;
  if (cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows * cols > 0 && (!x || !q || !sf)) return MOE_ERR_INVALID_ARGUMENT;
  return dev(launch_quantize_mx(x, rows, cols, elem, q, sf, (hipStream_t)stream));
}

}  // extern "C"
