// internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"
#include "device_common.h"

namespace moe {

// routing plan
constexpr int SORT_SINGLE_MAX_ROUTES = 8192;  // AUTO: one workgroup up to this many routes
constexpr int SORT_SPAN_MIN = 2048;           // routes per span at least
constexpr int SORT_MAX_SPANS = 1024;
constexpr int MAX_LOCAL_EXPERTS = 512;
int sort_max_spans(int64_t routes);
hipError_t launch_sort(const int32_t* ids, int M, int top_k, int offset, int route_order, const moe_plan_t* plan,
                       hipStream_t stream);

// grouped GEMMs
struct Gemm1Params {
  int mode;
  const void* x;
  const uint8_t* x_sf;
  int64_t x_row_stride;
  const moe_plan_t* plan;
  const uint8_t* w1;
  const uint8_t* w1_sf;
  const float* w1_alpha;
  const float* w1_alpha_up;      // NULL: w1_alpha for the up half too
  int H, I;
  GateAct act;
  const float* fc2_input_scale;
  const float* per_token_scale;  // W4A4 only; NULL: none
  const float* fc1_bias;         // NULL, or fp32 [E_l, 2I]
  void* y1;
  uint8_t* y1_sf;
};
struct Gemm2Params {
  int mode;
  const void* y1;
  const uint8_t* y1_sf;
  const moe_plan_t* plan;
  const uint8_t* w2;
  const uint8_t* w2_sf;
  const float* w2_alpha;
  const float* fc2_bias;  // NULL, or fp32 [E_l, H]
  int H, I;
  uint16_t* y2;
  const float* topk_weights;
  float routed_scaling_factor;
  uint16_t* out;
};
hipError_t launch_gemm1(const Gemm1Params& p, hipStream_t stream);
// W1 row pairs per expert that GEMM1 walks: gate / up pairs (I), or for the
// non-gated ReLU^2 rows j and I/2 + j of its I rows, whose outputs are
// y1 columns j and I/2 + j
inline int gemm1_pairs(const Gemm1Params& p) { return p.act.kind == ACT_RELU2 ? p.I / 2 : p.I; }
hipError_t launch_gemm2(const Gemm2Params& p, hipStream_t stream);
// GEMM1 without a store: atomically maxes the fp32 bits of |y1| (after its
// bf16 rounding) over every valid route and column into *amax
hipError_t launch_gemm1_amax(const Gemm1Params& p, unsigned* amax, hipStream_t stream);

// wide-tile kernels for 128-slot tiles (prefill-sized batches, W4A16 / W4A4)
bool wide_supported1(const Gemm1Params& p);
bool wide_supported2(const Gemm2Params& p);
hipError_t launch_gemm1_wide(const Gemm1Params& p, hipStream_t stream);
hipError_t launch_gemm2_wide(const Gemm2Params& p, hipStream_t stream);

// MXFP8 x MXFP4 on 128-slot tiles (prefill-sized batches)
bool mx_supported1(const Gemm1Params& p);
bool mx_supported2(const Gemm2Params& p);
hipError_t launch_gemm1_mx(const Gemm1Params& p, hipStream_t stream);
hipError_t launch_gemm2_mx(const Gemm2Params& p, hipStream_t stream);

// MXFP8 x MXFP4 on 256-slot tiles (large batches): LDS-DMA staged, 256 x 256 per workgroup
bool mxw_supported1(const Gemm1Params& p);
bool mxw_supported2(const Gemm2Params& p);
hipError_t launch_gemm1_mxw(const Gemm1Params& p, hipStream_t stream);
hipError_t launch_gemm2_mxw(const Gemm2Params& p, hipStream_t stream);

// NVFP4 x NVFP4 (W4A4) at plan tiles up to 64: one workgroup per (expert,
// 256 weight rows) streams the weights once for all of the expert's routes
bool nv_supported1(const Gemm1Params& p);
bool nv_supported2(const Gemm2Params& p);
hipError_t launch_gemm1_nv(const Gemm1Params& p, hipStream_t stream);
hipError_t launch_gemm1_nv_amax(const Gemm1Params& p, unsigned* amax, hipStream_t stream);
hipError_t launch_gemm2_nv(const Gemm2Params& p, hipStream_t stream);

// the two-launch W4A16 forward for decode-sized batches (plan tile 16)
struct DecodeParams {
  const int32_t* topk_ids;
  int local_expert_offset;
  const void* x;
  int64_t x_row_stride;  // elements
  const uint8_t *w1, *w1_sf;
  const float* w1_alpha;
  const float* w1_alpha_up;  // NULL: w1_alpha for the up half too
  const float* fc1_bias;     // NULL, or fp32 [E_l, 2I]
  const float* fc2_bias;     // NULL, or fp32 [E_l, H]
  const uint8_t *w2, *w2_sf;
  const float* w2_alpha;
  int H, I;
  GateAct act;
  uint16_t* y1;
  uint16_t* y2;
  int* counters;  // the decode counter block (DEC_COUNTER_BYTES); GEMM1 clears it for GEMM2
  const float* topk_weights;
  float routed_scaling_factor;
  int accumulate;
  int atomic;     // finalize: 0 deterministic (route order, in GEMM2's last workgroups), 1 packed-bf16 atomics
  uint16_t* out;
  const moe_plan_t* plan;
  void (*mark)(void* ctx, int phase);  // optional: called between the launches
  void* mark_ctx;
};
// Decode path limits.  Its counter block sits at the head of the forward
// workspace: one done count per 64 columns of H, each in a 256-byte slot of
// its own (atomics on one line queue at the memory side).  GEMM1 clears the
// counts GEMM2 will use, so the block needs no initial contents.
constexpr int DEC_MAX_ROUTES = 1024;
constexpr int DEC_MAX_COL_GROUPS = 1024;  // H <= 65536
constexpr int DEC_CTR_SLOT = 64;          // ints per counter slot
constexpr size_t DEC_COUNTER_BYTES = sizeof(int) * DEC_CTR_SLOT * DEC_MAX_COL_GROUPS;
bool decode_supported(int mode, int M, int top_k, int El, int H, int I);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// finalize and fills
hipError_t launch_finalize(const uint16_t* y2, const int32_t* e2p, const float* w, int64_t M, int top_k, int H,
                           float rsf, int accumulate, uint16_t* out, hipStream_t stream);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

// input quantisers
hipError_t launch_nvfp4_global_scale(const uint16_t* x, int64_t batches, int64_t n, float* gs, hipStream_t stream);
// gs[b] = (fp32 bits in gs[b]) / (6 * 448), correctly rounded
hipError_t launch_gscale_finish(float* gs, int64_t batches, hipStream_t stream);
hipError_t launch_quantize_nvfp4(const uint16_t* x, int64_t batches, int64_t rows, int64_t cols, const float* gs,
                                 uint8_t* q, uint8_t* sf, hipStream_t stream);
hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* sf,
                              hipStream_t stream);

}  // namespace moe
