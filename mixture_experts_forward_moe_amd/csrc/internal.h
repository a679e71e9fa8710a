// internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

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
  int H, I;
  float swiglu_alpha, swiglu_beta, swiglu_limit;
  const float* fc2_input_scale;
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
  int H, I;
  uint16_t* y2;
  const float* topk_weights;
  float routed_scaling_factor;
  uint16_t* out;
};
hipError_t launch_gemm1(const Gemm1Params& p, hipStream_t stream);
hipError_t launch_gemm2(const Gemm2Params& p, hipStream_t stream);

// finalize and fills
hipError_t launch_finalize(const uint16_t* y2, const int32_t* e2p, const float* w, int64_t M, int top_k, int H,
                           float rsf, int accumulate, uint16_t* out, hipStream_t stream);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

// input quantisers
hipError_t launch_nvfp4_global_scale(const uint16_t* x, int64_t batches, int64_t n, float* gs, hipStream_t stream);
hipError_t launch_quantize_nvfp4(const uint16_t* x, int64_t batches, int64_t rows, int64_t cols, const float* gs,
                                 uint8_t* q, uint8_t* sf, hipStream_t stream);
hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* sf,
                              hipStream_t stream);

}  // namespace moe
