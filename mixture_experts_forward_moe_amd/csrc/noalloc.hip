// noalloc.hip -- moe_forward_noalloc: the whole forward pass with its
// workspace in a fixed device array of this library instead of a caller
// buffer, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never uses the array's name as a device address (on the host it is only a
// stand-in symbol); the address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept per device.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include "internal.h"

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_lock;
void* g_scratch[MAX_DEVICES];  // device address of `scratch` on each device, once known

// the scratch array's device address on the current device (NULL on error)
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" moe_status_t moe_forward_noalloc(const void* x, const uint8_t* x_sf, const int32_t* topk_ids,
                                            const float* topk_weights, const uint8_t* w1, const uint8_t* w1_sf,
                                            const float* w1_alpha, const uint8_t* w2, const uint8_t* w2_sf,
                                            const float* w2_alpha, int num_experts, int top_k,
                                            int num_local_experts, int local_expert_offset,
                                            moe_quant_mode_t quant_mode, uint16_t* out, int M, int H, int I,
                                            const moe_opts_t* opts, moe_stream_t stream) {
  if (!opts || opts->workspace || opts->workspace_bytes) return MOE_ERR_INVALID_ARGUMENT;
  if (M < 0 || top_k < 1 || top_k > 64 || num_local_experts < 1) return MOE_ERR_INVALID_ARGUMENT;
  const int tile = opts->tile ? opts->tile : moe_default_tile(M, top_k, num_experts, num_local_experts, quant_mode);
  const size_t need = moe_workspace_size(M, H, I, top_k, num_local_experts, tile, quant_mode, opts->finalize_mode);
  if (need == 0) return MOE_ERR_INVALID_ARGUMENT;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_TOO_SMALL;
  void* ws = scratch_address();
  if (!ws) return MOE_ERR_DEVICE;
  moe_opts_t o;
  memcpy(&o, opts, sizeof(o));
  o.tile = tile;
  o.workspace = ws;
  o.workspace_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  return moe_forward(x, x_sf, topk_ids, topk_weights, w1, w1_sf, w1_alpha, w2, w2_sf, w2_alpha, num_experts, top_k,
                     num_local_experts, local_expert_offset, quant_mode, out, M, H, I, &o, stream);
}
