// finalize.hip -- the deterministic weighted top-k finalize, a zero fill, and
// the NVFP4 / MX input quantisers.
//
// Finalize ("flashinfer.fused_moe.alphamoe_nvfp4_routed_moe", summary:
// contributions finalized in route order, seeded from the caller's output;
// Parameters: accumulate, routed_scaling_factor):
//   acc = accumulate ? out : 0;  acc = acc + fp32(w * rsf) * y2[slot]  (j ascending)
//   out = bf16(acc)
// Each thread owns 8 consecutive columns of one token and reads its top_k
// slot rows with 16-byte loads: one pass over y2, HBM-bound.
#include "device_common.h"
#include "internal.h"

// The finalize's multiplies and adds are separate roundings (no fused
// multiply-add), as the route-order reduction states them.
#pragma clang fp contract(off)

namespace moe {

constexpr int FIN_THREADS = 256;

__global__ __launch_bounds__(FIN_THREADS) void finalize_kernel(const uint16_t* __restrict__ y2,
                                                               const int32_t* __restrict__ e2p,
                                                               const float* __restrict__ w, int top_k, int H,
                                                               float rsf, int accumulate, uint16_t* __restrict__ out,
                                                               int blocks_per_token) {
  const int64_t t = blockIdx.x / blocks_per_token;
  const int h0 = ((blockIdx.x % blocks_per_token) * FIN_THREADS + threadIdx.x) * 8;
  if (h0 >= H) return;
  float acc[8];
  uint16_t* o = out + t * H + h0;
  if (accumulate) {
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(o);
    for (int i = 0; i < 4; i++) {
      acc[2 * i] = __uint_as_float(v[i] << 16);
      acc[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
    for (int i = 0; i < 8; i++) acc[i] = 0.0f;
  }
  for (int j = 0; j < top_k; j++) {
    const int32_t s = e2p[t * top_k + j];
    if (s < 0) continue;
    const float wf = w[t * top_k + j] * rsf;
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(y2 + (int64_t)s * H + h0);
    for (int i = 0; i < 4; i++) {
      acc[2 * i] = acc[2 * i] + wf * __uint_as_float(v[i] << 16);
      acc[2 * i + 1] = acc[2 * i + 1] + wf * __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  u32x4_t r;
  for (int i = 0; i < 4; i++) r[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<u32x4_t*>(o) = r;
}

hipError_t launch_finalize(const uint16_t* y2, const int32_t* e2p, const float* w, int64_t M, int top_k, int H,
                           float rsf, int accumulate, uint16_t* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int bpt = (H / 8 + FIN_THREADS - 1) / FIN_THREADS;
  finalize_kernel<<<(unsigned)(M * bpt), FIN_THREADS, 0, stream>>>(y2, e2p, w, top_k, H, rsf, accumulate, out, bpt);
  return hipGetLastError();
}

// ---------------------------------------------------------------- fills

__global__ void zero_fill_kernel(u32x4_t* p, int64_t n16, uint8_t* tail, int64_t ntail) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < n16; k += stride) p[k] = u32x4_t{0u, 0u, 0u, 0u};
  if (i < ntail) tail[i] = 0;
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  int64_t n16 = (int64_t)(bytes / 16);
  int64_t ntail = (int64_t)(bytes % 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  zero_fill_kernel<<<(unsigned)blocks, 256, 0, stream>>>((u32x4_t*)p, n16, (uint8_t*)p + n16 * 16, ntail);
  return hipGetLastError();
}

// ---------------------------------------------------------------- quantisers

// gs[b] holds the fp32 bits of the running amax (non-negative floats order
// like their bit patterns), then becomes amax / (6 * 448).
__global__ void amax_kernel(const uint16_t* __restrict__ x, int64_t n, int blocks_per_batch, unsigned* gs_bits) {
  const int b = blockIdx.x / blocks_per_batch;
  const int part = blockIdx.x % blocks_per_batch;
  const uint16_t* xb = x + (int64_t)b * n;
  float m = 0.0f;
  for (int64_t i = ((int64_t)part * blockDim.x + threadIdx.x) * 8; i < n; i += (int64_t)blocks_per_batch * blockDim.x * 8) {
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(xb + i);
    for (int k = 0; k < 4; k++) {
      m = fmaxf(m, fabsf(__uint_as_float(v[k] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(v[k] & 0xffff0000u)));
    }
  }
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  __shared__ float wm[16];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.0f;
    for (int w = 0; w < (int)(blockDim.x >> 6); w++) r = fmaxf(r, wm[w]);
    atomicMax(gs_bits + b, __float_as_uint(r));
  }
}

__global__ void gscale_finish_kernel(float* gs, int64_t batches) {
  int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batches) gs[b] = __fdiv_rn(gs[b], 2688.0f);
}

hipError_t launch_gscale_finish(float* gs, int64_t batches, hipStream_t stream) {
  gscale_finish_kernel<<<(unsigned)((batches + 255) / 256), 256, 0, stream>>>(gs, batches);
  return hipGetLastError();
}

hipError_t launch_nvfp4_global_scale(const uint16_t* x, int64_t batches, int64_t n, float* gs, hipStream_t stream) {
  hipError_t e = launch_zero_fill(gs, sizeof(float) * batches, stream);
  if (e != hipSuccess) return e;
  int64_t bpb = (n / 8 + 255) / 256;
  if (bpb > 64) bpb = 64;
  if (bpb < 1) bpb = 1;
  amax_kernel<<<(unsigned)(batches * bpb), 256, 0, stream>>>(x, n, (int)bpb, (unsigned*)gs);
  gscale_finish_kernel<<<(unsigned)((batches + 255) / 256), 256, 0, stream>>>(gs, batches);
  return hipGetLastError();
}

// one thread per 16-element block
__global__ void quantize_nvfp4_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                      const float* __restrict__ gs, uint8_t* __restrict__ q,
                                      uint8_t* __restrict__ sf, int64_t total_blocks) {
  int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= total_blocks) return;
  const int64_t nb = cols / 16;
  const int64_t row = blk / nb;  // row over all batches
  const int64_t batch = row / rows;
  const float g = gs[batch];
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + blk * 16);
  u32x4_t a = src[0], b = src[1];
  float v[16];
  for (int k = 0; k < 4; k++) {
    v[2 * k] = __uint_as_float(a[k] << 16);
    v[2 * k + 1] = __uint_as_float(a[k] & 0xffff0000u);
    v[8 + 2 * k] = __uint_as_float(b[k] << 16);
    v[8 + 2 * k + 1] = __uint_as_float(b[k] & 0xffff0000u);
  }
  float m = 0.0f;
  for (int i = 0; i < 16; i++) m = fmaxf(m, fabsf(v[i]));
  uint32_t sc = nvfp4_scale_code(m, g);
  float sd = e4m3_to_f32(sc);
  uint32_t lo = 0, hi = 0;
  for (int i = 0; i < 8; i++) lo |= nvfp4_elem_code(v[i], sd, g) << (4 * i);
  for (int i = 0; i < 8; i++) hi |= nvfp4_elem_code(v[8 + i], sd, g) << (4 * i);
  reinterpret_cast<uint2*>(q)[blk] = make_uint2(lo, hi);
  sf[blk] = (uint8_t)sc;
}

hipError_t launch_quantize_nvfp4(const uint16_t* x, int64_t batches, int64_t rows, int64_t cols, const float* gs,
                                 uint8_t* q, uint8_t* sf, hipStream_t stream) {
  int64_t total = batches * rows * (cols / 16);
  if (total == 0) return hipSuccess;
  quantize_nvfp4_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(x, rows, cols, gs, q, sf, total);
  return hipGetLastError();
}

// one thread per 32-element block
__global__ void quantize_mx_kernel(const uint16_t* __restrict__ x, int elem, uint8_t* __restrict__ q,
                                   uint8_t* __restrict__ sf, int64_t total_blocks) {
  int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= total_blocks) return;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + blk * 32);
  float v[32];
  for (int c = 0; c < 4; c++) {
    u32x4_t a = src[c];
    for (int k = 0; k < 4; k++) {
      v[8 * c + 2 * k] = __uint_as_float(a[k] << 16);
      v[8 * c + 2 * k + 1] = __uint_as_float(a[k] & 0xffff0000u);
    }
  }
  float m = 0.0f;
  for (int i = 0; i < 32; i++) m = fmaxf(m, fabsf(v[i]));
  if (elem == 0) {
    uint32_t code = mx_scale_code(m, 8);
    u32x4_t o[2];
    for (int i = 0; i < 8; i++) {
      uint32_t p0 = f32x2_to_e4m3x2_mx(v[4 * i], v[4 * i + 1], code);
      uint32_t p1 = f32x2_to_e4m3x2_mx(v[4 * i + 2], v[4 * i + 3], code);
      o[i / 4][i % 4] = p0 | (p1 << 16);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(q + blk * 32);
    dst[0] = o[0];
    dst[1] = o[1];
    sf[blk] = (uint8_t)code;
  } else {
    uint32_t code = mx_scale_code(m, 2);
    float scale = e8m0_scale_operand(code);
    u32x4_t o;
    for (int i = 0; i < 4; i++) {
      uint32_t w = 0;
      for (int k = 0; k < 4; k++) w |= f32x2_to_e2m1x2(v[8 * i + 2 * k], v[8 * i + 2 * k + 1], scale) << (8 * k);
      o[i] = w;
    }
    reinterpret_cast<u32x4_t*>(q + blk * 16)[0] = o;
    sf[blk] = (uint8_t)code;
  }
}

hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int elem, uint8_t* q, uint8_t* sf,
                              hipStream_t stream) {
  int64_t total = rows * (cols / 32);
  if (total == 0) return hipSuccess;
  quantize_mx_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(x, elem, q, sf, total);
  return hipGetLastError();
}

}  // namespace moe
