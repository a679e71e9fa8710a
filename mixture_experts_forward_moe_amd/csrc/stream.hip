// stream.hip -- weight-streaming grouped GEMMs for small route tiles
// (decode-sized batches, a plan tile of 16 slots), where each expert's
// weights are used by a row or two and the pass is bound by HBM bandwidth
// on weight bytes.
//
// Same computation as gemm.hip (see there and "vllm.models.flint.ops.moe_cute",
// module docstring), organised for bandwidth instead of reuse:
//  - GEMM1: a workgroup owns one 16-slot tile and 16 gate + 16 up weight rows;
//    its 4 wavefronts split K in four, each streaming its quarter of the 32
//    rows straight from HBM into registers with several K-steps of loads in
//    flight; the partial sums meet in LDS and one wavefront applies the
//    expert scale, SwiGLU and the store.  Workgroups loop over tiles with a
//    stride, so a launch holds many thousands of wavefronts and no tile
//    count needs to be known on the host.
//  - GEMM2 + finalize: a workgroup owns 16 output columns for every tile;
//    its wavefronts take tiles round-robin, each streaming full K, and park
//    the bf16 y2 values of all slots in LDS; the workgroup then reduces each
//    token's routes in route order into `out` (the deterministic finalize of
//    "flashinfer.fused_moe.alphamoe_nvfp4_routed_moe", summary), so y2 never
//    goes to HBM.
// Lane roles follow v_mfma_f32_16x16x32_bf16: lane (c = lane%16, q = lane/16)
// holds weight row c and slot row c, and K [32q, 32q+32) of each 128-wide
// step, consumed in four 8-wide MFMA sub-steps.  Packed E2M1 weights are
// decoded with their E4M3 block scale in registers.
#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int ST_THREADS = 256;
constexpr int ST_DEPTH = 4;  // K-steps of loads in flight per wavefront

struct StreamArgs {
  const uint8_t* A;     // x (GEMM1) or y1 (GEMM2), bf16 rows
  int64_t a_row_bytes;
  const uint8_t* W;
  const uint8_t* W_sf;
  const float* alpha;
  const float* alpha_up;  // GEMM1: the up half's scale (NULL: alpha)
  const float* bias;      // NULL, or fp32 [E, 2I] (GEMM1: gate then up) / [E, H] (GEMM2)
  int K;
  int rows_per_expert;
  int I;
  int n_out;
  const int32_t* p2e;
  const int32_t* e2p;
  const int32_t* tile_expert;
  const int32_t* tile_limit;
  const int32_t* num_tiles;
  int top_k, M;
  GateAct act;          // FC1 activation
  uint16_t* Y;          // y1 (GEMM1) or y2 (GEMM2 without finalize)
  const float* topk_w;
  float rsf;
  int accumulate;
  uint16_t* out;        // GEMM2 fused finalize
};

// one K-step (128 wide) of a weight row for lane group q: 32 packed codes
// and the two E4M3 scale bytes of their blocks
struct WLoad {
  u32x4_t w;
  uint32_t s;
};

DEV WLoad load_w(const StreamArgs& a, int64_t row, int k) {
  WLoad r;
  r.w = *reinterpret_cast<const u32x4_t*>(a.W + row * (a.K / 2) + k / 2);
  r.s = *reinterpret_cast<const uint16_t*>(a.W_sf + row * (a.K / 16) + k / 16);
  return r;
}

struct ALoad {
  u32x4_t v[4];
};

DEV ALoad load_a(const StreamArgs& a, int64_t row, bool ok, int k) {
  ALoad r;
  if (ok) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(a.A + row * a.a_row_bytes + (int64_t)k * 2);
    r.v[0] = p[0];
    r.v[1] = p[1];
    r.v[2] = p[2];
    r.v[3] = p[3];
  } else {
    r.v[0] = r.v[1] = r.v[2] = r.v[3] = u32x4_t{0u, 0u, 0u, 0u};
  }
  return r;
}

DEV void mma_step(f32x4_t& acc, const ALoad& x, const WLoad& wl) {
  const float s0 = e4m3_to_f32(wl.s & 255u), s1 = e4m3_to_f32(wl.s >> 8);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.v[0]),
                                                e2m1x8_scaled_to_bf16(wl.w[0], s0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.v[1]),
                                                e2m1x8_scaled_to_bf16(wl.w[1], s0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.v[2]),
                                                e2m1x8_scaled_to_bf16(wl.w[2], s1), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.v[3]),
                                                e2m1x8_scaled_to_bf16(wl.w[3], s1), acc, 0, 0, 0);
}

// ---------------------------------------------------------------- GEMM1

__global__ __launch_bounds__(ST_THREADS) void gemm1_stream_kernel(const StreamArgs a) {
  __shared__ f32x4_t red[3][2][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int g = blockIdx.x;          // gate/up column group of 16
  const int KQ = a.K / 4;            // this wavefront's share of K
  const int k_base = wave * KQ + 32 * q;
  const int NI = KQ / 128;
  const int nt = *a.num_tiles;
  for (int pt = blockIdx.y; pt < nt; pt += gridDim.y) {
    const int e = a.tile_expert[pt];
    const int slot0 = pt * 16;
    const int valid = a.tile_limit[pt] - slot0;
    const bool row_ok = c < valid;
    const int64_t tok = row_ok ? (int64_t)(a.p2e[slot0 + c] / a.top_k) : 0;
    const int64_t rg = (int64_t)e * a.rows_per_expert + 16 * g + c;
    const int64_t ru = rg + a.I;
    f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    WLoad bg[ST_DEPTH], bu[ST_DEPTH];
    ALoad ax[ST_DEPTH];
#pragma unroll
    for (int d = 0; d < ST_DEPTH; d++) {
      if (d < NI) {
        const int k = k_base + 128 * d;
        ax[d] = load_a(a, tok, row_ok, k);
        bg[d] = load_w(a, rg, k);
        bu[d] = load_w(a, ru, k);
      }
    }
    for (int i0 = 0; i0 < NI; i0 += ST_DEPTH) {
#pragma unroll
      for (int d = 0; d < ST_DEPTH; d++) {
        const int i = i0 + d;
        if (i < NI) {
          mma_step(ag, ax[d], bg[d]);
          mma_step(au, ax[d], bu[d]);
          const int inext = i + ST_DEPTH;
          if (inext < NI) {
            const int k = k_base + 128 * inext;
            ax[d] = load_a(a, tok, row_ok, k);
            bg[d] = load_w(a, rg, k);
            bu[d] = load_w(a, ru, k);
          }
        }
      }
    }
    // partial sums of the four K quarters meet in LDS, summed in wave order
    if (wave > 0) {
      red[wave - 1][0][lane] = ag;
      red[wave - 1][1][lane] = au;
    }
    __syncthreads();
    if (wave == 0) {
      for (int w = 0; w < 3; w++) {
        ag += red[w][0][lane];
        au += red[w][1][lane];
      }
      const float al = a.alpha[e];
      const float alu = a.alpha_up ? a.alpha_up[e] : al;
      const int col = 16 * g + c;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 4 * q + i;
        float gs = ag[i] * al, us = au[i] * alu;
        if (a.bias) {
          gs = gs + a.bias[(int64_t)e * 2 * a.I + col];
          us = us + a.bias[(int64_t)e * 2 * a.I + a.I + col];
        }
        if (a.act.kind == ACT_RELU2) {  // non-gated: both rows are outputs
          if (row < valid) {
            a.Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(relu2_f32(gs));
            a.Y[(int64_t)(slot0 + row) * a.n_out + a.I + col] = f32_to_bf16(relu2_f32(us));
          }
        } else {
          const float y = gated_act_f32(gs, us, a.act);
          if (row < valid) a.Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(y);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- GEMM2 (+ finalize)

// y2 of all slots for this workgroup's 16 columns, as bf16 bits
constexpr int ST_MAX_SLOTS = 2048;

__global__ __launch_bounds__(ST_THREADS) void gemm2_stream_kernel(const StreamArgs a) {
  __shared__ uint16_t y2s[ST_MAX_SLOTS * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int g = blockIdx.x;  // output column group of 16
  const int NI = a.K / 128;
  const int nt = *a.num_tiles;
  const int my_tiles = nt > wave ? (nt - wave + 3) / 4 : 0;
  const int total = my_tiles * NI;  // flattened (tile, K-step) stream of this wavefront

  auto tile_of = [&](int f) { return wave + 4 * (f / NI); };
  auto load = [&](int f, ALoad& ax, WLoad& bw) {
    const int pt = tile_of(f);
    const int i = f % NI;
    const int e = a.tile_expert[pt];
    const int slot0 = pt * 16;
    const bool ok = c < a.tile_limit[pt] - slot0;
    const int k = 128 * i + 32 * q;
    ax = load_a(a, slot0 + c, ok, k);
    bw = load_w(a, (int64_t)e * a.rows_per_expert + 16 * g + c, k);
  };

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  WLoad bw[ST_DEPTH];
  ALoad ax[ST_DEPTH];
#pragma unroll
  for (int d = 0; d < ST_DEPTH; d++)
    if (d < total) load(d, ax[d], bw[d]);
  for (int f0 = 0; f0 < total; f0 += ST_DEPTH) {
#pragma unroll
    for (int d = 0; d < ST_DEPTH; d++) {
      const int f = f0 + d;
      if (f < total) {
        mma_step(acc, ax[d], bw[d]);
        if (f + ST_DEPTH < total) load(f + ST_DEPTH, ax[d], bw[d]);
        if (f % NI == NI - 1) {
          // end of a tile: y2 = bf16(alpha * acc) for its valid rows
          const int pt = tile_of(f);
          const int slot0 = pt * 16;
          const int valid = a.tile_limit[pt] - slot0;
          const int te = a.tile_expert[pt];
          const float al = a.alpha[te];
          const float bv = a.bias ? a.bias[(int64_t)te * a.n_out + 16 * g + c] : 0.0f;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 4 * q + i;
            float yv = acc[i] * al;
            if (a.bias) yv = yv + bv;
            const uint16_t v = f32_to_bf16(yv);
            if (row < valid) {
              if (a.out) y2s[(slot0 + row) * 16 + c] = v;
              else a.Y[(int64_t)(slot0 + row) * a.n_out + 16 * g + c] = v;
            }
          }
          acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
  if (!a.out) return;
  __syncthreads();
  // finalize this workgroup's 16 columns, each token's routes in order
  for (int idx = threadIdx.x; idx < a.M * 16; idx += ST_THREADS) {
    const int t = idx >> 4, cc = idx & 15;
    uint16_t* o = a.out + (int64_t)t * a.n_out + 16 * g + cc;
    float acc2 = a.accumulate ? bf16_to_f32(*o) : 0.0f;
    for (int j = 0; j < a.top_k; j++) {
      const int s = a.e2p[t * a.top_k + j];
      if (s < 0) continue;
      const float wf = a.topk_w[t * a.top_k + j] * a.rsf;
      acc2 = acc2 + wf * bf16_to_f32(y2s[s * 16 + cc]);
    }
    *o = f32_to_bf16(acc2);
  }
}

// ---------------------------------------------------------------- host side

bool stream_supported(int mode, const moe_plan_t* plan, int H, int I) {
  return mode == 0 && plan->tile == 16 && H % 512 == 0 && I % 512 == 0 && plan->route_slots <= ST_MAX_SLOTS;
}

static int tile_stride(const moe_plan_t* plan) { return plan->max_tiles < 64 ? plan->max_tiles : 64; }

hipError_t launch_gemm1_stream(const Gemm1Params& p, hipStream_t stream) {
  StreamArgs a = {};
  a.A = reinterpret_cast<const uint8_t*>(p.x);
  a.a_row_bytes = p.x_row_stride * 2;
  a.W = p.w1;
  a.W_sf = p.w1_sf;
  a.alpha = p.w1_alpha;
  a.alpha_up = p.w1_alpha_up;
  a.bias = p.fc1_bias;
  a.K = p.H;
  const int IP = gemm1_pairs(p);
  a.rows_per_expert = 2 * IP;
  a.I = IP;
  a.n_out = p.I;
  a.p2e = p.plan->permuted_to_expanded;
  a.tile_expert = p.plan->tile_to_expert;
  a.tile_limit = p.plan->tile_to_mn_limit;
  a.num_tiles = p.plan->num_tiles;
  a.top_k = p.plan->top_k;
  a.M = p.plan->M;
  a.act = p.act;
  a.Y = reinterpret_cast<uint16_t*>(p.y1);
  const int P = tile_stride(p.plan);
  if (P == 0) return hipSuccess;
  gemm1_stream_kernel<<<dim3(IP / 16, P), ST_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm2_stream(const Gemm2Params& p, int accumulate, hipStream_t stream) {
  StreamArgs a = {};
  a.A = reinterpret_cast<const uint8_t*>(p.y1);
  a.a_row_bytes = (int64_t)p.I * 2;
  a.W = p.w2;
  a.W_sf = p.w2_sf;
  a.alpha = p.w2_alpha;
  a.bias = p.fc2_bias;
  a.K = p.I;
  a.rows_per_expert = p.H;
  a.I = p.I;
  a.n_out = p.H;
  a.p2e = p.plan->permuted_to_expanded;
  a.e2p = p.plan->expanded_to_permuted;
  a.tile_expert = p.plan->tile_to_expert;
  a.tile_limit = p.plan->tile_to_mn_limit;
  a.num_tiles = p.plan->num_tiles;
  a.top_k = p.plan->top_k;
  a.M = p.plan->M;
  a.Y = p.y2;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.accumulate = accumulate;
  a.out = p.out;
  gemm2_stream_kernel<<<p.H / 16, ST_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
