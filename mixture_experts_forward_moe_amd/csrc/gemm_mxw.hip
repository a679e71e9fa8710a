// gemm_mxw.hip -- grouped GEMM1 (+ SwiGLU + MXFP8 requantisation) and GEMM2
// for MXFP8 activations x MXFP4 weights on 256-slot route tiles (the
// large-batch tile of pull request 4440's benchmark).
//
// The computation is the one gemm_mx.hip states (pull request 4440,
// description: MXFP8 activations and FC1 intermediate, MXFP4 weights, E8M0
// block-32 scales; "vllm.models.flint.ops.moe_cute", grouped_moe, for the
// plan):
//   GEMM1: y1 = SwiGLU(alpha1[e] * x W1[e]^T), gate/up in fp32, rounded once
//          to bf16, then requantised to MXFP8 from that bf16 value.
//   GEMM2: y2 = alpha2[e] * y1 W2[e]^T, bf16 rows or weighted packed-bf16
//          atomics into out.
//
// Shape for gfx950 (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 A x E2M1 B):
//  - a workgroup of 4 wavefronts owns one 256-slot tile and 256 weight rows;
//    wavefront (wm, wn) = (wave >> 1, wave & 1) computes slots 128 wm .. and
//    weight rows 128 wn .. as 8 x 8 tiles of 16 x 16 (256 accumulators).
//    GEMM1: the wavefront's 128 weight rows are 64 gate rows and the 64
//    matching up rows, so SwiGLU pairs and whole 32-column MXFP8 blocks of y1
//    stay inside one lane group.
//  - every operand goes global -> LDS with the LDS-DMA loads
//    (global_load_lds, 16 bytes a lane; 4 bytes for the scale words), into a
//    ring of 3 stages of 128 K (activations 32 KiB, weights 16 KiB, their
//    E8M0 scales 1 KiB each): stage s + 2 is in flight while stage s feeds
//    the MFMAs, and no register holds data in transit.  The waits are
//    explicit: a wave waits for its own loads of stage s (vmcnt counts the
//    later stage's loads, which complete after them), then the workgroup
//    barrier (s_barrier alone: a release fence would wait for every load in
//    flight) makes everyone's loads of stage s visible.
//  - the LDS positions a DMA load fills are fixed (lane i writes 16 i past
//    the wave's base), so the swizzles that keep the MFMA operand reads free
//    of bank conflicts are applied on the source side: each lane loads the
//    16-byte chunk that belongs at its position.  The scale words are placed
//    so that one lane's eight row tiles have their scales in 32 consecutive
//    bytes (two 16-byte reads per stage).
//  - per 128-K stage a wavefront issues 64 MFMAs (2048 cycles at the fp8
//    rate) against 28 LDS reads of 16 bytes and 14 LDS-DMA loads.
//  - every row tile runs its MFMAs, also past the tile's routes (a branch
//    around them would serialise the operand reads with the MFMAs); only the
//    epilogue skips row tiles without routes.  Work items (tile, weight-row
//    block) go heaviest tile first, a pair of tiles and all its weight-row
//    blocks per XCD at a time (see the kernel).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "tile_order.h"

namespace moe {

namespace {

constexpr int MT = 256;                     // threads
constexpr int MS = 256;                     // slots per tile
constexpr int MN = 256;                     // weight rows per workgroup
constexpr int MK = 128;                     // K per stage
constexpr int NBUF = 3;                     // stages in the LDS ring
constexpr int A_OFF = 0;                    // activations [256 slots][8 chunks of 16 B], swizzled
constexpr int AS_OFF = MS * MK;             // activation scale words [wm][r16][m] x 4 B
constexpr int B_OFF = AS_OFF + MS * 4;      // weights [256 rows][4 chunks of 16 B], swizzled
constexpr int BS_OFF = B_OFF + MN * MK / 2; // weight scale words [wn][r16][n] x 4 B
constexpr int STAGE = BS_OFF + MN * 4;      // 51200 B
constexpr int LDS_BYTES = NBUF * STAGE;     // 150 KiB
constexpr int DMA_PER_STAGE = 8 + 1 + 4 + 1;  // LDS-DMA loads a wavefront issues per stage
constexpr int GT = 4;                       // tiles sharing the weight blocks on one XCD

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8); counters not named are not waited for
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(3))) void lds_void_t;

struct MArgs {
  const uint8_t* A;     // x (GEMM1) or y1 (GEMM2): E4M3 rows
  int64_t a_row_bytes;
  const uint8_t* A_sf;  // their E8M0 scales, K/32 per row
  int64_t a_sf_row;
  const uint8_t* W;     // packed E2M1 rows, K/2 bytes
  const uint8_t* W_sf;  // E8M0, K/32 per row
  const float* alpha;
  const float* alpha_up;  // GEMM1: the up half's scale (NULL: alpha)
  const float* bias;      // NULL, or fp32 [E, 2I] (GEMM1: gate then up) / [E, H] (GEMM2)
  int K;
  int rows_per_expert;
  int I;
  int n_out;
  int n_blocks;         // weight-row blocks of 256 (GEMM1: 128 gate + 128 up)
  const int32_t* p2e;
  const int32_t* tile_expert;
  const int32_t* tile_limit;
  const int32_t* num_tiles;
  int top_k;
  GateAct act;
  void* Y;              // y1 E4M3 codes / y2 bf16
  uint8_t* Y_sf;        // y1 E8M0 scales
  const float* topk_w;
  float rsf;
  uint16_t* out;
};

// one LDS-DMA load: lane i moves `bytes` from g to base + bytes * i (base is
// wave-uniform)
DEV void dma16(const uint8_t* g, uint8_t* base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)base, 16, 0, 0);
}
DEV void dma4(const uint8_t* g, uint8_t* base) { __builtin_amdgcn_global_load_lds(g, (lds_void_t*)base, 4, 0, 0); }

// workgroup barrier over LDS that waits for this wave's LDS reads only (no
// release fence: it would also wait for every LDS-DMA load in flight)
DEV void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 32-column MXFP8 block of a y1 row (columns cb + r16 and cb + 16 + r16
// in this lane): the E8M0 scale from the block's 16-lane max, element pairs
// stored as 16-bit words, the scale by lane 0.
DEV void put_block(const MArgs& a, uint8_t* Yq, float y0, float y1, int row, int valid, int slot0, int cb, int r16) {
  const float am = warp_max16(fmaxf(fabsf(y0), fabsf(y1)));
  const uint32_t code = mx_scale_code(am, 8);
  const float y0n = __shfl_xor(y0, 1), y1n = __shfl_xor(y1, 1);
  if (row < valid) {
    const int64_t slot = slot0 + row;
    if ((r16 & 1) == 0) {
      *reinterpret_cast<uint16_t*>(Yq + slot * a.n_out + cb + r16) = (uint16_t)f32x2_to_e4m3x2_mx(y0, y0n, code);
      *reinterpret_cast<uint16_t*>(Yq + slot * a.n_out + cb + 16 + r16) = (uint16_t)f32x2_to_e4m3x2_mx(y1, y1n, code);
    }
    if (r16 == 0) a.Y_sf[slot * (a.n_out / 32) + cb / 32] = (uint8_t)code;
  }
}

template <int GEMM, bool ATOMIC, int AK, bool BIAS2>
DEV void item(const MArgs& a, uint8_t* smem, int e, int slot0, int valid, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int KT = a.K / MK;

  // ---- sources of this lane's LDS-DMA loads (the stage's K offset is added per stage)
  // activation row of tile slot s: the token's x row (GEMM1) or the slot's y1 row;
  // slots past the routes load the first route's row (their results are not stored)
  const int32_t first = a.p2e[slot0];
  auto arow = [&](int s) -> int64_t {
    if constexpr (GEMM == 1) return (int64_t)((s < valid ? a.p2e[slot0 + s] : first) / a.top_k);
    return (int64_t)(slot0 + min(s, valid - 1));
  };
  // weight row of local row b (0..255) of this block
  auto wrow = [&](int b) -> int64_t {
    if constexpr (GEMM == 1) {
      const int w = b >> 7, j = b & 127;
      const int col = nb * 128 + 64 * w + (j & 63);
      return (int64_t)e * a.rows_per_expert + (j < 64 ? col : a.I + col);
    } else {
      return (int64_t)e * a.rows_per_expert + nb * MN + b;
    }
  };
  const uint8_t* a_src[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int s = 64 * wave + 8 * j + (lane >> 3);         // slot of LDS position 64 (8 wave + j) + lane
    const int c = (lane & 7) ^ ((s >> 1) & 7);              // logical chunk stored there
    a_src[j] = a.A + arow(s) * a.a_row_bytes + 16 * c;
  }
  const uint8_t* as_src;
  {
    const int p = 64 * wave + lane;                          // scale word position [wm][r16][m]
    const int s = 128 * (p >> 7) + 16 * (p & 7) + ((p >> 3) & 15);
    as_src = a.A_sf + arow(s) * a.a_sf_row;
  }
  const uint8_t* b_src[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int b = 64 * wave + 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ ((b >> 2) & 3);
    b_src[j] = a.W + wrow(b) * (a.K / 2) + 16 * c;
  }
  const uint8_t* bs_src;
  {
    const int p = 64 * wave + lane;
    const int b = 128 * (p >> 7) + 16 * (p & 7) + ((p >> 3) & 15);
    bs_src = a.W_sf + wrow(b) * (a.K / 32);
  }
  auto issue = [&](int s) {
    uint8_t* st = smem + (s % NBUF) * STAGE;
    const int k0 = s * MK;
#pragma unroll
    for (int j = 0; j < 8; j++) dma16(a_src[j] + k0, st + A_OFF + 1024 * (8 * wave + j));
    dma4(as_src + k0 / 32, st + AS_OFF + 256 * wave);
#pragma unroll
    for (int j = 0; j < 4; j++) dma16(b_src[j] + k0 / 2, st + B_OFF + 1024 * (4 * wave + j));
    dma4(bs_src + k0 / 32, st + BS_OFF + 256 * wave);
  };

  // rows tiles of this wavefront that hold routes
  const int mt = __builtin_amdgcn_readfirstlane(min(8, max(0, (valid - 128 * wm + 15) >> 4)));

  f32x4_t acc[8][8];
#pragma unroll
  for (int m = 0; m < 8; m++)
#pragma unroll
    for (int n = 0; n < 8; n++) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // every wave of the previous item has read its last stage
  ring_barrier();
  issue(0);
  if (KT > 1) issue(1);

  const int a_sw = (r16 >> 1) & 7;  // activation chunk swizzle of this lane's rows
  const int b_sw = (r16 >> 2) & 3;  // weight chunk swizzle
#pragma unroll 1
  for (int s = 0; s < KT; s++) {
    // this wave's loads of stage s are done once at most the next stage's are in flight
    if (s + 1 < KT) __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA_PER_STAGE));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    ring_barrier();
    if (s + 2 < KT) issue(s + 2);
    {
      // the stage's operands: all fragment reads go out before the first
      // MFMA (no branch between them, so the waits are per fragment; a
      // branch around the MFMAs would also cost the accumulators their
      // registers across the loop)
      const uint8_t* st = smem + (s % NBUF) * STAGE;
      const u32x4_t* As = reinterpret_cast<const u32x4_t*>(st + A_OFF);
      const u32x4_t* Bs = reinterpret_cast<const u32x4_t*>(st + B_OFF);
      const u32x4_t* ASw = reinterpret_cast<const u32x4_t*>(st + AS_OFF + (128 * wm + 8 * r16) * 4);
      const u32x4_t* BSw = reinterpret_cast<const u32x4_t*>(st + BS_OFF + (128 * wn + 8 * r16) * 4);
      const u32x4_t as0 = ASw[0], as1 = ASw[1];
      const u32x4_t bs0 = BSw[0], bs1 = BSw[1];
      i32x8_t bf[8];
#pragma unroll
      for (int n = 0; n < 8; n++) {
        const int b = 128 * wn + 16 * n + r16;
        const u32x4_t v = Bs[b * 4 + (q ^ b_sw)];
        bf[n] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      }
      i32x8_t af[8];
#pragma unroll
      for (int m = 0; m < 8; m++) {
        const int row = 128 * wm + 16 * m + r16;
        const u32x4_t lo = As[row * 8 + (q ^ a_sw)];
        const u32x4_t hi = As[row * 8 + ((4 + q) ^ a_sw)];
        af[m] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int m = 0; m < 8; m++) {
        const uint32_t aw = m < 4 ? as0[m] : as1[m - 4];
        const int asc = (int)((aw >> (8 * q)) & 255u);
#pragma unroll
        for (int n = 0; n < 8; n++) {
          const uint32_t bw = n < 4 ? bs0[n] : bs1[n - 4];
          const int bsc = (int)((bw >> (8 * q)) & 255u);
          acc[m][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[m], bf[n], acc[m][n], 0, 4, 0, asc, 0, bsc);
        }
      }
    }
  }

  // ---- epilogue.  Lane holds slots 128 wm + 16 m + 4 q + i, column r16 of each tile.
  const float alpha = a.alpha[e];
  if constexpr (GEMM == 1) {
    const float alpha_u = a.alpha_up ? a.alpha_up[e] : alpha;
    const int col0 = nb * 128 + 64 * wn;  // this wave's 64 y1 columns (gate tiles n = 0..3, up n + 4)
    uint8_t* Yq = reinterpret_cast<uint8_t*>(a.Y);
#pragma unroll
    for (int m = 0; m < 8; m++) {
      if (m >= mt) continue;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 128 * wm + 16 * m + 4 * q + i;
#pragma unroll
        for (int bb = 0; bb < 2; bb++) {  // y1 block of 32 columns: tiles 2 bb, 2 bb + 1
          float y[2], z[2];
#pragma unroll
          for (int h = 0; h < 2; h++) {
            const int n = 2 * bb + h;
            float g = acc[m][n][i] * alpha;
            float u = acc[m][n + 4][i] * alpha_u;
            if (a.bias) {
              g = g + a.bias[(int64_t)e * 2 * a.I + col0 + 16 * n + r16];
              u = u + a.bias[(int64_t)e * 2 * a.I + a.I + col0 + 16 * n + r16];
            }
            // y1 is rounded once to bf16; requantisation starts from that value
            if constexpr (AK == ACT_RELU2) {
              y[h] = bf16_to_f32(f32_to_bf16(relu2_f32(g)));
              z[h] = bf16_to_f32(f32_to_bf16(relu2_f32(u)));
            } else {
              y[h] = bf16_to_f32(f32_to_bf16(gated_act_k<AK>(g, u, a.act)));
            }
          }
          put_block(a, Yq, y[0], y[1], row, valid, slot0, col0 + 32 * bb, r16);
          if constexpr (AK == ACT_RELU2) put_block(a, Yq, z[0], z[1], row, valid, slot0, a.I + col0 + 32 * bb, r16);
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < 8; m++) {
      if (m >= mt) continue;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 128 * wm + 16 * m + 4 * q + i;
        if constexpr (!ATOMIC) {
          uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y);
          if (row < valid) {
#pragma unroll
            for (int n = 0; n < 8; n++) {
              const int col = nb * MN + 128 * wn + 16 * n + r16;
              float v = acc[m][n][i] * alpha;
              if constexpr (BIAS2) v = v + a.bias[(int64_t)e * a.n_out + col];
              Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(v);
            }
          }
        } else {
          const int32_t route = (row < valid) ? a.p2e[slot0 + row] : -1;
          const float wf = (route >= 0) ? __fmul_rn(a.topk_w[route], a.rsf) : 0.0f;
#pragma unroll
          for (int n = 0; n < 8; n++) {
            const int col = nb * MN + 128 * wn + 16 * n + r16;
            float v = acc[m][n][i] * alpha;
            if constexpr (BIAS2) v = v + a.bias[(int64_t)e * a.n_out + col];
            const float y2 = bf16_to_f32(f32_to_bf16(v));
            const float c = __fmul_rn(wf, y2);
            const float cn = __shfl_xor(c, 1);
            if (route >= 0 && (r16 & 1) == 0) {
              const int64_t t = route / a.top_k;
              bf16x2_t v2 = {(__bf16)c, (__bf16)cn};
              __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<bf16x2_t*>(a.out + t * a.n_out + col), v2);
            }
          }
        }
      }
    }
  }
}

template <int GEMM, bool ATOMIC, int AK, bool BIAS2>
__global__ __launch_bounds__(MT, 1) void mxw_gemm_kernel(const MArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // A persistent grid: K blocks per XCD, block b on XCD b & 7 (workgroups
  // are dealt to the XCDs round-robin).  Tiles go in groups of GT
  // consecutive ranks of the heaviest-first order (tiles of one expert,
  // mostly), group g to XCD g & 7.  An XCD's K blocks take its items in
  // order, and a group's items are ordered in passes of K / GT weight-row
  // blocks, the GT tiles' items of one block next to each other: the K
  // concurrent items of an XCD then share each weight block among GT tiles
  // and each tile's activation rows among K / GT weight blocks, in that
  // XCD's L2.
  const int T = *a.num_tiles;
  const int x = blockIdx.x & 7;
  const int K = gridDim.x >> 3;
  const int G = (T + GT - 1) / GT;
  const int per_group = GT * a.n_blocks;
  const int pw = max(1, min(a.n_blocks, K / GT));  // weight-row blocks per pass
  for (int j = blockIdx.x >> 3;; j += K) {
    const int g = x + 8 * (j / per_group);
    if (g >= G) return;
    const int idx = j % per_group;
    const int pass = idx / (GT * pw);
    const int in = idx % (GT * pw);
    const int nb = pass * pw + in / GT;
    const int r = GT * g + in % GT;
    if (r >= T || nb >= a.n_blocks) continue;
    const int pt = tile_of_rank(a.tile_limit, T, MS, r, MT);
    const int e = __builtin_amdgcn_readfirstlane(a.tile_expert[pt]);
    const int slot0 = pt * MS;
    const int valid = __builtin_amdgcn_readfirstlane(min(MS, a.tile_limit[pt] - slot0));
    item<GEMM, ATOMIC, AK, BIAS2>(a, smem, e, slot0, valid, nb);
  }
}

void plan_args(MArgs& a, const moe_plan_t* plan) {
  a.p2e = plan->permuted_to_expanded;
  a.tile_expert = plan->tile_to_expert;
  a.tile_limit = plan->tile_to_mn_limit;
  a.num_tiles = plan->num_tiles;
  a.top_k = plan->top_k;
}

template <int GEMM, bool ATOMIC, int AK, bool BIAS2>
hipError_t launch_one(const MArgs& a, int max_tiles, hipStream_t s) {
  auto kern = mxw_gemm_kernel<GEMM, ATOMIC, AK, BIAS2>;
  // the launch needs more than the default 64 KiB of dynamic LDS: allow it
  // once per device
  static bool attr[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64 || !attr[dev]) {
    err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr[dev] = true;
  }
  // one persistent workgroup per compute unit (the LDS ring fits one)
  static int cus[64] = {};
  if (dev >= 0 && dev < 64 && !cus[dev]) {
    err = hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
  }
  const int ncu = (dev >= 0 && dev < 64 && cus[dev] > 0) ? cus[dev] : 256;
  const int grid = std::max(8, ncu / 8 * 8);
  if (max_tiles == 0) return hipSuccess;
  kern<<<grid, MT, LDS_BYTES, s>>>(a);
  return hipGetLastError();
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

}  // namespace

// 256-slot plan tiles; K a multiple of 128; whole weight-row blocks;
// 16-byte aligned activation rows; 4-byte aligned scale rows and arrays
bool mxw_supported1(const Gemm1Params& p) {
  const int64_t stride = p.x_row_stride ? p.x_row_stride : p.H;
  return p.mode == MOE_QUANT_MXFP8_MXFP4 && p.plan->tile == MS && p.H % MK == 0 && gemm1_pairs(p) % 128 == 0 &&
         stride % 16 == 0 && ((uintptr_t)p.x & 15) == 0 && aligned4(p.x_sf) && aligned4(p.w1_sf) &&
         aligned4(p.y1_sf) && ((uintptr_t)p.y1 & 1) == 0 && ((uintptr_t)p.w1 & 15) == 0;
}
bool mxw_supported2(const Gemm2Params& p) {
  return p.mode == MOE_QUANT_MXFP8_MXFP4 && p.plan->tile == MS && p.I % MK == 0 && p.H % MN == 0 &&
         ((uintptr_t)p.y1 & 15) == 0 && aligned4(p.y1_sf) && aligned4(p.w2_sf) && ((uintptr_t)p.w2 & 15) == 0;
}

hipError_t launch_gemm1_mxw(const Gemm1Params& p, hipStream_t stream) {
  MArgs a = {};
  plan_args(a, p.plan);
  a.A = reinterpret_cast<const uint8_t*>(p.x);
  a.a_row_bytes = p.x_row_stride ? p.x_row_stride : p.H;
  a.A_sf = p.x_sf;
  a.a_sf_row = p.H / 32;
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
  a.n_blocks = IP / 128;
  a.act = p.act;
  a.Y = p.y1;
  a.Y_sf = p.y1_sf;
  const int mt = p.plan->max_tiles;
  switch (p.act.kind) {
    case ACT_GEGLU_TANH: return launch_one<1, false, ACT_GEGLU_TANH, false>(a, mt, stream);
    case ACT_SITU: return launch_one<1, false, ACT_SITU, false>(a, mt, stream);
    case ACT_RELU2: return launch_one<1, false, ACT_RELU2, false>(a, mt, stream);
    default: return launch_one<1, false, ACT_SWIGLU, false>(a, mt, stream);
  }
}

hipError_t launch_gemm2_mxw(const Gemm2Params& p, hipStream_t stream) {
  MArgs a = {};
  plan_args(a, p.plan);
  a.A = reinterpret_cast<const uint8_t*>(p.y1);
  a.a_row_bytes = p.I;
  a.A_sf = p.y1_sf;
  a.a_sf_row = p.I / 32;
  a.W = p.w2;
  a.W_sf = p.w2_sf;
  a.alpha = p.w2_alpha;
  a.bias = p.fc2_bias;
  a.K = p.I;
  a.rows_per_expert = p.H;
  a.I = p.I;
  a.n_out = p.H;
  a.n_blocks = p.H / MN;
  a.Y = p.y2;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.out = p.out;
  const int mt = p.plan->max_tiles;
  if (p.out) {
    if (p.fc2_bias) return launch_one<2, true, ACT_SWIGLU, true>(a, mt, stream);
    return launch_one<2, true, ACT_SWIGLU, false>(a, mt, stream);
  }
  if (p.fc2_bias) return launch_one<2, false, ACT_SWIGLU, true>(a, mt, stream);
  return launch_one<2, false, ACT_SWIGLU, false>(a, mt, stream);
}

}  // namespace moe
