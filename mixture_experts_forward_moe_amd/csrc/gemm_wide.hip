// gemm_wide.hip -- grouped GEMM1 (+ SwiGLU) and GEMM2 for prefill-sized
// batches with bf16 activations (W4A16) on 128-slot route tiles.
//
// Same computation as the narrow-tile kernels ("vllm.models.flint.ops.moe_cute",
// grouped_moe; "flashinfer.fused_moe.cute_dsl_fused_moe", Parameters): GEMM1
// y1 = SwiGLU(alpha1[e] * x W1[e]^T) with the weights' E2M1 x E4M3 products
// exact in bf16 and fp32 accumulation; GEMM2 y2 = alpha2[e] * y1 W2[e]^T.
//
// Why a second shape: with bf16 activations the E2M1 weights have to be
// decoded to bf16 on the vector ALU before an MFMA can use them (16 VALU
// instructions per 8 codes), so the ratio of decode work to MFMA work is set
// by how many slots reuse one decoded fragment.  Here each wavefront keeps
// all 128 slots of a tile against 64 weight rows in its accumulators (8 x 4
// tiles of 16 x 16), so a decoded fragment feeds up to 8 MFMAs.  The decode
// is interleaved with the MFMAs of the same wavefront (MFMA and VALU
// overlap far better inside one instruction stream than across wavefronts):
// a stage runs in two halves, the MFMAs of weight-row groups 0, 1 while
// groups 2, 3 are decoded, then those of groups 2, 3 while groups 0, 1 of
// the next stage are decoded.  The 16-slot row groups that hold no route are
// skipped whole: the tile's used height picks one of eight unrolled bodies.
//
//  - workgroup: 4 wavefronts, one 128-slot tile x 256 weight rows.  GEMM1:
//    128 gate rows j0.. and the 128 matching up rows I+j0.., wavefront w
//    holding gate rows j0+32w.. and up rows I+j0+32w.. so that SwiGLU pairs
//    sit in one lane.  GEMM2: output columns n0+64w...
//  - Operands are staged through registers: every thread loads its share
//    of a stage with 16-byte loads two stages before the stage is used and
//    writes it to LDS one stage before.  Codes and scales are staged by the
//    wavefront that uses them, so only the activations need the barrier.  Activations come in 32-K stages
//    (2-slot LDS ring), codes in 128-K groups of 64 bytes per weight row and
//    their scales in 8-byte pieces (2-slot rings), a group written a quarter
//    per stage during the group before it.  52 KiB of LDS, two workgroups
//    per CU; the wait counts are the compiler's and the loop body has no
//    branch.
//  - LDS layouts, swizzled per 16-byte chunk so that the operand reads are
//    (nearly) bank-conflict free: activations [slot][4 chunks], chunk c at
//    c ^ sa(slot); codes [row][4 chunks], chunk c at c ^ ((row >> 2) & 3);
//    scales [row][8 bytes].
//  - reduction order: in a stage lane group q takes K [8q, 8q + 8), one
//    dword of codes under one E4M3 block scale.
//  - tile order: heaviest tiles first (by used height), so that the short
//    tiles fill the tail; each XCD (block b runs on XCD b & 7) takes a fixed
//    eighth of the weight-row blocks of every tile, so an expert's weights
//    are read by one XCD and the load is the same on all eight.  This is the
//    eight-domain form of the localized weights of
//    "flashinfer.fused_moe.cute_dsl_fused_moe" (Parameters: FC1 split by I,
//    FC2 by H, each locality domain reading only its part).
#include "device_common.h"
#include "internal.h"
#include "tile_order.h"

namespace moe {

namespace {

constexpr int WT = 256;   // threads
constexpr int WM = 128;   // slots per tile
constexpr int WN = 256;   // weight rows per workgroup
constexpr int AK = 32;    // K per activation stage
constexpr int GK = 128;   // K per code / scale group (4 stages)
constexpr int P = 2;      // stages between an activation load and its use
constexpr int A_STAGE = WM * AK * 2;   // 8 KiB
constexpr int B_GROUP = WN * GK / 2;   // 16 KiB
constexpr int S_GROUP = WN * GK / 16;  // 2 KiB
constexpr int B_OFF = 2 * A_STAGE;
constexpr int S_OFF = B_OFF + 2 * B_GROUP;
constexpr int LDS_BYTES = S_OFF + 2 * S_GROUP;  // 52 KiB

struct WArgs {
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
  int n_blocks;         // weight-row blocks of 256 (GEMM1: 128 gate + 128 up)
  const int32_t* p2e;
  const int32_t* tile_expert;
  const int32_t* tile_limit;
  const int32_t* num_tiles;
  int top_k;
  GateAct act;          // FC1 activation
  void* Y;
  const float* topk_w;
  float rsf;
  uint16_t* out;
};

// activation chunk swizzle (depends on slot & 15 only, so that the 16 rows
// of an MFMA tile hit 16 distinct 16-byte bank groups)
DEV int sa(int slot) { return (((slot & 15) >> 1) ^ ((slot & 15) >> 3)) & 3; }
// code chunk swizzle: the 4 rows r, r+4, r+8, r+12 of a 16-row group (64 B
// per row, so they share banks) get 4 distinct chunks, and a wavefront's
// dword reads of one stage hit 64 distinct banks
DEV int sb(int row) { return (row >> 2) & 3; }

template <int GEMM, bool ATOMIC, int MTV>
DEV void wide_body(const WArgs& a, uint8_t* smem, int e, int slot0, int valid, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;

  // ---- what each thread loads and where it lands
  // activations: stage chunk j = 256 i + tid (i = 0, 1) holds slot j >> 2,
  // logical chunk (j & 3) ^ sa(slot).  Slots past the tile's routes read
  // the first route's row (GEMM1) or their own slot (GEMM2: y1 has every
  // slot of the plan); they only feed accumulator rows that are never
  // stored.
  const int32_t first_route = a.p2e[slot0];
  uint32_t a_off[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int j = 256 * i + tid;
    const int slot = j >> 2;
    const int c = (j & 3) ^ sa(slot);
    int64_t src = slot0 + slot;
    if constexpr (GEMM == 1) src = (slot < valid ? a.p2e[slot0 + slot] : first_route) / a.top_k;
    a_off[i] = (uint32_t)(src * a.a_row_bytes) + (uint32_t)c * 16u;
  }
  auto wrow = [&](int lc) -> int {
    if constexpr (GEMM == 1) {
      const int w = lc >> 6, n = (lc >> 4) & 3, r = lc & 15;
      return (n < 2) ? nb * 128 + 32 * w + 16 * n + r : a.I + nb * 128 + 32 * w + 16 * (n - 2) + r;
    } else {
      return nb * WN + lc;
    }
  };
  const uint8_t* Wb = a.W + (int64_t)e * a.rows_per_expert * (a.K / 2);
  const uint8_t* Sb = a.W_sf + (int64_t)e * a.rows_per_expert * (a.K / 16);
  // codes and scales are staged by the wavefront that uses them (its 64
  // weight rows), so they need no workgroup barrier.  Code quarter qq of a
  // group: lane l writes row 64 wave + 16 qq + l / 4, physical chunk l & 3
  // (logical chunk (l & 3) ^ sb(row)); scales: row tid, 8 bytes.
  uint32_t b_off[4];
#pragma unroll
  for (int qq = 0; qq < 4; qq++) {
    const int row = 64 * wave + 16 * qq + (lane >> 2);
    const int c = (lane & 3) ^ sb(row);
    b_off[qq] = (uint32_t)wrow(row) * (uint32_t)(a.K / 2) + (uint32_t)c * 16u;
  }
  uint32_t s_off = (uint32_t)wrow(tid) * (uint32_t)(a.K / 16);
  // GEMM2: keep the load offsets opaque; recomputing them inside the loop
  // costs registers the accumulators need
  if constexpr (GEMM == 2) {
#pragma unroll
    for (int i = 0; i < 2; i++) asm volatile("" : "+v"(a_off[i]));
#pragma unroll
    for (int i = 0; i < 4; i++) asm volatile("" : "+v"(b_off[i]));
    asm volatile("" : "+v"(s_off));
  }

  const int KT = a.K / AK;
  const int KG = KT / 4;
  u32x4_t ra[P][2];   // activation stages, by stage index mod P
  u32x4_t rb[2];      // code quarters, by quarter index mod 2
  uint2 rs;           // its scales
  auto load_a = [&](u32x4_t* r, int s) {
    const uint32_t k0 = (uint32_t)min(s, KT - 1) * (AK * 2);
#pragma unroll
    for (int i = 0; i < 2; i++) r[i] = *reinterpret_cast<const u32x4_t*>(a.A + (a_off[i] + k0));
  };
  auto load_b = [&](int qq, int g) {
    const uint32_t k0 = (uint32_t)min(g, KG - 1) * (GK / 2);
    rb[qq & 1] = *reinterpret_cast<const u32x4_t*>(Wb + (b_off[qq] + k0));
  };
  auto load_s = [&](int g) {
    const uint32_t k0 = (uint32_t)min(g, KG - 1) * (GK / 16);
    rs = *reinterpret_cast<const uint2*>(Sb + (s_off + k0));
  };
  auto store_a = [&](const u32x4_t* r, int slot) {
    u32x4_t* As = reinterpret_cast<u32x4_t*>(smem + slot * A_STAGE);
#pragma unroll
    for (int i = 0; i < 2; i++) As[256 * i + tid] = r[i];
  };
  auto store_b = [&](int qq, int gslot) {
    reinterpret_cast<u32x4_t*>(smem + B_OFF + gslot * B_GROUP)[256 * wave + 64 * qq + lane] = rb[qq & 1];
  };
  auto store_s = [&](int gslot) { reinterpret_cast<uint2*>(smem + S_OFF + gslot * S_GROUP)[tid] = rs; };

  f32x4_t acc[MTV][4];
#pragma unroll
  for (int m = 0; m < MTV; m++)
#pragma unroll
    for (int n = 0; n < 4; n++) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int a_lane = r16 * (AK * 2) + ((q ^ sa(r16)) << 4);
  // this lane's code dword and scale of weight-row group n at stage t of
  // group g (rows 64 wave + 16 n + r16, K [8q, 8q + 8) of the stage)
  const int b_lane = (64 * wave + r16) * 64 + 4 * q;
  const int b_sw = sb(r16);
  const int s_lane = (64 * wave + r16) * 8 + (q >> 1);
  auto decode = [&](int t, int g, int n) -> bf16x8_t {
    const uint8_t* Bs = smem + B_OFF + (g & 1) * B_GROUP + b_lane + n * 16 * 64 + ((t ^ b_sw) << 4);
    const uint8_t* Ss = smem + S_OFF + (g & 1) * S_GROUP + s_lane + n * 16 * 8 + 2 * t;
    return e2m1x8_scaled_to_bf16(*reinterpret_cast<const uint32_t*>(Bs),
                                 __builtin_amdgcn_cvt_f32_fp8((int)*Ss, 0));
  };
  // Stage t of group g in two halves: the MFMAs of weight-row groups 0, 1
  // run while groups 2, 3 of this stage are decoded, those of groups 2, 3
  // while groups 0, 1 of the next stage (tn of group gn) are decoded.
  // Activation fragments are read from LDS once per half.
  bf16x8_t bf[4];
  auto compute = [&](int t, int g, int tn, int gn) {
    const uint8_t* As = smem + (t & 1) * A_STAGE + a_lane;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(As);
#pragma unroll
      for (int m = 0; m < MTV; m++) {
        bf16x8_t nf = af;
        if (m + 1 < MTV) nf = *reinterpret_cast<const bf16x8_t*>(As + (m + 1) * 16 * AK * 2);
        acc[m][2 * h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[2 * h], acc[m][2 * h], 0, 0, 0);
        acc[m][2 * h + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[2 * h + 1], acc[m][2 * h + 1], 0, 0, 0);
        if (m == 0) {
          if (h == 0) bf[2] = decode(t, g, 2); else bf[0] = decode(tn, gn, 0);
        }
        if (m == (MTV > 1 ? 1 : 0)) {
          if (h == 0) bf[3] = decode(t, g, 3); else bf[1] = decode(tn, gn, 1);
        }
        af = nf;
      }
    }
  };

  // ---- prologue: stage 0, group 0 and its scales in LDS; registers hold
  // stages 1 and 2, code quarters 0 and 1 of group 1 and its scales
  load_a(ra[0], 0);
  load_s(0);
  store_a(ra[0], 0);
  store_s(0);
#pragma unroll
  for (int qq = 0; qq < 4; qq++) {
    load_b(qq, 0);
    store_b(qq, 0);
  }
#pragma unroll
  for (int s = 1; s <= P; s++) load_a(ra[s % P], s);
  load_b(0, 1);
  load_b(1, 1);
  load_s(1);
  __syncthreads();
  bf[0] = decode(0, 0, 0);
  bf[1] = decode(0, 0, 1);

  // ---- main loop, one code group (4 stages) per trip.  At stage s = 4g + t:
  // write stage s+1 (loaded at s-2) and code quarter t of group g+1 (loaded
  // at s-2), load stage s+3 and the code quarter written at s+2; at t = 0
  // write the scales of group g+1 and load those of g+2; compute stage s;
  // barrier.  Loads past the end re-read the last stage / group into slots
  // nobody reads again.
#pragma unroll 1
  for (int g = 0; g < KG; g++) {
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const int s = 4 * g + t;
      store_a(ra[(t + 1) % P], (t + 1) & 1);
      load_a(ra[(t + 1) % P], s + 1 + P);
      store_b(t, (g + 1) & 1);
      if (t < 2)
        load_b(t + 2, g + 1);
      else
        load_b(t - 2, g + 2);
      if (t == 0) {
        store_s((g + 1) & 1);
        load_s(g + 2);
      }
      compute(t, g, (t + 1) & 3, t == 3 ? g + 1 : g);
      // only global loads may move across stages: interleaving the MFMAs of
      // two stages renames the accumulators and runs out of registers
      __builtin_amdgcn_sched_barrier(0x0010);
      __syncthreads();
    }
  }

  // ---- epilogue.  Lane holds slots 16m + 4q + i, column r16 of each 16-wide tile.
  const float alpha = a.alpha[e];
  if constexpr (GEMM == 1) {
    const float alpha_u = a.alpha_up ? a.alpha_up[e] : alpha;
#pragma unroll
    for (int n = 0; n < 2; n++) {
      const int col = nb * 128 + 32 * wave + 16 * n + r16;  // y1 column
      // gated: one output per gate / up pair; ReLU^2 (non-gated): the two
      // rows of a pair are outputs col and a.I + col
      const bool two = a.act.kind == ACT_RELU2;
      uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y);
#pragma unroll
      for (int m = 0; m < MTV; m++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float g = acc[m][n][i] * alpha;
          float u = acc[m][n + 2][i] * alpha_u;
          if (a.bias) {
            g = g + a.bias[(int64_t)e * 2 * a.I + col];
            u = u + a.bias[(int64_t)e * 2 * a.I + a.I + col];
          }
          const int row = 16 * m + 4 * q + i;
          // y1 is rounded once to bf16
          if (row < valid) {
            if (two) {
              Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(relu2_f32(g));
              Y[(int64_t)(slot0 + row) * a.n_out + a.I + col] = f32_to_bf16(relu2_f32(u));
            } else {
              Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(gated_act_f32(g, u, a.act));
            }
          }
        }
    }
  } else {
#pragma unroll
    for (int m = 0; m < MTV; m++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 16 * m + 4 * q + i;
        if constexpr (!ATOMIC) {
          uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y);
          if (row < valid) {
#pragma unroll
            for (int n = 0; n < 4; n++) {
              const int col = nb * WN + 64 * wave + 16 * n + r16;
              float v = acc[m][n][i] * alpha;
              if (a.bias) v = v + a.bias[(int64_t)e * a.n_out + col];
              Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(v);
            }
          }
        } else {
          const int32_t route = (row < valid) ? a.p2e[slot0 + row] : -1;
          const float wf = (route >= 0) ? __fmul_rn(a.topk_w[route], a.rsf) : 0.0f;
#pragma unroll
          for (int n = 0; n < 4; n++) {
            const int col = nb * WN + 64 * wave + 16 * n + r16;
            float v = acc[m][n][i] * alpha;
            if (a.bias) v = v + a.bias[(int64_t)e * a.n_out + col];
            const float y2 = bf16_to_f32(f32_to_bf16(v));
            const float c = __fmul_rn(wf, y2);
            const float cn = __shfl_xor(c, 1);
            if (route >= 0 && (r16 & 1) == 0) {
              const int64_t t = route / a.top_k;
              bf16x2_t v = {(__bf16)c, (__bf16)cn};
              __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<bf16x2_t*>(a.out + t * a.n_out + col), v);
            }
          }
        }
      }
  }
}



template <int GEMM, bool ATOMIC>
__global__ __launch_bounds__(WT, 2) void wide_gemm_kernel(const WArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  // ---- tile of this workgroup.  Tiles 0 .. num_tiles-1 are in use.  The
  // workgroup's rank r in the heaviest-first order and its weight-row block:
  // XCD x takes blocks [x nbx, (x+1) nbx) of every tile when the blocks
  // split evenly, else a contiguous range of (rank, block) pairs.
  const int T = *a.num_tiles;
  const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
  int r, nb;
  if (a.n_blocks % 8 == 0) {
    const int nbx = a.n_blocks >> 3;
    r = i / nbx;
    nb = x * nbx + i % nbx;
  } else {
    const int per = (T * a.n_blocks + 7) >> 3;
    const int L = x * per + i;
    if (i >= per) return;
    r = L / a.n_blocks;
    nb = L % a.n_blocks;
  }
  if (r >= T) return;

  const int pt = tile_of_rank(a.tile_limit, T, WM, r, WT);
  const int e = __builtin_amdgcn_readfirstlane(a.tile_expert[pt]);
  const int slot0 = pt * WM;
  const int valid = __builtin_amdgcn_readfirstlane(min(WM, a.tile_limit[pt] - slot0));

  switch ((valid + 15) >> 4) {
    case 1: wide_body<GEMM, ATOMIC, 1>(a, smem, e, slot0, valid, nb); break;
    case 2: wide_body<GEMM, ATOMIC, 2>(a, smem, e, slot0, valid, nb); break;
    case 3: wide_body<GEMM, ATOMIC, 3>(a, smem, e, slot0, valid, nb); break;
    case 4: wide_body<GEMM, ATOMIC, 4>(a, smem, e, slot0, valid, nb); break;
    case 5: wide_body<GEMM, ATOMIC, 5>(a, smem, e, slot0, valid, nb); break;
    case 6: wide_body<GEMM, ATOMIC, 6>(a, smem, e, slot0, valid, nb); break;
    case 7: wide_body<GEMM, ATOMIC, 7>(a, smem, e, slot0, valid, nb); break;
    default: wide_body<GEMM, ATOMIC, 8>(a, smem, e, slot0, valid, nb); break;
  }
}

void plan_args(WArgs& a, const moe_plan_t* plan) {
  a.p2e = plan->permuted_to_expanded;
  a.tile_expert = plan->tile_to_expert;
  a.tile_limit = plan->tile_to_mn_limit;
  a.num_tiles = plan->num_tiles;
  a.top_k = plan->top_k;
}

template <int GEMM, bool ATOMIC>
hipError_t launch(const WArgs& a, int max_tiles, hipStream_t s) {
  const int grid = (max_tiles * a.n_blocks + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  wide_gemm_kernel<GEMM, ATOMIC><<<grid, WT, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

// W4A16 on 128-slot plan tiles, K in whole code groups, whole weight-row
// blocks, and every activation / weight byte offset inside 32 bits
bool wide_supported1(const Gemm1Params& p) {
  const int64_t stride = p.x_row_stride ? p.x_row_stride : p.H;
  return p.mode == MOE_QUANT_W4A16 && p.plan->tile == WM && p.H % GK == 0 && gemm1_pairs(p) % 128 == 0 &&
         (int64_t)p.plan->M * stride * 2 < (1ll << 32) && (int64_t)2 * p.I * (p.H / 2) < (1ll << 32);
}
bool wide_supported2(const Gemm2Params& p) {
  return p.mode == MOE_QUANT_W4A16 && p.plan->tile == WM && p.I % GK == 0 && p.H % WN == 0 &&
         p.plan->route_slots * p.I * 2 < (1ll << 32) && (int64_t)p.H * (p.I / 2) < (1ll << 32);
}

hipError_t launch_gemm1_wide(const Gemm1Params& p, hipStream_t stream) {
  WArgs a = {};
  plan_args(a, p.plan);
  a.A = reinterpret_cast<const uint8_t*>(p.x);
  a.a_row_bytes = (p.x_row_stride ? p.x_row_stride : p.H) * 2;
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
  return launch<1, false>(a, p.plan->max_tiles, stream);
}

hipError_t launch_gemm2_wide(const Gemm2Params& p, hipStream_t stream) {
  WArgs a = {};
  plan_args(a, p.plan);
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
  a.n_blocks = p.H / WN;
  a.Y = p.y2;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.out = p.out;
  if (p.out) return launch<2, true>(a, p.plan->max_tiles, stream);
  return launch<2, false>(a, p.plan->max_tiles, stream);
}

}  // namespace moe
