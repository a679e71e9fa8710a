// gemm_mx.hip -- grouped GEMM1 (+ SwiGLU + MXFP8 requantisation) and GEMM2
// for MXFP8 activations x MXFP4 weights on 128-slot route tiles.
//
// The computation (pull request 4440, description: MXFP8 activations and FC1
// intermediate, MXFP4 weights, E8M0 block-32 scales; "vllm.models.flint.ops.moe_cute",
// grouped_moe, for the plan):
//   GEMM1: y1 = SwiGLU(alpha1[e] * x W1[e]^T), gate/up in fp32, rounded once
//          to bf16, then requantised to MXFP8 (E4M3 codes, one E8M0 scale per
//          32 columns) from that bf16 value.
//   GEMM2: y2 = alpha2[e] * y1 W2[e]^T, bf16 rows (deterministic finalize)
//          or weighted packed-bf16 atomics into out.
//
// Both operands go straight into v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 A,
// E2M1 B, E8M0 scales per 32 K), so no vector-ALU decode sits in the K loop
// and the kernel is bound by the MFMA rate alone if the operands keep up:
//  - workgroup: 4 wavefronts, one 128-slot tile x 256 weight rows.  Each
//    wavefront keeps all 128 slots against its own 64 weight rows (8 x 4
//    tiles of 16 x 16 in its accumulators).  GEMM1: wavefront w holds gate
//    rows j0+32w.. and the matching up rows I+j0+32w.. so that SwiGLU pairs
//    and whole 32-column MXFP8 blocks of y1 sit in one wavefront; GEMM2:
//    output columns n0+64w...
//  - weights are not shared between wavefronts, so each lane loads its
//    16-byte weight fragment (K [32q, 32q+32) of one row, the layout the
//    MFMA reads) and that block's E8M0 scale byte straight from global
//    memory into registers.  Every scale is loaded as the byte its user
//    needs, so no ALU step touches a freshly loaded value (the scheduler
//    would hoist it next to the load, and the wait for it would drain every
//    load in flight).  Only the activations, shared by all
//    four wavefronts, pass through LDS: 128-K stages of 128 slots x 128
//    bytes in a 2-slot ring, loaded into registers two stages ahead and
//    written one stage ahead, 16-byte chunks swizzled by (slot >> 1) & 7 so
//    that the 16 rows of an MFMA tile read 16 distinct bank groups.  Their
//    scales sit in LDS as [block pair][slot & 15][slot >> 4][2 blocks]: a
//    thread stores the two scale bytes it loaded as one 16-bit word, and a
//    lane reads the scales of all eight of its row tiles as one 16-byte
//    word.
//  - per 128-K stage a wavefront issues 32 MFMAs against 16 LDS reads of 16
//    bytes (all issued before the first MFMA), 4 weight loads and 4 scale
//    loads.  Weights are loaded NR-1 stages and activations NR stages
//    ahead of use: with one wavefront per SIMD, the loads in flight have to
//    cover L2-miss latency on their own.
//  - row groups of 16 slots that hold no route are skipped: the tile's used
//    height picks one of eight bodies.  Tiles go heaviest first, and each XCD
//    (block b runs on XCD b & 7) takes a fixed share of the weight-row blocks
//    of every tile, so an expert's weights are read by one XCD.  The grid is
//    capped and loops over the work.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "tile_order.h"

namespace moe {

namespace {

constexpr int XT = 256;                        // threads
constexpr int XM = 128;                        // slots per tile
constexpr int XN = 256;                        // weight rows per workgroup
constexpr int XK = 128;                        // K per stage (one MFMA step)
constexpr int A_STAGE = XM * XK;               // 16 KiB of E4M3 activations
constexpr int AS_STAGE = XM * (XK / 32);       // 512 B of their E8M0 scales
constexpr int STAGE_BYTES = A_STAGE + AS_STAGE;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;     // 33 KiB
constexpr int MAX_GRID = 8192;
constexpr int NR = 4;                          // register ring: stages in flight

struct XArgs {
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
  GateAct act;          // FC1 activation
  void* Y;              // y1 E4M3 codes / y2 bf16
  uint8_t* Y_sf;        // y1 E8M0 scales
  const float* topk_w;
  float rsf;
  uint16_t* out;
};

// physical 16-byte chunk of logical chunk c in an activation row of the stage
DEV int xsw(int slot) { return (slot >> 1) & 7; }

// One 32-column MXFP8 block of a y1 row (columns cb + r16 and cb + 16 + r16
// in this lane): the E8M0 scale from the block's 16-lane max, element pairs
// stored as 16-bit words, the scale by lane 0.
DEV void mx_put_block(const XArgs& a, uint8_t* Yq, float y0, float y1, int row, int valid, int slot0, int cb,
                      int r16) {
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

template <int GEMM, bool ATOMIC, int MTV, int AK, bool BIAS2>
DEV void mx_body(const XArgs& a, uint8_t* smem, int e, int slot0, int valid, int nb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int KT = a.K / XK;

  // ---- activation staging: thread tid moves physical chunks j = 256 i + tid
  // (i < 4) of a stage, slot j >> 3, logical chunk (j & 7) ^ xsw(slot).  Slots
  // past the tile's routes read the first route's row (GEMM1) or their own
  // slot (GEMM2: y1 has every slot of the plan); they only feed accumulator
  // rows that are never stored.
  const int32_t first_route = a.p2e[slot0];
  auto src_row = [&](int slot) -> int64_t {
    if constexpr (GEMM == 1) return (int64_t)((slot < valid ? a.p2e[slot0 + slot] : first_route) / a.top_k);
    return (int64_t)(slot0 + slot);
  };
  // byte offsets of this thread's loads (inside 32 bits: the launcher checks
  // the tensor sizes)
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int slot = 32 * i + (tid >> 3);
    const int c = (tid & 7) ^ xsw(slot);
    a_off[i] = (uint32_t)(src_row(slot) * a.a_row_bytes) + (uint32_t)c * 16u;
  }
  // scales: thread tid moves block scales 2h, 2h+1 (h = tid & 1) of slot tid >> 1
  uint32_t as_off = (uint32_t)(src_row(tid >> 1) * a.a_sf_row) + 2u * (tid & 1);

  // ---- weight fragments of this lane: rows of column tile n, K [32q, 32q+32)
  // of each stage, and the row's 4 block scales of the stage
  auto wrow = [&](int n) -> int {
    if constexpr (GEMM == 1) {
      return (n < 2) ? nb * 128 + 32 * wave + 16 * n + r16 : a.I + nb * 128 + 32 * wave + 16 * (n - 2) + r16;
    } else {
      return nb * XN + 64 * wave + 16 * n + r16;
    }
  };
  const uint8_t* Wb = a.W + (int64_t)e * a.rows_per_expert * (a.K / 2);
  const uint8_t* Sb = a.W_sf + (int64_t)e * a.rows_per_expert * (a.K / 32);
  uint32_t b_off[4], bs_off[4];
#pragma unroll
  for (int n = 0; n < 4; n++) {
    b_off[n] = (uint32_t)wrow(n) * (uint32_t)(a.K / 2) + (uint32_t)q * 16u;
    bs_off[n] = (uint32_t)wrow(n) * (uint32_t)(a.K / 32) + (uint32_t)q;
  }
  // keep the offsets opaque: otherwise the compiler precomputes one address
  // per unrolled stage and runs out of the registers the accumulators need
#pragma unroll
  for (int i = 0; i < 4; i++) {
    asm volatile("" : "+v"(a_off[i]));
    asm volatile("" : "+v"(b_off[i]));
    asm volatile("" : "+v"(bs_off[i]));
  }
  asm volatile("" : "+v"(as_off));

  u32x4_t ra[NR][4];   // activation stages in flight, by stage index mod NR
  uint16_t ras[NR];    // their scales (2 bytes per thread)
  u32x4_t rb[NR][4];   // weight fragments, by stage index mod NR
  uint32_t rbs[NR][4]; // this lane's weight block scale of each column tile
  // activation loads of a stage in two halves (h = 0: chunks 0, 1; h = 1:
  // chunks 2, 3 and the scales)
  auto load_a = [&](int i2, int s, int h) {
    const int k0 = min(s, KT - 1) * XK;
#pragma unroll
    for (int i = 2 * h; i < 2 * h + 2; i++)
      ra[i2][i] = *reinterpret_cast<const u32x4_t*>(a.A + (a_off[i] + (uint32_t)k0));
    if (h == 1) ras[i2] = *reinterpret_cast<const uint16_t*>(a.A_sf + (as_off + (uint32_t)(k0 / 32)));
  };
  auto store_a = [&](int i2, int buf) {
    u32x4_t* As = reinterpret_cast<u32x4_t*>(smem + buf * STAGE_BYTES);
#pragma unroll
    for (int i = 0; i < 4; i++) As[256 * i + tid] = ra[i2][i];
    const int slot = tid >> 1;
    *reinterpret_cast<uint16_t*>(smem + buf * STAGE_BYTES + A_STAGE + 256 * (tid & 1) + (slot & 15) * 16 +
                                 (slot >> 4) * 2) = ras[i2];
  };
  auto load_b = [&](int i2, int s, int n) {
    const int k0 = min(s, KT - 1) * XK;
    rb[i2][n] = *reinterpret_cast<const u32x4_t*>(Wb + (b_off[n] + (uint32_t)(k0 / 2)));
    rbs[i2][n] = Sb[bs_off[n] + (uint32_t)(k0 / 32)];
  };

  f32x4_t acc[MTV][4];
#pragma unroll
  for (int m = 0; m < MTV; m++)
#pragma unroll
    for (int n = 0; n < 4; n++) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int sw_lane = xsw(r16);  // xsw(16 m + r16) for every m
  // a stage's activation fragments and scales, all read before its MFMAs
  // so that the LDS latency is paid once per stage
  u32x4_t fa[MTV][2];
  u32x4_t asc16;
  auto read_frags = [&](int buf) {
    const uint8_t* st = smem + buf * STAGE_BYTES;
    const u32x4_t* As = reinterpret_cast<const u32x4_t*>(st);
    asc16 = *reinterpret_cast<const u32x4_t*>(st + A_STAGE + (q >> 1) * 256 + r16 * 16);
#pragma unroll
    for (int m = 0; m < MTV; m++) {
      const int row = 16 * m + r16;
      fa[m][0] = As[row * 8 + (q ^ sw_lane)];
      fa[m][1] = As[row * 8 + ((4 + q) ^ sw_lane)];
    }
  };
  // the stage's MFMAs, row tile by row tile; after the MFMAs of row tile m
  // the wavefront issues slice m of the stage's other work, so that its
  // memory instructions never queue up in one burst in front of MFMAs
  auto mfmas = [&](int i2, auto&& work) {
    i32x8_t bf[4];
#pragma unroll
    for (int n = 0; n < 4; n++) {
      const u32x4_t b = rb[i2][n];
      bf[n] = i32x8_t{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    }
#pragma unroll
    for (int m = 0; m < MTV; m++) {
      const u32x4_t a0 = fa[m][0], a1 = fa[m][1];
      const i32x8_t af = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                 (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      const int asc = (int)((asc16[m >> 1] >> (16 * (m & 1) + 8 * (q & 1))) & 255u);
#pragma unroll
      for (int n = 0; n < 4; n++)
        acc[m][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[n], acc[m][n], 0, 4, 0, asc, 0,
                                                                     (int)rbs[i2][n]);
      __builtin_amdgcn_sched_barrier(0);
      if (m < 7) work(m);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = MTV; m < 7; m++) work(m);
  };

  // ---- prologue: activation stage 0 in LDS, stages 1 .. NR in registers;
  // weights of stages 0 .. NR-2 in registers
  load_a(0, 0, 0);
  load_a(0, 0, 1);
#pragma unroll
  for (int t = 0; t + 1 < NR; t++)
#pragma unroll
    for (int n = 0; n < 4; n++) load_b(t, t, n);
  store_a(0, 0);
#pragma unroll
  for (int t = 1; t <= NR; t++) {
    load_a(t % NR, t, 0);
    load_a(t % NR, t, 1);
  }
  __syncthreads();

  // ---- main loop, NR stages per trip (K is a whole number of NR-stage
  // groups, so the ring indices are compile-time constants and no stage is
  // conditional).  At stage s: read the stage's activation fragments from
  // LDS, then run the MFMAs row tile by row tile and between them load the
  // weights of stage s+NR-1 (one column tile per slice), write activation
  // stage s+1 (loaded NR stages earlier) to LDS and load stage s+1+NR in
  // its place; barrier.  The weights thus have NR-1 stages and
  // the activations NR stages to arrive.  Loads past the end re-read the
  // last stage into registers nobody reads again.
  auto stage = [&](int s, int j) {
    read_frags(s & 1);
    mfmas(j, [&](int slice) {
      if (slice < 4) load_b((j + NR - 1) % NR, s + NR - 1, slice);
      else if (slice == 4) store_a((j + 1) % NR, (s + 1) & 1);
      else load_a((j + 1) % NR, s + 1 + NR, slice - 5);
    });
    // only global loads may move across stages: a value hoisted next to its
    // load would wait for every load in flight
    __builtin_amdgcn_sched_barrier(0x0010);
    __syncthreads();
  };
#pragma unroll 1
  for (int s = 0; s < KT; s += NR) {
#pragma unroll
    for (int j = 0; j < NR; j++) stage(s + j, j);
  }

  // ---- epilogue.  Lane holds slots 16m + 4q + i, column r16 of each 16-wide tile.
  const float alpha = a.alpha[e];
  if constexpr (GEMM == 1) {
    const float alpha_u = a.alpha_up ? a.alpha_up[e] : alpha;
    // y1 block of 32 columns nb*128 + 32 wave .. : tiles 0 (gate) / 2 (up)
    // give columns +r16, tiles 1 / 3 columns 16 + r16
    const int col0 = nb * 128 + 32 * wave;
    uint8_t* Yq = reinterpret_cast<uint8_t*>(a.Y);
    // gated: one output block per gate / up pair block; ReLU^2 (non-gated):
    // the two row blocks are output blocks col0 and a.I + col0
    // (AK is the template form of a.act.kind: each body holds the code of one
    // activation, so the unrolled epilogue stays small)
#pragma unroll
    for (int m = 0; m < MTV; m++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float g[2], u[2];
#pragma unroll
        for (int n = 0; n < 2; n++) {
          g[n] = acc[m][n][i] * alpha;
          u[n] = acc[m][n + 2][i] * alpha_u;
          if (a.bias) {
            g[n] = g[n] + a.bias[(int64_t)e * 2 * a.I + col0 + 16 * n + r16];
            u[n] = u[n] + a.bias[(int64_t)e * 2 * a.I + a.I + col0 + 16 * n + r16];
          }
        }
        const int row = 16 * m + 4 * q + i;
        // y1 is rounded once to bf16; requantisation starts from that value
        if constexpr (AK == ACT_RELU2) {
          mx_put_block(a, Yq, bf16_to_f32(f32_to_bf16(relu2_f32(g[0]))), bf16_to_f32(f32_to_bf16(relu2_f32(g[1]))),
                       row, valid, slot0, col0, r16);
          mx_put_block(a, Yq, bf16_to_f32(f32_to_bf16(relu2_f32(u[0]))), bf16_to_f32(f32_to_bf16(relu2_f32(u[1]))),
                       row, valid, slot0, a.I + col0, r16);
        } else {
          mx_put_block(a, Yq, bf16_to_f32(f32_to_bf16(gated_act_k<AK>(g[0], u[0], a.act))),
                       bf16_to_f32(f32_to_bf16(gated_act_k<AK>(g[1], u[1], a.act))), row, valid, slot0, col0, r16);
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
              const int col = nb * XN + 64 * wave + 16 * n + r16;
              float v = acc[m][n][i] * alpha;
              if constexpr (BIAS2) v = v + a.bias[(int64_t)e * a.n_out + col];
              Y[(int64_t)(slot0 + row) * a.n_out + col] = f32_to_bf16(v);
            }
          }
        } else {
          const int32_t route = (row < valid) ? a.p2e[slot0 + row] : -1;
          const float wf = (route >= 0) ? __fmul_rn(a.topk_w[route], a.rsf) : 0.0f;
#pragma unroll
          for (int n = 0; n < 4; n++) {
            const int col = nb * XN + 64 * wave + 16 * n + r16;
            float v = acc[m][n][i] * alpha;
            if constexpr (BIAS2) v = v + a.bias[(int64_t)e * a.n_out + col];
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
__global__ __launch_bounds__(XT, 1) void mx_gemm_kernel(const XArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  // Work item w = (rank r in the heaviest-first order, weight-row block nb).
  // Block b runs on XCD b & 7 and the grid is a multiple of 8, so every item
  // a block takes stays on its XCD: XCD x takes blocks [x nbx, (x+1) nbx)
  // of every tile when the blocks split evenly, else a contiguous range of
  // (rank, block) pairs.
  const int T = *a.num_tiles;
  const int x = blockIdx.x & 7;
  for (int i = blockIdx.x >> 3;; i += gridDim.x >> 3) {
    int r, nb;
    if (a.n_blocks % 8 == 0) {
      const int nbx = a.n_blocks >> 3;
      r = i / nbx;
      nb = x * nbx + i % nbx;
    } else {
      const int per = (T * a.n_blocks + 7) >> 3;
      if (i >= per) return;
      const int L = x * per + i;
      r = L / a.n_blocks;
      nb = L % a.n_blocks;
    }
    if (r >= T) return;
    const int pt = tile_of_rank(a.tile_limit, T, XM, r, XT);
    const int e = __builtin_amdgcn_readfirstlane(a.tile_expert[pt]);
    const int slot0 = pt * XM;
    const int valid = __builtin_amdgcn_readfirstlane(min(XM, a.tile_limit[pt] - slot0));
    // one body per (used height, activation); GEMM2 has no activation but a
    // body with and one without its bias (BIAS2; GEMM1 checks its bias at run time)
    const int ak = GEMM == 1 ? a.act.kind : ACT_SWIGLU;
    auto run = [&](auto h) {
      constexpr int H = decltype(h)::value;
      if constexpr (GEMM == 1) {
        switch (ak) {
          case ACT_GEGLU_TANH: mx_body<GEMM, ATOMIC, H, ACT_GEGLU_TANH, false>(a, smem, e, slot0, valid, nb); break;
          case ACT_SITU: mx_body<GEMM, ATOMIC, H, ACT_SITU, false>(a, smem, e, slot0, valid, nb); break;
          case ACT_RELU2: mx_body<GEMM, ATOMIC, H, ACT_RELU2, false>(a, smem, e, slot0, valid, nb); break;
          default: mx_body<GEMM, ATOMIC, H, ACT_SWIGLU, false>(a, smem, e, slot0, valid, nb); break;
        }
      } else if (a.bias) {
        mx_body<GEMM, ATOMIC, H, ACT_SWIGLU, true>(a, smem, e, slot0, valid, nb);
      } else {
        mx_body<GEMM, ATOMIC, H, ACT_SWIGLU, false>(a, smem, e, slot0, valid, nb);
      }
    };
    switch ((valid + 15) >> 4) {
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      case 3: run(std::integral_constant<int, 3>{}); break;
      case 4: run(std::integral_constant<int, 4>{}); break;
      case 5: run(std::integral_constant<int, 5>{}); break;
      case 6: run(std::integral_constant<int, 6>{}); break;
      case 7: run(std::integral_constant<int, 7>{}); break;
      default: run(std::integral_constant<int, 8>{}); break;
    }
    // the next item's tile lookup and prologue reuse the LDS
    __syncthreads();
  }
}

void plan_args(XArgs& a, const moe_plan_t* plan) {
  a.p2e = plan->permuted_to_expanded;
  a.tile_expert = plan->tile_to_expert;
  a.tile_limit = plan->tile_to_mn_limit;
  a.num_tiles = plan->num_tiles;
  a.top_k = plan->top_k;
}

template <int GEMM, bool ATOMIC>
hipError_t launch(const XArgs& a, int max_tiles, hipStream_t s) {
  const int64_t items = (int64_t)max_tiles * a.n_blocks;
  const int grid = (int)((std::min<int64_t>(items, MAX_GRID) + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
  mx_gemm_kernel<GEMM, ATOMIC><<<grid, XT, 0, s>>>(a);
  return hipGetLastError();
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

}  // namespace

// MXFP8 x MXFP4 on 128-slot plan tiles: K in whole groups of NR 128-K stages, whole
// weight-row blocks, 16-byte aligned activation rows, 4-byte aligned scale
// arrays, every activation / weight byte offset inside 32 bits
bool mx_supported1(const Gemm1Params& p) {
  const int64_t stride = p.x_row_stride ? p.x_row_stride : p.H;
  if ((int64_t)p.plan->M * stride >= (1ll << 32) || (int64_t)2 * p.I * (p.H / 2) >= (1ll << 32)) return false;
  return p.mode == MOE_QUANT_MXFP8_MXFP4 && p.plan->tile == XM && p.H % (NR * XK) == 0 &&
         gemm1_pairs(p) % 128 == 0 &&
         stride % 16 == 0 && aligned4(p.x_sf) && aligned4(p.w1_sf) && aligned4(p.y1_sf) &&
         ((uintptr_t)p.y1 & 1) == 0;
}
bool mx_supported2(const Gemm2Params& p) {
  if (p.plan->route_slots * p.I >= (1ll << 32) || (int64_t)p.H * (p.I / 2) >= (1ll << 32)) return false;
  return p.mode == MOE_QUANT_MXFP8_MXFP4 && p.plan->tile == XM && p.I % (NR * XK) == 0 && p.H % XN == 0 &&
         aligned4(p.y1_sf) && aligned4(p.w2_sf);
}

hipError_t launch_gemm1_mx(const Gemm1Params& p, hipStream_t stream) {
  XArgs a = {};
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
  return launch<1, false>(a, p.plan->max_tiles, stream);
}

hipError_t launch_gemm2_mx(const Gemm2Params& p, hipStream_t stream) {
  XArgs a = {};
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
  a.n_blocks = p.H / XN;
  a.Y = p.y2;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.out = p.out;
  if (p.out) return launch<2, true>(a, p.plan->max_tiles, stream);
  return launch<2, false>(a, p.plan->max_tiles, stream);
}

}  // namespace moe
