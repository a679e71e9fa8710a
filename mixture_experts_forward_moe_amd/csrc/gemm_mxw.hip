// gemm_mxw.hip -- grouped GEMM1 (+ gated activation + MXFP8 requantisation)
// and GEMM2 for MXFP8 activations x MXFP4 weights on 256-slot route tiles
// (the large-batch tile of pull request 4440's benchmark).
//
// The computation is the one gemm_mx.hip states (pull request 4440,
// description: MXFP8 activations and FC1 intermediate, MXFP4 weights, E8M0
// block-32 scales; "vllm.models.flint.ops.moe_cute", grouped_moe, for the
// plan):
//   GEMM1: y1 = act(alpha1[e] * x W1[e]^T), gate/up in fp32, rounded once to
//          bf16, then requantised to MXFP8 from that bf16 value.
//   GEMM2: y2 = alpha2[e] * y1 W2[e]^T, bf16 rows or weighted packed-bf16
//          atomics into out.
//
// Shape for gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 weights as the A
// operand, E4M3 activations as B):
//  - a work item is (plan tile of 256 slots, block of 256 weight rows); a
//    workgroup of 4 wavefronts computes it, wavefront (ww, ws) = (wave & 1,
//    wave >> 1) the 128 weight rows 128 ww .. and the 128 slots 128 ws .. as
//    4 x 4 MFMA tiles of 32 x 32 (256 accumulators).  GEMM1: a wavefront's
//    128 weight rows are 64 gate rows (tiles 0, 1) and the 64 matching up
//    rows (tiles 2, 3), so SwiGLU pairs sit in one lane.
//  - the weight rows of an MFMA tile are loaded in the order that gives lane
//    (slot r, half h) the 16 consecutive output columns 16 h .. 16 h + 15 of
//    the tile: a 32-column MXFP8 block of one y1 row is two lanes, its codes
//    one 16-byte store per lane.
//  - every operand goes global -> LDS with the LDS-DMA loads
//    (global_load_lds: 16 bytes a lane, 4 for route ids, bias and routing
//    weights) into a ring of 3 stages of 128 K; the ring runs on across
//    work items, so the next item's first stages load while this item
//    finishes and writes its epilogue.  The E8M0 scales come in groups of 4
//    stages (16 bytes a row) into one LDS area; each lane keeps its rows'
//    records in registers.  A wavefront's loads per stage are fixed by the
//    stage's place in its group (activations 8, weights 4; the next item's
//    bias and this item's routing weights when the epilogue uses them; the
//    group's scales and the next item's route ids with the group's first
//    stage), so "stage s + 1 has landed" is a fixed vmcnt wait, then a bare
//    s_barrier (a release fence would also wait for the loads in flight)
//    publishes every wavefront's part.  The epilogue reads only LDS and
//    scalars: a vector load there would make the compiler wait for every
//    DMA in flight.
//  - operand fragments are double-buffered in registers per 64-K half
//    stage: the half-stage reads go out while the other half's 16 MFMAs
//    run, so the matrix cores do not wait for LDS.  One barrier per stage.
//  - the LDS positions a DMA load fills are fixed (lane i writes 16 i past
//    the wave's base), so the swizzles that keep fragment reads free of bank
//    conflicts (64 banks of 4 bytes, 8 lanes a clock for 16-byte reads) are
//    applied on the source side: each lane loads the chunk that belongs at
//    its position.
//  - every MFMA tile runs, also past a tile's routes; only the epilogue
//    skips slots without routes.  Items go in plan order, groups of GT
//    consecutive tiles (tiles of one expert, mostly) per XCD with all their
//    weight-row blocks, so an XCD's workgroups share each weight block among
//    GT tiles in that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace moe {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int MT = 256;                          // threads
constexpr int MS = 256;                          // slots per tile
constexpr int MN = 256;                          // weight rows per item
constexpr int MK = 128;                          // K per stage
constexpr int NBUF = 3;                          // stages in the LDS ring
constexpr int GS = 4;                            // stages per scale group
constexpr int X_OFF = 0;                         // activations [256 slots][8 chunks of 16 B]
constexpr int W_OFF = MS * MK;                   // weights [256 rows][4 chunks of 16 B]
constexpr int STAGE = W_OFF + MN * MK / 2;       // 48 KiB
constexpr int SX_OFF = NBUF * STAGE;             // a scale group: activation scales [256 slots][16 B]
constexpr int SW_OFF = SX_OFF + MS * 16;         // and weight scales [256 rows][16 B]
constexpr int P_OFF = SW_OFF + MN * 16;          // route ids: two buffers of 256
constexpr int B_OFF = P_OFF + 2 * 1024;          // bias: two buffers of 256 fp32
constexpr int T_OFF = B_OFF + 2 * 1024;          // routing weights: two buffers of 256 fp32
constexpr int LDS_BYTES = T_OFF + 2 * 1024;      // 158 KiB
constexpr int GT = 4;                            // tiles sharing the weight blocks on one XCD
constexpr int MIN_KT = 8;                        // stages per item the ring schedule needs

static_assert(LDS_BYTES <= 160 * 1024, "LDS ring exceeds the CU's LDS");

// LDS-DMA loads a wavefront issues for one stage: activations 8, weights 4,
// the next item's bias 1 (BIAS), this item's routing weights 1 (TOPW); the
// first stage of a scale group also loads the group's activation and
// weight scales (16 bytes a row: 4 stages) and the next item's route ids
template <bool BIAS, bool TOPW>
constexpr int dma_base() { return 12 + (BIAS ? 1 : 0) + (TOPW ? 1 : 0); }
constexpr int DMA_GROUP = 3;

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
  int I;                // GEMM1: row pairs per expert
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
DEV void dma16(const void* g, uint8_t* base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)base, 16, 0, 0);
}
DEV void dma4(const void* g, uint8_t* base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)base, 4, 0, 0);
}

// workgroup barrier over LDS that waits for this wave's LDS reads only (no
// release fence: it would also wait for every LDS-DMA load in flight)
DEV void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A copy of v that the compiler cannot see through: index arithmetic built
// on it is redone where it is used instead of being hoisted out of the
// loops and kept live (the registers go to the operand fragments).
DEV int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
DEV uint32_t ou(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Word of slot s in a route-id buffer: the ids a lane's 8 activation loads
// need are 8 consecutive words (wave w, lane group g = lane >> 3: slots
// 64 w + 8 j + g at word 64 w + 8 g + j).
DEV int p_word(int s) { return (s >> 6) * 64 + (s & 7) * 8 + ((s >> 3) & 7); }

// Output column (0..31) that MFMA row i of a tile stands for: lane half h,
// element j of the 32x32 result holds row 8 (j / 4) + 4 h + j % 4, which is
// column 16 h + j.
DEV int tile_col(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// Row of weight-row position b (0..255) of an item, counted from the
// item's first row (expert e, block nb: row block_row(nb) of the expert;
// GEMM1's up rows are I further on).
template <int GEMM>
DEV int weight_row(const MArgs& a, int b) {
  const int col = tile_col(b & 31);
  if constexpr (GEMM == 1) {
    const int m = (b >> 5) & 3;
    const int c = 64 * (b >> 7) + 32 * (m & 1) + col;
    return m < 2 ? c : a.I + c;
  } else {
    return (b & ~31) + col;
  }
}
template <int GEMM>
DEV int block_row(int nb) { return nb * (GEMM == 1 ? 128 : MN); }

// A work item's wave-uniform facts: plan tile, weight-row block, local
// expert, routes in the tile.
struct Item {
  int pt, nb, e, valid;
};

// Per-lane 32-bit source offsets (the stage's K offset, and what is
// uniform over an item, go into the wave-uniform bases): the activation
// chunks and the scale row of this lane's scale-group load (slot position
// 64 wave + lane), its routing weight (TOPW) -- per item in GEMM1, whose
// rows are gathered tokens -- and the weight chunks and weight scale row,
// the same for every item.
struct Src {
  uint32_t x[8], xs, tw;
};
struct WSrc {
  uint32_t w[4], ws;
};

// Fragments of one 64-K half stage: weight tiles m (this lane's row, K half
// h: 32 E2M1 codes) and slot tiles n (32 E4M3 codes in two pieces).
struct Frag {
  u32x4_t w[4];
  u32x4_t x[4][2];
};
// A scale group in registers: this lane's rows of weight tiles m and slot
// tiles n, 16 E8M0 bytes each (word g: the 4 blocks of the group's stage g).
struct Group {
  u32x4_t w[4], x[4];
};

DEV Item load_item(const MArgs& a, int pt, int nb) {
  Item it;
  it.pt = pt;
  it.nb = nb;
  it.e = ld_uniform(a.tile_expert + pt);
  it.valid = min(MS, ld_uniform(a.tile_limit + pt) - pt * MS);
  return it;
}

// Source offsets of an item; its route ids are in buffer P.  GEMM2's
// activation rows are the tile's own slots (padding slots read their own,
// unused rows of y1: an output element depends only on its own slot), so
// without TOPW its offsets are the same for every item.
template <int GEMM, bool TOPW>
DEV Src sources(const MArgs& a, const Item& it, const uint8_t* P, int wave, int lane_) {
  const int lane = opaque(lane_);
  Src s;
  const int g = lane >> 3;
  // (32-bit arithmetic: the host checks that every offset fits in 31 bits)
  const uint32_t rb = (uint32_t)a.a_row_bytes, sb = (uint32_t)a.a_sf_row;
  const int p = 64 * wave + lane;  // slot position of this lane's scale-group load
  int32_t rt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int32_t first = 0, rp = 0;
  if constexpr (GEMM == 1 || TOPW) rp = *reinterpret_cast<const int32_t*>(P + 4 * p_word(p));
  if constexpr (GEMM == 1) {
    const u32x4_t r0 = *reinterpret_cast<const u32x4_t*>(P + 4 * (64 * wave + 8 * g));
    const u32x4_t r1 = *reinterpret_cast<const u32x4_t*>(P + 4 * (64 * wave + 8 * g) + 16);
    first = *reinterpret_cast<const int32_t*>(P);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      rt[j] = (int32_t)r0[j];
      rt[4 + j] = (int32_t)r1[j];
    }
  }
  // GEMM1: the token of the slot's route (padding slots: the tile's first
  // route); GEMM2: the slot, counted from the tile's first
  auto row_of = [&](int slot, int32_t route) -> uint32_t {
    if constexpr (GEMM == 1) return (uint32_t)((slot < it.valid ? route : first) / a.top_k);
    return (uint32_t)slot;
  };
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int slot = 64 * wave + 8 * j + g;
    const int c = (lane & 7) ^ ((slot >> 1) & 7);  // logical chunk of physical chunk lane & 7
    s.x[j] = row_of(slot, rt[j]) * rb + 16u * c;
  }
  s.xs = row_of(p, rp) * sb;
  // routing weight of slot p (padding slots load entry 0; it is not used)
  s.tw = TOPW ? 4u * (uint32_t)max(0, rp) : 0u;
  return s;
}

template <int GEMM>
DEV WSrc weight_sources(const MArgs& a, int wave, int lane_) {
  const int lane = opaque(lane_);
  WSrc s;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int b = 64 * wave + 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ ((b >> 2) & 3);
    s.w[j] = (uint32_t)weight_row<GEMM>(a, b) * (uint32_t)(a.K / 2) + 16u * c;
  }
  s.ws = (uint32_t)weight_row<GEMM>(a, 64 * wave + lane) * (uint32_t)(a.K / 32);
  return s;
}

// What one stage loads, and where to.
struct Dst {
  const uint8_t *xb, *wb, *xsb, *wsb;  // sources at the stage's K offset: activations, weights, their scales
  uint8_t* st;                         // stage buffer
  const int32_t* p2e_tile;             // next item's route ids -> P
  uint8_t* P;
  const float* bias;                   // next item's 256 bias values (BIAS) -> B
  uint8_t* B;
  uint8_t* T;                          // routing weights of the sources' item (TOPW)
};

template <int GEMM>
DEV void stage_bases(const MArgs& a, const Item& it, int k0, Dst& d) {
  const int64_t wrow0 = (int64_t)it.e * a.rows_per_expert + block_row<GEMM>(it.nb);
  const int64_t xrow0 = GEMM == 1 ? 0 : (int64_t)it.pt * MS;  // GEMM2: the tile's first slot row
  d.xb = a.A + xrow0 * a.a_row_bytes + k0;
  d.wb = a.W + wrow0 * (a.K / 2) + k0 / 2;
  d.xsb = a.A_sf + xrow0 * a.a_sf_row + k0 / 32;
  d.wsb = a.W_sf + wrow0 * (a.K / 32) + k0 / 32;
}

// Per-lane LDS offsets of the fragment and scale reads (swizzled chunks,
// see sources) and of the per-item loads; recomputed for every item from
// an opaque lane id, so that none of them is live across the epilogue.
struct LaneOffs {
  int wo0, wo1, xo0, xo1, xo2, xo3;  // fragment reads
  int sw, sx;                        // scale records of weight tile 0 / slot tile 0 (+ 512 B a tile)
  int sh;                            // 8 h: the byte of block 2 u + h in a stage's word is 2 u + h
  uint32_t p_lane, b_lane;
};

template <int GEMM>
DEV LaneOffs lane_offsets(const MArgs& a, int wave, int lane_) {
  const int lane = opaque(lane_);
  const int ww = wave & 1, ws = wave >> 1;
  const int r = lane & 31, h = lane >> 5;
  LaneOffs L;
  const int wrow = W_OFF + (128 * ww + r) * (MK / 2), wsw = (r >> 2) & 3;
  L.wo0 = wrow + 16 * (h ^ wsw);
  L.wo1 = wrow + 16 * ((2 + h) ^ wsw);
  const int xrow = X_OFF + (128 * ws + r) * MK, xsw = (r >> 1) & 7;
  L.xo0 = xrow + 16 * (h ^ xsw);
  L.xo1 = xrow + 16 * ((2 + h) ^ xsw);
  L.xo2 = xrow + 16 * ((4 + h) ^ xsw);
  L.xo3 = xrow + 16 * ((6 + h) ^ xsw);
  L.sw = SW_OFF + 16 * (128 * ww + r);
  L.sx = SX_OFF + 16 * (128 * ws + r);
  L.sh = 8 * h;
  // route-id load: position 64 wave + lane holds slot 64 wave + 8 (lane & 7)
  // + (lane >> 3); bias load: value 64 wave + lane (GEMM1: gate columns
  // 0..127 of the block, then the up half)
  L.p_lane = 4u * (uint32_t)(64 * wave + 8 * (lane & 7) + (lane >> 3));
  const int bpos = 64 * wave + lane;
  L.b_lane = 4u * (uint32_t)(GEMM == 1 && bpos >= 128 ? a.I + bpos - 128 : bpos);
  return L;
}

// The loads of one stage (the prologue's; the loop interleaves its own).
template <bool BIAS, bool TOPW>
DEV void issue(const MArgs& a, const Dst& d, const Src& s, const WSrc& ws, const LaneOffs& L, uint8_t* smem, int wave,
               bool group) {
#pragma unroll
  for (int j = 0; j < 8; j++) dma16(d.xb + ou(s.x[j]), d.st + X_OFF + 1024 * (8 * wave + j));
#pragma unroll
  for (int j = 0; j < 4; j++) dma16(d.wb + ou(ws.w[j]), d.st + W_OFF + 1024 * (4 * wave + j));
  if constexpr (BIAS) dma4(reinterpret_cast<const uint8_t*>(d.bias) + ou(L.b_lane), d.B + 256 * wave);
  if constexpr (TOPW) dma4(reinterpret_cast<const uint8_t*>(a.topk_w) + ou(s.tw), d.T + 256 * wave);
  if (group) {
    dma4(reinterpret_cast<const uint8_t*>(d.p2e_tile) + ou(L.p_lane), d.P + 256 * wave);
    dma16(d.xsb + ou(s.xs), smem + SX_OFF + 1024 * wave);
    dma16(d.wsb + ou(ws.ws), smem + SW_OFF + 1024 * wave);
  }
}

DEV void read_frag(const uint8_t* st, int wo, int xa, int xb, Frag& f) {
#pragma unroll
  for (int m = 0; m < 4; m++) f.w[m] = *reinterpret_cast<const u32x4_t*>(st + wo + 2048 * m);
#pragma unroll
  for (int n = 0; n < 4; n++) {
    f.x[n][0] = *reinterpret_cast<const u32x4_t*>(st + xa + 4096 * n);
    f.x[n][1] = *reinterpret_cast<const u32x4_t*>(st + xb + 4096 * n);
  }
}

DEV void read_group(const uint8_t* smem, const LaneOffs& L, Group& g) {
#pragma unroll
  for (int m = 0; m < 4; m++) g.w[m] = *reinterpret_cast<const u32x4_t*>(smem + L.sw + 512 * m);
#pragma unroll
  for (int n = 0; n < 4; n++) g.x[n] = *reinterpret_cast<const u32x4_t*>(smem + L.sx + 512 * n);
}

DEV void mfma_one(f32x16_t& acc, const u32x4_t& w, const u32x4_t (&x)[2], int wsc, int xsc) {
  const i32x8_t av = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
  const i32x8_t bv = {(int)x[0][0], (int)x[0][1], (int)x[0][2], (int)x[0][3],
                      (int)x[1][0], (int)x[1][1], (int)x[1][2], (int)x[1][3]};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 0, 0, wsc, 0, xsc);
}

// First half of stage G of a group (K half u = 0): 16 MFMAs on f0.
template <int G>
DEV void first_half(f32x16_t (&acc)[4][4], const Frag& f, const Group& sg, int sh) {
  int ws[4], xs[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    ws[i] = (int)((sg.w[i][G] >> sh) & 255u);
    xs[i] = (int)((sg.x[i][G] >> sh) & 255u);
  }
#pragma unroll
  for (int m = 0; m < 4; m++)
#pragma unroll
    for (int n = 0; n < 4; n++) mfma_one(acc[m][n], f.w[m], f.x[n], ws[m], xs[n]);
}

// Instruction order of a first half for the scheduler (groups: 0x008
// MFMA, 0x100 LDS read): its 12 fragment reads between the first 12 MFMAs.
DEV void order_first_half() {
#pragma unroll
  for (int i = 0; i < 12; i++) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Second half of stage G (K half u = 1), written in issue order: load i of
// the stage, MFMA i on f1, read i of the next stage's first half into f0
// (in the order the next first half uses them) and, at the group's last
// stage, of the next group's scales into sg (this half's scale bytes are
// taken from it before the loop).  READS false: an item's last
// stage leaves them to after the epilogue, which then has their registers.
// (LDS-DMA loads are scheduling boundaries, so the interleave is set here
// rather than left to the scheduler.)
template <int G, int NB, bool BIAS, bool TOPW, bool READS>
DEV void second_half(const MArgs& a, f32x16_t (&acc)[4][4], const Frag& f1, Group& sg, const Dst& d,
                     const Src& s, const WSrc& ws, const LaneOffs& L, uint8_t* smem, int wave, const uint8_t* stn,
                     Frag& f0) {
  constexpr bool GDMA = G == 1;  // this stage loads the next group's scales (and route ids)
  constexpr int ND = NB + (GDMA ? DMA_GROUP : 0);
  constexpr int NR = READS ? 12 + (G == GS - 1 ? 8 : 0) : 0;
  constexpr int X0 = BIAS ? 1 : 0, X1 = X0 + (TOPW ? 1 : 0);
  int wsc[4], xsc[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    wsc[i] = (int)((sg.w[i][G] >> (L.sh + 16)) & 255u);
    xsc[i] = (int)((sg.x[i][G] >> (L.sh + 16)) & 255u);
  }
#pragma unroll
  for (int i = 0; i < 20; i++) {
    if (i < ND) {
      // (offsets through opaque(): a zero-extension hoisted out of the loop
      // would hold each offset in two registers and lose the scalar-base form)
      if (i < 8) dma16(d.xb + ou(s.x[i]), d.st + X_OFF + 1024 * (8 * wave + i));
      else if (i < 12) dma16(d.wb + ou(ws.w[i - 8]), d.st + W_OFF + 1024 * (4 * wave + i - 8));
      else if (BIAS && i - 12 == 0) dma4(reinterpret_cast<const uint8_t*>(d.bias) + ou(L.b_lane), d.B + 256 * wave);
      else if (TOPW && i - 12 == X0) dma4(reinterpret_cast<const uint8_t*>(a.topk_w) + ou(s.tw), d.T + 256 * wave);
      else if (GDMA && i - 12 == X1) dma4(reinterpret_cast<const uint8_t*>(d.p2e_tile) + ou(L.p_lane), d.P + 256 * wave);
      else if (GDMA && i - 12 == X1 + 1) dma16(d.xsb + ou(s.xs), smem + SX_OFF + 1024 * wave);
      else if (GDMA && i - 12 == X1 + 2) dma16(d.wsb + ou(ws.ws), smem + SW_OFF + 1024 * wave);
    }
    if (i < 16) mfma_one(acc[i >> 2][i & 3], f1.w[i >> 2], f1.x[i & 3], wsc[i >> 2], xsc[i & 3]);
    if (i < NR) {
      if (i == 0) f0.w[0] = *reinterpret_cast<const u32x4_t*>(stn + L.wo0);
      else if (i < 9) {
        const int n = (i - 1) >> 1, piece = (i - 1) & 1;
        f0.x[n][piece] = *reinterpret_cast<const u32x4_t*>(stn + (piece ? L.xo1 : L.xo0) + 4096 * n);
      } else if (i < 12) f0.w[i - 8] = *reinterpret_cast<const u32x4_t*>(stn + L.wo0 + 2048 * (i - 8));
      else if (i < 16) sg.w[i - 12] = *reinterpret_cast<const u32x4_t*>(smem + L.sw + 512 * (i - 12));
      else sg.x[i - 16] = *reinterpret_cast<const u32x4_t*>(smem + L.sx + 512 * (i - 16));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// SwiGLU of one gate/up pair with the hardware exp2 and reciprocal (a few
// fp32 ulps, against the MFMA's own accumulation error of about 2^-21 of
// the sum): min(g, l) * sigmoid(alpha * min(g, l)) * (clamp(u, -l, l) + beta).
DEV float swiglu_fast(float g, float u, const GateAct& p) {
  const float gc = fminf(g, p.limit);
  const float uc = fminf(fmaxf(u, -p.limit), p.limit);
  const float e = __builtin_amdgcn_exp2f(-p.alpha * 1.4426950408889634f * gc);
  return gc * __builtin_amdgcn_rcpf(1.0f + e) * (uc + p.beta);
}

template <int AK>
DEV float act_value(float g, float u, const GateAct& p) {
  if constexpr (AK == ACT_SWIGLU) return swiglu_fast(g, u, p);
  else return gated_act_k<AK>(g, u, p);
}

DEV float bf16_round(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// 16 consecutive fp32 values from LDS
DEV void lds16(const uint8_t* p, float (&v)[16]) {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const u32x4_t q = reinterpret_cast<const u32x4_t*>(p)[k];
#pragma unroll
    for (int i = 0; i < 4; i++) v[4 * k + i] = __uint_as_float(q[i]);
  }
}

// One 32-column MXFP8 block of a y1 row: this lane holds 16 consecutive
// columns (from `col`), lane ^ 32 the other 16.  The block max decides the
// E8M0 code; values are clamped to the code's E4M3 range and converted in
// fours; half h = 0 writes the scale byte.
DEV void put_block16(const MArgs& a, const float (&y)[16], int64_t yrow, int col, bool ok, int h) {
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) am = fmaxf(am, fabsf(y[j]));
  am = fmaxf(am, __shfl_xor(am, 32));
  const uint32_t code = mx_scale_code(am, 8);
  const float lim = __builtin_ldexpf(448.0f, (int)code - 127);
  const float sc = e8m0_scale_operand(code);
  u32x4_t q;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = fminf(fmaxf(y[4 * k + i], -lim), lim);
    i16x2_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v[0], v[1], sc, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v[2], v[3], sc, true);
    q[k] = __builtin_bit_cast(uint32_t, r);
  }
  if (ok) {
    uint8_t* Yq = reinterpret_cast<uint8_t*>(a.Y);
    *reinterpret_cast<u32x4_t*>(Yq + yrow * a.n_out + col) = q;
    if (h == 0) a.Y_sf[yrow * (a.n_out / 32) + col / 32] = (uint8_t)code;
  }
}

// GEMM1 epilogue; Bv: the item's bias (gate columns, then up columns)
template <int AK, bool BIAS>
DEV void epilogue1(const MArgs& a, const f32x16_t (&acc)[4][4], const Item& it, const uint8_t* Bv, int ww, int ws,
                   int lane_) {
  const int lane = opaque(lane_);
  const int r = lane & 31, h = lane >> 5;
  const float alpha = ld_uniform(a.alpha + it.e);
  const float alpha_u = a.alpha_up ? ld_uniform(a.alpha_up + it.e) : alpha;
#pragma unroll
  for (int m = 0; m < 2; m++) {
    const int lc = 64 * ww + 32 * m + 16 * h;  // this lane's first column inside the block
    const int col = it.nb * 128 + lc;
    float bg[16], bu[16];
    if constexpr (BIAS) {
      lds16(Bv + 4 * lc, bg);
      lds16(Bv + 4 * (128 + lc), bu);
    }
#pragma unroll
    for (int n = 0; n < 4; n++) {
      const int slot = 128 * ws + 32 * n + r;
      const bool ok = slot < it.valid;
      const int64_t yrow = (int64_t)it.pt * MS + slot;
      float y[16], z[16];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        float g = acc[m][n][j] * alpha;
        float u = acc[m + 2][n][j] * alpha_u;
        if constexpr (BIAS) {
          g = g + bg[j];
          u = u + bu[j];
        }
        // y1 is rounded once to bf16; requantisation starts from that value
        if constexpr (AK == ACT_RELU2) {
          y[j] = bf16_round(relu2_f32(g));
          z[j] = bf16_round(relu2_f32(u));
        } else {
          y[j] = bf16_round(act_value<AK>(g, u, a.act));
        }
      }
      put_block16(a, y, yrow, col, ok, h);
      if constexpr (AK == ACT_RELU2) put_block16(a, z, yrow, a.I + col, ok, h);
      // one block at a time: keeps the accumulator reads from being hoisted
      // in bulk into registers the fragments hold
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// GEMM2 epilogue; P, Bv, Tw: the item's route ids, bias, routing weights
template <bool ATOMIC, bool BIAS>
DEV void epilogue2(const MArgs& a, const f32x16_t (&acc)[4][4], const Item& it, const uint8_t* P, const uint8_t* Bv,
                   const uint8_t* Tw, int ww, int ws, int lane_) {
  const int lane = opaque(lane_);
  const int r = lane & 31, h = lane >> 5;
  const float alpha = ld_uniform(a.alpha + it.e);
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const int lc = 128 * ww + 32 * m + 16 * h;
    const int col = it.nb * MN + lc;
    float bv[16];
    if constexpr (BIAS) lds16(Bv + 4 * lc, bv);
#pragma unroll
    for (int n = 0; n < 4; n++) {
      const int slot = 128 * ws + 32 * n + r;
      const bool ok = slot < it.valid;
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        v[j] = acc[m][n][j] * alpha;
        if constexpr (BIAS) v[j] = v[j] + bv[j];
      }
      if constexpr (!ATOMIC) {
        u32x4_t lo, hi;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          lo[k] = (uint32_t)f32_to_bf16(v[2 * k]) | ((uint32_t)f32_to_bf16(v[2 * k + 1]) << 16);
          hi[k] = (uint32_t)f32_to_bf16(v[8 + 2 * k]) | ((uint32_t)f32_to_bf16(v[8 + 2 * k + 1]) << 16);
        }
        if (ok) {
          uint16_t* Y = reinterpret_cast<uint16_t*>(a.Y) + ((int64_t)it.pt * MS + slot) * a.n_out + col;
          reinterpret_cast<u32x4_t*>(Y)[0] = lo;
          reinterpret_cast<u32x4_t*>(Y)[1] = hi;
        }
      } else {
        const int32_t route = ok ? *reinterpret_cast<const int32_t*>(P + 4 * p_word(slot)) : -1;
        if (route >= 0) {
          const float wf = __fmul_rn(*reinterpret_cast<const float*>(Tw + 4 * slot), a.rsf);
          uint16_t* o = a.out + (int64_t)(route / a.top_k) * a.n_out + col;
#pragma unroll
          for (int k = 0; k < 8; k++) {
            const float c0 = __fmul_rn(wf, bf16_round(v[2 * k]));
            const float c1 = __fmul_rn(wf, bf16_round(v[2 * k + 1]));
            bf16x2_t v2 = {(__bf16)c0, (__bf16)c1};
            __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<bf16x2_t*>(o + 2 * k), v2);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int GEMM, bool ATOMIC, int AK, bool BIAS>
__global__ __launch_bounds__(MT, 1) void mxw_gemm_kernel(const MArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr bool TOPW = GEMM == 2 && ATOMIC;
  constexpr int NB = dma_base<BIAS, TOPW>();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ww = wave & 1, ws = wave >> 1;
  const int KT = a.K / MK;

  // A persistent grid: KB workgroups per XCD, workgroup b on XCD b & 7
  // (workgroups are dealt to the XCDs round-robin).  Tiles go in groups of
  // GT consecutive plan tiles, group g to XCD g & 7.  An XCD's workgroups
  // take its items in order, and a group's items are ordered in passes of
  // KB / GT weight-row blocks, the GT tiles' items of one block next to each
  // other: the KB concurrent items of an XCD then share each weight block
  // among GT tiles and each tile's activation rows among KB / GT weight
  // blocks, in that XCD's L2.
  const int T = ld_uniform(a.num_tiles);
  const int xcd = blockIdx.x & 7;
  const int KB = gridDim.x >> 3;
  const int G = (T + GT - 1) / GT;
  const int per_group = GT * a.n_blocks;
  const int pw = max(1, min(a.n_blocks, KB / GT));
  // first item at or after position j of this XCD's sequence; -1: none
  auto find = [&](int j, int& pt, int& nb) -> int {
    for (;; j += KB) {
      const int g = xcd + 8 * (j / per_group);
      if (g >= G) return -1;
      const int idx = j % per_group;
      const int in = idx % (GT * pw);
      nb = (idx / (GT * pw)) * pw + in / GT;
      pt = GT * g + in % GT;
      if (pt < T && nb < a.n_blocks) return j;
    }
  };
  // the item's 256 bias values: GEMM1 128 gate then 128 up columns of its
  // block, GEMM2 its 256 output columns
  auto bias_of = [&](const Item& it) -> const float* {
    if constexpr (GEMM == 1) return a.bias + (int64_t)it.e * 2 * a.I + it.nb * 128;
    return a.bias + (int64_t)it.e * a.n_out + it.nb * MN;
  };

  int cpt = 0, cnb = 0;
  int cj = find(blockIdx.x >> 3, cpt, cnb);
  if (cj < 0) return;
  Item cur = load_item(a, cpt, cnb);
  int npt = cpt, nnb = cnb;
  int nj = find(cj + KB, npt, nnb);
  Item nxt = nj >= 0 ? load_item(a, npt, nnb) : cur;

  auto Pb = [&](int i) -> uint8_t* { return smem + P_OFF + i * 1024; };
  auto Bb = [&](int i) -> uint8_t* { return smem + B_OFF + i * 1024; };
  auto Tb = [&](int i) -> uint8_t* { return smem + T_OFF + i * 1024; };
  int pb = 0;

  // route ids (and bias) of the first item, then its sources
  LaneOffs L = lane_offsets<GEMM>(a, wave, lane);
  dma4(reinterpret_cast<const uint8_t*>(a.p2e + (int64_t)cur.pt * MS) + ou(L.p_lane), Pb(0) + 256 * wave);
  if constexpr (BIAS) dma4(reinterpret_cast<const uint8_t*>(bias_of(cur)) + ou(L.b_lane), Bb(0) + 256 * wave);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  ring_barrier();
  Src cs = sources<GEMM, TOPW>(a, cur, Pb(0), wave, lane);
  WSrc wsrc = weight_sources<GEMM>(a, wave, lane);

  // the first three stages (the first with its scale group and the next
  // item's route ids); every stage's loads also refresh the next item's bias
  {
    Dst d;
    d.p2e_tile = a.p2e + (int64_t)nxt.pt * MS;
    d.P = Pb(1);
    d.bias = BIAS ? bias_of(nxt) : nullptr;
    d.B = Bb(1);
    d.T = Tb(0);
#pragma unroll 1
    for (int s = 0; s < NBUF; s++) {
      d.st = smem + s * STAGE;
      stage_bases<GEMM>(a, cur, s * MK, d);
      issue<BIAS, TOPW>(a, d, cs, wsrc, L, smem, wave, s == 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NB));
  ring_barrier();

  Frag f0, f1;
  Group sg;
  f32x16_t acc[4][4];
  int buf = 0;
#pragma unroll 1
  for (;;) {
    // the item's first scale group and the first half of its first stage
    // (visible since the last stage's barrier; their buffers are refilled
    // only after the next barrier)
    L = lane_offsets<GEMM>(a, wave, lane);
    read_group(smem, L, sg);
    read_frag(smem + buf * STAGE, L.wo0, L.xo0, L.xo1, f0);
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
      for (int n = 0; n < 4; n++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[m][n][i] = 0.0f;

    // stage s (G = s % GS) of the item; it loads stage s + 3 of the
    // stream: of this item while SAME, else the next item's
    auto stage = [&](int s, auto G_, auto last_, auto same_) {
      constexpr int Gs = decltype(G_)::value;
      constexpr bool last = decltype(last_)::value, same = decltype(same_)::value;
      uint8_t* st = smem + buf * STAGE;
      const int nbuf = buf == NBUF - 1 ? 0 : buf + 1;
      const uint8_t* stn = smem + nbuf * STAGE;
      // what this stage loads (scalar work, done among the first half's MFMAs)
      Dst d;
      stage_bases<GEMM>(a, same ? cur : nxt, (same ? s + 3 : s + 3 - KT) * MK, d);
      d.st = st;
      d.p2e_tile = a.p2e + (int64_t)nxt.pt * MS;
      d.P = Pb(pb ^ 1);
      d.bias = BIAS ? bias_of(nxt) : nullptr;
      d.B = Bb(pb ^ 1);
      d.T = Tb(same ? pb : pb ^ 1);

      // first half: its fragments are in f0; read the second half's
      read_frag(st, L.wo1, L.xo2, L.xo3, f1);
      first_half<Gs>(acc, f0, sg, L.sh);
      order_first_half();
      __builtin_amdgcn_sched_barrier(0);
      // stage + 1 has landed once only the last stage's loads are in flight
      // (those of stage + 2: NB, and the group's when it starts one)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(NB + (Gs == 2 ? DMA_GROUP : 0)));
      ring_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // every wave is done with this stage's buffer: refill it three stages
      // on; second half, while the next stage's first half is read
      second_half<Gs, NB, BIAS, TOPW, !last>(a, acc, f1, sg, d, cs, wsrc, L, smem, wave, stn, f0);
      buf = nbuf;
    };
    using G0 = std::integral_constant<int, 0>;
    using G1 = std::integral_constant<int, 1>;
    using G2 = std::integral_constant<int, 2>;
    using G3 = std::integral_constant<int, 3>;
    const std::false_type no;
    const std::true_type yes;
#pragma unroll 1
    for (int q = 0; q < KT / GS - 1; q++) {
      stage(GS * q, G0{}, no, yes);
      stage(GS * q + 1, G1{}, no, yes);
      stage(GS * q + 2, G2{}, no, yes);
      stage(GS * q + 3, G3{}, no, yes);
    }
    // the last group: from its second stage on, the loads are the next
    // item's, whose route ids have landed (they went out with this item's
    // second stage, and again with every group since)
    stage(KT - 4, G0{}, no, yes);
    if constexpr (GEMM == 1 || TOPW) {
      __builtin_amdgcn_sched_barrier(0);
      cs = sources<GEMM, TOPW>(a, nxt, Pb(pb ^ 1), wave, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    stage(KT - 3, G1{}, no, no);
    stage(KT - 2, G2{}, no, no);
    stage(KT - 1, G3{}, yes, no);
    // the accumulators are complete here: an MFMA whose result only the
    // epilogue's guarded stores use may not be sunk into them (that would
    // keep its operands live across the epilogue)
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
      for (int n = 0; n < 4; n++) asm volatile("" : "+a"(acc[m][n]));

    if constexpr (GEMM == 1) epilogue1<AK, BIAS>(a, acc, cur, Bb(pb), ww, ws, lane);
    else epilogue2<ATOMIC, BIAS>(a, acc, cur, Pb(pb), Bb(pb), Tb(pb), ww, ws, lane);

    if (nj < 0) break;
    cur = nxt;
    cj = nj;
    pb ^= 1;
    nj = find(cj + KB, npt, nnb);
    if (nj >= 0) nxt = load_item(a, npt, nnb);
  }
  // no LDS-DMA load may still be writing when the workgroup ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

void plan_args(MArgs& a, const moe_plan_t* plan) {
  a.p2e = plan->permuted_to_expanded;
  a.tile_expert = plan->tile_to_expert;
  a.tile_limit = plan->tile_to_mn_limit;
  a.num_tiles = plan->num_tiles;
  a.top_k = plan->top_k;
}

template <int GEMM, bool ATOMIC, int AK, bool BIAS>
hipError_t launch_one(const MArgs& a, int max_tiles, hipStream_t s) {
  auto kern = mxw_gemm_kernel<GEMM, ATOMIC, AK, BIAS>;
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

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
constexpr int64_t OFF_LIMIT = (int64_t)1 << 31;  // the 32-bit lane offsets stay below this

}  // namespace

// 256-slot plan tiles; K a multiple of 512 (whole scale groups) with at
// least MIN_KT stages; whole weight-row blocks; 16-byte aligned rows and
// scale arrays; every source offset inside 31 bits
bool mxw_supported1(const Gemm1Params& p) {
  const int64_t stride = p.x_row_stride ? p.x_row_stride : p.H;
  const int IP = gemm1_pairs(p);
  return p.mode == MOE_QUANT_MXFP8_MXFP4 && p.plan->tile == MS && p.H % (MK * GS) == 0 && p.H / MK >= MIN_KT &&
         IP % 128 == 0 && stride % 16 == 0 && ((uintptr_t)p.x & 15) == 0 && aligned16(p.x_sf) &&
         aligned16(p.w1_sf) && ((uintptr_t)p.y1 & 15) == 0 && ((uintptr_t)p.w1 & 15) == 0 &&
         (int64_t)p.plan->M * stride < OFF_LIMIT && (int64_t)2 * IP * (p.H / 2) < OFF_LIMIT;
}
bool mxw_supported2(const Gemm2Params& p) {
  return p.mode == MOE_QUANT_MXFP8_MXFP4 && p.plan->tile == MS && p.I % (MK * GS) == 0 && p.I / MK >= MIN_KT &&
         p.H % MN == 0 && ((uintptr_t)p.y1 & 15) == 0 && aligned16(p.y1_sf) && aligned16(p.w2_sf) &&
         ((uintptr_t)p.w2 & 15) == 0 && (!p.y2 || ((uintptr_t)p.y2 & 15) == 0) &&
         p.plan->route_slots * p.I < OFF_LIMIT && (int64_t)p.H * (p.I / 2) < OFF_LIMIT;
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
  if (p.fc1_bias) {
    switch (p.act.kind) {
      case ACT_GEGLU_TANH: return launch_one<1, false, ACT_GEGLU_TANH, true>(a, mt, stream);
      case ACT_SITU: return launch_one<1, false, ACT_SITU, true>(a, mt, stream);
      case ACT_RELU2: return launch_one<1, false, ACT_RELU2, true>(a, mt, stream);
      default: return launch_one<1, false, ACT_SWIGLU, true>(a, mt, stream);
    }
  }
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
