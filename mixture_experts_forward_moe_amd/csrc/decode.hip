// decode.hip -- the W4A16 forward for decode-sized batches in two launches.
//
// At decode sizes (a route or two per active expert) the pass is bound by
// HBM bandwidth on weight bytes: each weight byte meets one or two
// activation rows.
//
//  dec_gemm1: every workgroup builds the batch's routing plan in LDS
//    (per-expert counts, 16-slot tiles, stable slots in route order: the
//    plan moe_sort builds, so there is no separate sort launch), picks its
//    tiles, stages the tile's token rows of x in LDS and streams 32 gate +
//    32 up weight rows of the tile's expert in two passes of 16 (expert
//    scale, SwiGLU, bf16 y1).  Its first weight loads go out as soon as the
//    tile's expert is known, before the slots and x are.  Workgroup (0, 0)
//    writes the plan out.
//  dec_gemm2: reads that plan; a workgroup streams 64 rows of W2 for a tile
//    against the tile's y1 rows and writes y2.  The last workgroup of a
//    column group applies the deterministic route-order finalize to those
//    64 columns ("flashinfer.fused_moe.alphamoe_nvfp4_routed_moe", summary:
//    contributions in route order, seeded from the output).
//
// (A single persistent launch with per-tile ready counts measured slower on
// the decode workload: 49.6 against 45.5 us per forward in graph replay.)
//
// Inner product without matrix cores: lane (rr, ch) owns weight row rr of
// its wavefront's four and the 16-byte chunks ch, ch+16, ... of that row
// (32 codes, two E4M3 blocks each).  Codes become bf16 pairs with
// v_cvt_scalef32_pk_bf16_fp4 (scale 1: exact E2M1 values), v_dot2_f32_bf16
// multiplies them with bf16 activation pairs read from LDS, and each
// block's partial sum is multiplied by its decoded scale
// (v_cvt_f32_fp8): about one VALU instruction per weight element and
// activation row, where a decode to scaled bf16 costs two.  The 16 chunk
// lanes of a row reduce with a fixed xor tree, so results are reproducible.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace moe {

// A workgroup barrier that orders LDS accesses only: global loads and
// stores in flight stay in flight (a full __syncthreads waits for all of
// them, which would drain the weight stream at every barrier).
DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int DEC_THREADS = 256;
constexpr int DEC_ROWS = 1;        // activation rows per pass
constexpr int DEC_TILE_STRIDE = 8; // workgroups per column group, looping over tiles

constexpr int DEC_T = 16;          // plan tile
constexpr int G1_NP = 2;           // GEMM1 passes of 16 columns per workgroup
constexpr int G1_D = 4;            // GEMM1 K-steps in flight per lane

struct DecArgs {
  const int32_t* ids;
  int M, top_k, El, offset;
  const uint16_t* x;
  int64_t x_row_stride;  // elements
  const uint8_t* w1;
  const uint8_t* w1_sf;
  const float* w1_alpha;
  const float* w1_alpha_up;  // NULL: w1_alpha for the up half too
  const float* fc1_bias;     // NULL, or fp32 [El, 2I]
  const float* fc2_bias;     // NULL, or fp32 [El, H]
  const uint8_t* w2;
  const uint8_t* w2_sf;
  const float* w2_alpha;
  int H, I;
  int ip;                // W1 row pairs per expert: I (gated), I/2 (ReLU^2: rows j, I/2 + j)
  GateAct act;          // FC1 activation
  uint16_t* y1;          // [slots, I]
  uint16_t* y2;          // [slots, H]
  int* counters;         // the decode counter block: one done count per 64 columns, zero between calls
  const float* topk_w;
  float rsf;
  int accumulate;
  int zero_out;          // GEMM1 clears out (the atomic finalize adds into it)
  uint16_t* out;
  // plan arrays written by dec_gemm1's first workgroup
  int32_t *e2p, *p2e, *tile_expert, *tile_limit, *num_tiles, *offsets, *counts;
  int64_t slots;
  int max_tiles;
};

struct LocalPlan {
  int* cnt;    // [El]
  int* tbase;  // [El+1] first tile of each expert; [El] = tiles in use
  int* run;    // [El]
  int* e2p;    // [R]
  int* tmp;    // [DEC_THREADS / 64]
};

DEV int dec_local(const DecArgs& a, const int* ids, int r) {
  const int id = ids[r];
  const int le = id - a.offset;
  return (id >= a.offset && le < a.El) ? le : -1;
}

// exclusive scan of v[0..n) in LDS by the whole workgroup; returns the total
DEV int dec_scan(int* v, int n, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + DEC_THREADS - 1) / DEC_THREADS;
  const int lo = tid * per;
  int s = 0;
  for (int i = 0; i < per; i++)
    if (lo + i < n) s += v[lo + i];
  int x = s;
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < DEC_THREADS / 64; w++) {
    if (w < wave) base += tmp[w];
    total += tmp[w];
  }
  int run = base + x - s;
  for (int i = 0; i < per; i++)
    if (lo + i < n) {
      int c = v[lo + i];
      v[lo + i] = run;
      run += c;
    }
  __syncthreads();
  return total;
}

// The batch's plan in LDS, in two parts.  plan_counts: per-expert counts and
// tile bases (slots of expert e start at 16 * tbase[e]), which is all a
// workgroup needs to find its tile's expert; it leaves the route ids in
// e2p.  plan_slots: every route's slot, in ascending route order within its
// expert.
DEV int plan_counts(const DecArgs& a, const LocalPlan& P) {
  const int R = a.M * a.top_k;
  const int tid = threadIdx.x;
  for (int e = tid; e < a.El; e += DEC_THREADS) P.cnt[e] = 0;
  for (int r = tid; r < R; r += DEC_THREADS) P.e2p[r] = a.ids[r];  // ids first, slots later
  __syncthreads();
  for (int r = tid; r < R; r += DEC_THREADS) {
    const int le = dec_local(a, P.e2p, r);
    if (le >= 0) atomicAdd(&P.cnt[le], 1);
  }
  __syncthreads();
  for (int e = tid; e < a.El; e += DEC_THREADS) P.tbase[e] = (P.cnt[e] + DEC_T - 1) / DEC_T;
  __syncthreads();
  const int nt = dec_scan(P.tbase, a.El, P.tmp);
  if (tid == 0) P.tbase[a.El] = nt;
  for (int e = tid; e < a.El; e += DEC_THREADS) P.run[e] = P.tbase[e] * DEC_T;
  __syncthreads();
  return nt;
}

// stable slots: wavefront 0 walks the routes 64 at a time
DEV void plan_slots(const DecArgs& a, const LocalPlan& P) {
  const int R = a.M * a.top_k;
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int nbits = 0;
    while ((1 << nbits) <= a.El) nbits++;
    for (int r0 = 0; r0 < R; r0 += 64) {
      const int r = r0 + lane;
      const int le = r < R ? dec_local(a, P.e2p, r) : -1;
      const int key = le < 0 ? a.El : le;
      uint64_t m = ~0ull;
      for (int b = 0; b < nbits; b++) {
        const int bit = (key >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      const int rank = __popcll(m & below);
      int slot = -1;
      if (le >= 0) slot = P.run[le] + rank;
      if (r < R) P.e2p[r] = slot;
      // the highest-ranked lane of each expert advances its counter
      if (le >= 0 && rank == __popcll(m) - 1) P.run[le] = slot + 1;
    }
  }
  __syncthreads();
}

// expert of tile pt: the last expert whose first tile is <= pt
DEV int tile_owner(const LocalPlan& P, int El, int pt) {
  int lo = 0, hi = El - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (P.tbase[mid] <= pt) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// one K-step of one weight row for one lane: 32 codes + two scale codes.
// The two scale bytes of chunk kc sit at byte 2 kc of the row's scales;
// the lane loads the aligned 32-bit word holding them (kc and kc ^ 1
// share it) and dot_chunk shifts the pair down for odd kc.  A 16-bit load
// would need a zero-extension that the compiler may place where it has to
// wait for every load in flight.  The scale rows must be 4-byte aligned.
struct Chunk {
  u32x4_t w;
  uint32_t s;
};

DEV Chunk load_chunk(const uint8_t* W, const uint8_t* Wsf, int64_t row, int K, int kc) {
  Chunk c;
  c.w = *reinterpret_cast<const u32x4_t*>(W + row * (K / 2) + (int64_t)kc * 16);
  c.s = *reinterpret_cast<const uint32_t*>(Wsf + row * (K / 16) + (int64_t)(kc & ~1) * 2);
  return c;
}

DEV uint32_t chunk_scales(const Chunk& c, int kc) { return c.s >> (16 * (kc & 1)); }

// two E2M1 codes (byte B of w) as a bf16 pair, exact
template <int B>
DEV uint32_t e2m1x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}

// acc[t] += sum over the chunk's 32 elements of x_t * w, blockwise scaled
template <int NR>
DEV void dot_chunk(const Chunk& c, const uint32_t* xs, int x_stride_words, int kc, float* acc) {
  uint32_t wb[16];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    wb[4 * j + 0] = e2m1x2_bf16<0>(c.w[j]);
    wb[4 * j + 1] = e2m1x2_bf16<1>(c.w[j]);
    wb[4 * j + 2] = e2m1x2_bf16<2>(c.w[j]);
    wb[4 * j + 3] = e2m1x2_bf16<3>(c.w[j]);
  }
  const int sc = (int)chunk_scales(c, kc);
  const float s0 = __builtin_amdgcn_cvt_f32_fp8(sc, 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8(sc, 1);
#pragma unroll
  for (int t = 0; t < NR; t++) {
    // activation pairs as scalars (bit-casting an element of a vector
    // register in place is not reliable, so copy the words out first)
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(xs + t * x_stride_words + kc * 16);
    uint32_t xw[16];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u32x4_t v = xr[j];
      xw[4 * j + 0] = v.x;
      xw[4 * j + 1] = v.y;
      xw[4 * j + 2] = v.z;
      xw[4 * j + 3] = v.w;
    }
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
      p0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw[i]), __builtin_bit_cast(bf16x2_t, wb[i]),
                                           p0, false);
#pragma unroll
    for (int i = 8; i < 16; i++)
      p1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw[i]), __builtin_bit_cast(bf16x2_t, wb[i]),
                                           p1, false);
    acc[t] = acc[t] + s0 * p0;
    acc[t] = acc[t] + s1 * p1;
  }
}

// gate and up chunks of the same K range against the same activations:
// each activation word is read from LDS once for both rows
template <int NR>
DEV void dot_chunk2(const Chunk& cg, const Chunk& cu, const uint32_t* xs, int x_stride_words, int kc, float* ag,
                    float* au) {
  uint32_t wg[16], wu[16];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    wg[4 * j + 0] = e2m1x2_bf16<0>(cg.w[j]);
    wg[4 * j + 1] = e2m1x2_bf16<1>(cg.w[j]);
    wg[4 * j + 2] = e2m1x2_bf16<2>(cg.w[j]);
    wg[4 * j + 3] = e2m1x2_bf16<3>(cg.w[j]);
    wu[4 * j + 0] = e2m1x2_bf16<0>(cu.w[j]);
    wu[4 * j + 1] = e2m1x2_bf16<1>(cu.w[j]);
    wu[4 * j + 2] = e2m1x2_bf16<2>(cu.w[j]);
    wu[4 * j + 3] = e2m1x2_bf16<3>(cu.w[j]);
  }
  const int gs = (int)chunk_scales(cg, kc), us = (int)chunk_scales(cu, kc);
  const float g0 = __builtin_amdgcn_cvt_f32_fp8(gs, 0), g1 = __builtin_amdgcn_cvt_f32_fp8(gs, 1);
  const float u0 = __builtin_amdgcn_cvt_f32_fp8(us, 0), u1 = __builtin_amdgcn_cvt_f32_fp8(us, 1);
#pragma unroll
  for (int t = 0; t < NR; t++) {
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(xs + t * x_stride_words + kc * 16);
    float pg0 = 0.0f, pg1 = 0.0f, pu0 = 0.0f, pu1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u32x4_t v = xr[j];
      const uint32_t xw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xw[b]);
        if (j < 2) {
          pg0 = __builtin_amdgcn_fdot2_f32_bf16(xp, __builtin_bit_cast(bf16x2_t, wg[4 * j + b]), pg0, false);
          pu0 = __builtin_amdgcn_fdot2_f32_bf16(xp, __builtin_bit_cast(bf16x2_t, wu[4 * j + b]), pu0, false);
        } else {
          pg1 = __builtin_amdgcn_fdot2_f32_bf16(xp, __builtin_bit_cast(bf16x2_t, wg[4 * j + b]), pg1, false);
          pu1 = __builtin_amdgcn_fdot2_f32_bf16(xp, __builtin_bit_cast(bf16x2_t, wu[4 * j + b]), pu1, false);
        }
      }
    }
    ag[t] = ag[t] + g0 * pg0;
    ag[t] = ag[t] + g1 * pg1;
    au[t] = au[t] + u0 * pu0;
    au[t] = au[t] + u1 * pu1;
  }
}

DEV float sum16(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

// GEMM1's stream: a lane's gate and up rows g, u (pass 0), then g + 16,
// u + 16 (pass 1), over its chunks of K.  D K-steps of loads stay in flight
// and the caller issues the first D before staging the activations, so
// their latency overlaps the staging; pass 0's last D loads are pass 1's
// first steps.  Every load in the loop is unconditional (D divides the
// step count), so the compiler waits only for the step it is about to use.
template <int D>
DEV void prefetch_pairs(const uint8_t* W, const uint8_t* Wsf, int64_t g, int64_t u, int K, int ch, Chunk* bg,
                        Chunk* bu) {
#pragma unroll
  for (int d = 0; d < D; d++) {
    bg[d] = load_chunk(W, Wsf, g, K, ch + 16 * d);
    bu[d] = load_chunk(W, Wsf, u, K, ch + 16 * d);
    __builtin_amdgcn_sched_barrier(0);  // issue in the stream loop's order
  }
}

template <int D, int NP>
DEV void stream_pairs(const uint8_t* W, const uint8_t* Wsf, int64_t g, int64_t u, int K, int ch,
                      const uint32_t* xs, Chunk* bg, Chunk* bu, float* ag, float* au) {
  const int NS = K / 512;  // a multiple of D
#pragma unroll
  for (int p = 0; p < NP; p++) {
    const int64_t gp = g + 16 * p, up = u + 16 * p;
    const int end = p + 1 < NP ? NS : NS - D;  // the last pass's last D steps load nothing
    for (int s0 = 0; s0 < end; s0 += D) {
#pragma unroll
      for (int d = 0; d < D; d++) {
        dot_chunk2<1>(bg[d], bu[d], xs, 0, ch + 16 * (s0 + d), &ag[p], &au[p]);
        const int sn = s0 + d + D;
        const bool wrap = sn >= NS;  // not the last pass: the next loads are the next pass's
        const int kn = ch + 16 * (wrap ? sn - NS : sn);
        bg[d] = load_chunk(W, Wsf, wrap ? gp + 16 : gp, K, kn);
        bu[d] = load_chunk(W, Wsf, wrap ? up + 16 : up, K, kn);
        __builtin_amdgcn_sched_barrier(0);  // keep one step's values live at a time
      }
    }
  }
#pragma unroll
  for (int d = 0; d < D; d++)
    dot_chunk2<1>(bg[d], bu[d], xs, 0, ch + 16 * (NS - D + d), &ag[NP - 1], &au[NP - 1]);
}

// GEMM2's done count of column group c (64 columns of H)
DEV int* done_count(const DecArgs& a, int c) { return a.counters + DEC_CTR_SLOT * c; }

// ---------------------------------------------------------------- GEMM1

// Workgroup (bx, y) computes y1 columns 32 bx .. 32 bx + 31 (16 per pass)
// of tiles y, y + gridDim.y, ...; wavefront w, lane (rr, ch) owns column
// 32 bx + 16 p + 4 w + rr of pass p.
template <int D, int NP, int AK>
__global__ __launch_bounds__(DEC_THREADS) void dec_gemm1_kernel(const DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dsm[];
  const int R = a.M * a.top_k;
  LocalPlan P;
  P.cnt = (int*)dsm;
  P.tbase = P.cnt + a.El;
  P.run = P.tbase + a.El + 1;
  P.tmp = P.run + a.El;
  P.e2p = P.tmp + DEC_THREADS / 64;
  int* rows = P.e2p + R;  // [16] routes of this tile
  // the x row at the next 16-byte boundary; offset arithmetic on the LDS
  // array itself (an integer round trip would turn every read into a flat
  // load, and flat loads make each step wait for all weight loads in flight)
  const int xs_word = (3 * a.El + 1 + DEC_THREADS / 64 + R + DEC_T + 3) & ~3;
  uint32_t* xs = dsm + xs_word;  // [H/2]

  // GEMM2 of this forward counts finished workgroups per column group from
  // zero; it runs after this launch in the same stream
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int c = threadIdx.x; c < a.H / 64; c += DEC_THREADS)
      __hip_atomic_store(done_count(a, c), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the atomic finalize of GEMM2 adds into out: clear it here, 16 bytes a
  // thread over the whole grid (out is not read by this launch)
  if (a.zero_out) {
    const int64_t n16 = (int64_t)a.M * a.H / 8;
    const int64_t nthr = (int64_t)gridDim.x * gridDim.y * DEC_THREADS;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * DEC_THREADS + threadIdx.x; i < n16; i += nthr)
      reinterpret_cast<u32x4_t*>(a.out)[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
  const int nt = plan_counts(a, P);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane >> 4, ch = lane & 15;
  const int col = 16 * NP * blockIdx.x + 4 * wave + rr;
  bool slots_done = false;

  for (int pt = blockIdx.y; pt < nt; pt += gridDim.y) {
    const int e = tile_owner(P, a.El, pt);
    const int slot0 = pt * DEC_T;
    const int valid = min(DEC_T, P.tbase[e] * DEC_T + P.cnt[e] - slot0);
    const int64_t rg = (int64_t)e * 2 * a.ip + col;
    const int64_t ru = rg + a.ip;
    const float al = a.w1_alpha[e];
    const float alu = a.w1_alpha_up ? a.w1_alpha_up[e] : al;
    for (int r0 = 0; r0 < valid; r0++) {
      Chunk bg[D], bu[D];
      prefetch_pairs<D>(a.w1, a.w1_sf, rg, ru, a.H, ch, bg, bu);
      if (!slots_done) {
        plan_slots(a, P);
        slots_done = true;
      }
      if (r0 == 0) {
        if (tid < DEC_T) rows[tid] = -1;
        __syncthreads();
        for (int r = tid; r < R; r += DEC_THREADS) {
          const int s = P.e2p[r];
          if (s >= slot0 && s < slot0 + DEC_T) rows[s - slot0] = r;
        }
        __syncthreads();
      }
      // stage the route's token row of x
      {
        const int64_t tok = rows[r0] / a.top_k;
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.x + tok * a.x_row_stride);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(xs);
        for (int i = tid; i < a.H / 8; i += DEC_THREADS) dst[i] = src[i];
      }
      __syncthreads();
      float ag[NP] = {}, au[NP] = {};
      stream_pairs<D, NP>(a.w1, a.w1_sf, rg, ru, a.H, ch, xs, bg, bu, ag, au);
#pragma unroll
      for (int p = 0; p < NP; p++) {
        const float g = sum16(ag[p]);
        const float u = sum16(au[p]);
        if (ch == 0) {
          float gs = g * al, us = u * alu;
          if (a.fc1_bias) {
            gs = gs + a.fc1_bias[(int64_t)e * 2 * a.ip + col + 16 * p];
            us = us + a.fc1_bias[(int64_t)e * 2 * a.ip + a.ip + col + 16 * p];
          }
          uint16_t* yrow = a.y1 + (int64_t)(slot0 + r0) * a.I;
          if constexpr (AK == ACT_RELU2) {  // non-gated: both rows are outputs
            yrow[col + 16 * p] = f32_to_bf16(relu2_f32(gs));
            yrow[a.ip + col + 16 * p] = f32_to_bf16(relu2_f32(us));
          } else {
            yrow[col + 16 * p] = f32_to_bf16(gated_act_k<AK>(gs, us, a.act));
          }
        }
      }
      __syncthreads();
    }
  }
  if (!slots_done) plan_slots(a, P);

  if (blockIdx.x == 0 && blockIdx.y == 0) {
    // the plan, for the record and for GEMM2
    for (int r = tid; r < R; r += DEC_THREADS) a.e2p[r] = P.e2p[r];
    for (int64_t s = tid; s < a.slots; s += DEC_THREADS) a.p2e[s] = -1;
    for (int i = tid; i < a.max_tiles; i += DEC_THREADS) {
      int te = -1, tl = -1;
      if (i < nt) {
        te = tile_owner(P, a.El, i);
        tl = min((i + 1) * DEC_T, P.tbase[te] * DEC_T + P.cnt[te]);
      }
      a.tile_expert[i] = te;
      a.tile_limit[i] = tl;
    }
    for (int e = tid; e < a.El; e += DEC_THREADS) {
      a.offsets[e] = P.tbase[e] * DEC_T;
      a.counts[e] = P.cnt[e];
    }
    if (tid == 0) {
      a.offsets[a.El] = nt * DEC_T;
      *a.num_tiles = nt;
    }
    __syncthreads();
    for (int r = tid; r < R; r += DEC_THREADS)
      if (P.e2p[r] >= 0) a.p2e[P.e2p[r]] = r;
  }
}

// ---------------------------------------------------------------- GEMM2

// One lane's share of 16 rows x K: rows 4g + rr (g = 0..3), chunks ch + 16 s.
// The four row groups are streamed interleaved (flattened index f: group
// f % 4, step f / 4) so that all their loads are in flight together; D
// divides the 4 * K/512 flattened steps and every load in the loop is
// unconditional.  The caller issues the first D loads (prefetch16) before
// staging the activations.
template <int D>
DEV void prefetch16(const uint8_t* W, const uint8_t* Wsf, int64_t row0, int K, int ch, Chunk* b) {
#pragma unroll
  for (int d = 0; d < D; d++) {
    b[d] = load_chunk(W, Wsf, row0 + 4 * (d & 3), K, ch + 16 * (d >> 2));
    __builtin_amdgcn_sched_barrier(0);  // issue in the stream loop's order
  }
}

template <int NR, int D>
DEV void stream_rows16(const uint8_t* W, const uint8_t* Wsf, int64_t row0, int K, int ch, const uint32_t* xs,
                       int xsw, Chunk* b, float (*acc)[DEC_ROWS]) {
  const int total = 4 * (K / 512);
  int f0 = 0;
  for (; f0 + D < total; f0 += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      const int f = f0 + d;
      dot_chunk<NR>(b[d], xs, xsw, ch + 16 * (f >> 2), acc[f & 3]);
      const int fn = f + D;
      b[d] = load_chunk(W, Wsf, row0 + 4 * (fn & 3), K, ch + 16 * (fn >> 2));
      __builtin_amdgcn_sched_barrier(0);  // keep one step's values live at a time
    }
  }
#pragma unroll
  for (int d = 0; d < D; d++) {
    const int f = f0 + d;
    dot_chunk<NR>(b[d], xs, xsw, ch + 16 * (f >> 2), acc[f & 3]);
  }
}

// ---------------------------------------------------------------- finalize in GEMM2
//
// The route-order finalize of a column group needs y2 from every tile, which
// other workgroups compute.  Those go through device-scope stores (they
// bypass the CU's L1 and stay coherent across the L2s of all XCDs); each
// workgroup waits for its stores to complete and then bumps its column
// group's count (cleared by GEMM1 of the same forward), and the workgroup
// that brings the count to the number of workgroups per column group
// finalizes those columns for every token.  Nothing waits on anything, so
// there is no forward-progress condition.  The stores write through to memory, so
// a workgroup gathers a row's 64 outputs in LDS and stores them as one
// 128-byte line from 32 lanes.

DEV void st_dev(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// every wavefront waits for its stores to complete (vmcnt 0), then after the
// barrier thread 0 bumps *c; the previous value goes to thread 0
DEV int publish_bump(int* c) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // keeps the stores above the wait
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0): expcnt and lgkmcnt not waited
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

// out[m, col], out[m, col + 1] in route order, every y2 load of the token
// issued before the sums.  s[j], w[j]: route j's slot (or -1) and weight x
// routed scaling factor, for the first DEC_FJ routes (any further routes
// are read here).
constexpr int DEC_FJ = 8;
DEV void finalize_token(const DecArgs& a, int m, int col, const int* s, const float* w) {
  uint32_t* o = reinterpret_cast<uint32_t*>(a.out + (int64_t)m * a.H + col);
  const uint32_t seed = a.accumulate ? *o : 0u;
  int sj[DEC_FJ];
  uint32_t v[DEC_FJ];
#pragma unroll
  for (int j = 0; j < DEC_FJ; j++) {
    sj[j] = s[j];
    v[j] = sj[j] >= 0 ? ld_dev(reinterpret_cast<const uint32_t*>(a.y2 + (int64_t)sj[j] * a.H + col)) : 0u;
  }
  float acc0 = __uint_as_float(seed << 16), acc1 = __uint_as_float(seed & 0xffff0000u);
#pragma unroll
  for (int j = 0; j < DEC_FJ; j++) {
    if (sj[j] < 0) continue;
    acc0 = acc0 + w[j] * __uint_as_float(v[j] << 16);
    acc1 = acc1 + w[j] * __uint_as_float(v[j] & 0xffff0000u);
  }
  for (int j = DEC_FJ; j < a.top_k; j++) {
    const int r = m * a.top_k + j;
    const int sr = a.e2p[r];
    if (sr < 0) continue;
    const float wf = a.topk_w[r] * a.rsf;
    const uint32_t y = ld_dev(reinterpret_cast<const uint32_t*>(a.y2 + (int64_t)sr * a.H + col));
    acc0 = acc0 + wf * __uint_as_float(y << 16);
    acc1 = acc1 + wf * __uint_as_float(y & 0xffff0000u);
  }
  *o = pack_bf16x2(acc0, acc1);
}

// the first DEC_FJ routes of token m: slots (or -1) and scaled weights
DEV void load_fin_routes(const DecArgs& a, int m, int* s, float* w) {
#pragma unroll
  for (int j = 0; j < DEC_FJ; j++) {
    const bool ok = m < a.M && j < a.top_k;
    const int r = ok ? m * a.top_k + j : 0;
    s[j] = ok ? a.e2p[r] : -1;
    w[j] = a.topk_w[r] * a.rsf;
  }
}

// out[:, c0 : c0 + 64] in route order for every token.  Thread (tt, p) owns
// columns c0 + 2p and c0 + 2p + 1 of tokens tt, tt + 8, ...; the route
// inputs of tokens 0..7 come preloaded in LDS (fs, fw).
DEV void finalize_cols(const DecArgs& a, int c0, const int (*fs)[DEC_FJ], const float (*fw)[DEC_FJ]) {
  const int tid = threadIdx.x;
  const int p = tid & 31, tt = tid >> 5;
  const int col = c0 + 2 * p;
  if (tt < a.M) finalize_token(a, tt, col, fs[tt], fw[tt]);
  for (int m = tt + DEC_THREADS / 32; m < a.M; m += DEC_THREADS / 32) {
    int s[DEC_FJ];
    float w[DEC_FJ];
    load_fin_routes(a, m, s, w);
    finalize_token(a, m, col, s, w);
  }
}

constexpr int DEC_YMAX = 4;  // u32x4 per thread for one y1 row: I <= 8192

// Workgroup (bx, y): y2 columns 64 bx .. 64 bx + 63 of tiles y, y +
// gridDim.y, ...  Per route row: the y1 row goes into registers, the first
// D weight steps are issued, then y1 goes to LDS (waiting for its own loads
// only) and the stream starts.  ATOMIC: each row's 64 outputs, rounded to
// bf16 and times the route's weight x routed_scaling_factor, are added into
// out with packed-bf16 atomics (out cleared by GEMM1 unless accumulating);
// no y2, no count, no finalize.
template <int D, bool ATOMIC>
__global__ __launch_bounds__(DEC_THREADS) void dec_gemm2_kernel(const DecArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t xs[8192 / 2];
  __shared__ uint16_t ybuf[64];
  __shared__ int last;
  __shared__ int fs[DEC_THREADS / 32][DEC_FJ];    // finalize inputs of tokens 0..7
  __shared__ float fw[DEC_THREADS / 32][DEC_FJ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane >> 4, ch = lane & 15;
  const int c0 = 64 * blockIdx.x;
  const int xsw = a.I / 2;
  const int xn = a.I / 8;  // u32x4 per y1 row
  // the tile count and this workgroup's first tile in one round of loads
  // (the tile arrays hold max_tiles >= gridDim.y entries)
  const int nt = *a.num_tiles;
  int te = a.tile_expert[blockIdx.y], tl = a.tile_limit[blockIdx.y];
  if (tid < DEC_THREADS / 32 * DEC_FJ) {
    const int m = tid / DEC_FJ, j = tid % DEC_FJ;
    const bool ok = m < a.M && j < a.top_k;
    const int r = ok ? m * a.top_k + j : 0;
    fs[m][j] = ok ? a.e2p[r] : -1;
    fw[m][j] = a.topk_w[r] * a.rsf;
  }
  for (int pt = blockIdx.y; pt < nt; pt += gridDim.y) {
    if (pt != (int)blockIdx.y) {
      te = a.tile_expert[pt];
      tl = a.tile_limit[pt];
    }
    const int e = te;
    const int slot0 = pt * DEC_T;
    const int valid = tl - slot0;
    const float al = a.w2_alpha[e];
    const int64_t row0 = (int64_t)e * a.H + c0 + 16 * wave + rr;
    for (int r0 = 0; r0 < valid; r0++) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.y1 + (int64_t)(slot0 + r0) * a.I);
      u32x4_t yv[DEC_YMAX];
#pragma unroll
      for (int j = 0; j < DEC_YMAX; j++) yv[j] = src[min(tid + DEC_THREADS * j, xn - 1)];
      __builtin_amdgcn_sched_barrier(0);  // the y1 loads go out before the weight loads
      Chunk b[D];
      prefetch16<D>(a.w2, a.w2_sf, row0, a.I, ch, b);
      lds_barrier();  // the previous row's xs and ybuf are no longer read
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(xs);
#pragma unroll
      for (int j = 0; j < DEC_YMAX; j++)
        if (tid + DEC_THREADS * j < xn) dst[tid + DEC_THREADS * j] = yv[j];
      lds_barrier();
      float acc[4][DEC_ROWS] = {};
      stream_rows16<DEC_ROWS, D>(a.w2, a.w2_sf, row0, a.I, ch, xs, xsw, b, acc);
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const float v = sum16(acc[g][0]);
        float y2v = v * al;
        if (a.fc2_bias) y2v = y2v + a.fc2_bias[(int64_t)e * a.H + c0 + 16 * wave + 4 * g + rr];
        if (ch == 0) ybuf[16 * wave + 4 * g + rr] = f32_to_bf16(y2v);
      }
      lds_barrier();
      if constexpr (ATOMIC) {
        if (tid < 32) {
          const int route = a.p2e[slot0 + r0];
          const float wf = __fmul_rn(a.topk_w[route], a.rsf);
          const uint32_t yy = reinterpret_cast<const uint32_t*>(ybuf)[tid];
          const float v0 = __fmul_rn(wf, __uint_as_float(yy << 16));
          const float v1 = __fmul_rn(wf, __uint_as_float(yy & 0xffff0000u));
          bf16x2_t pv = {(__bf16)v0, (__bf16)v1};
          __builtin_amdgcn_global_atomic_fadd_v2bf16(
              reinterpret_cast<bf16x2_t*>(a.out + (int64_t)(route / a.top_k) * a.H + c0 + 2 * tid), pv);
        }
      } else {
        // the row's 64 outputs: one 128-byte line from 32 lanes
        if (tid < 32)
          st_dev(reinterpret_cast<uint32_t*>(a.y2 + (int64_t)(slot0 + r0) * a.H + c0) + tid,
                 reinterpret_cast<const uint32_t*>(ybuf)[tid]);
      }
    }
  }
  if constexpr (ATOMIC) return;
  const int old = publish_bump(done_count(a, blockIdx.x));
  if (tid == 0) last = (old == (int)gridDim.y - 1);
  __syncthreads();
  if (last) finalize_cols(a, c0, fs, fw);
}

// ---------------------------------------------------------------- host side

static size_t plan_lds(int El, int R) {
  return sizeof(int) * ((size_t)El * 3 + 1 + DEC_THREADS / 64 + (size_t)R + DEC_T + 4) + 16;
}

bool decode_supported(int mode, int M, int top_k, int El, int H, int I) {
  const int R = M * top_k;
  const size_t lds = plan_lds(El, R) + sizeof(uint16_t) * DEC_ROWS * (size_t)H + 16;
  return mode == 0 && M > 0 && (int64_t)M * top_k <= DEC_MAX_ROUTES && El <= MAX_LOCAL_EXPERTS &&
         H % 512 == 0 && H <= 64 * DEC_MAX_COL_GROUPS && I % 512 == 0 && I <= 8192 && lds <= 65536;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  DecArgs a = {};
  a.ids = p.topk_ids;
  a.M = p.plan->M;
  a.top_k = p.plan->top_k;
  a.El = p.plan->num_local_experts;
  a.offset = p.local_expert_offset;
  a.x = reinterpret_cast<const uint16_t*>(p.x);
  a.x_row_stride = p.x_row_stride;
  a.w1 = p.w1;
  a.w1_sf = p.w1_sf;
  a.w1_alpha = p.w1_alpha;
  a.w1_alpha_up = p.w1_alpha_up;
  a.fc1_bias = p.fc1_bias;
  a.fc2_bias = p.fc2_bias;
  a.w2 = p.w2;
  a.w2_sf = p.w2_sf;
  a.w2_alpha = p.w2_alpha;
  a.H = p.H;
  a.I = p.I;
  a.ip = p.act.kind == ACT_RELU2 ? p.I / 2 : p.I;
  a.act = p.act;
  a.y1 = p.y1;
  a.y2 = p.y2;
  a.counters = p.counters;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.accumulate = p.accumulate;
  a.zero_out = p.atomic && !p.accumulate;
  a.out = p.out;
  a.e2p = p.plan->expanded_to_permuted;
  a.p2e = p.plan->permuted_to_expanded;
  a.tile_expert = p.plan->tile_to_expert;
  a.tile_limit = p.plan->tile_to_mn_limit;
  a.num_tiles = p.plan->num_tiles;
  a.offsets = p.plan->expert_offsets;
  a.counts = p.plan->expert_counts;
  a.slots = p.plan->route_slots;
  a.max_tiles = p.plan->max_tiles;
  const int R = a.M * a.top_k;
  const int P = a.max_tiles < DEC_TILE_STRIDE ? (a.max_tiles > 0 ? a.max_tiles : 1) : DEC_TILE_STRIDE;
  const size_t lds1 = plan_lds(a.El, R) + sizeof(uint16_t) * DEC_ROWS * a.H + 16;
  // prefetch depth: the deepest that divides the K-step count
  const int ns1 = a.H / 512;
  const dim3 g1(a.ip / (16 * G1_NP), P), g2(a.H / 64, P);
  if (p.mark) p.mark(p.mark_ctx, 1);
  // one kernel per activation: the epilogue holds only its own code
  auto go = [&](auto dk, auto ak) {
    dec_gemm1_kernel<decltype(dk)::value, G1_NP, decltype(ak)::value><<<g1, DEC_THREADS, lds1, stream>>>(a);
  };
  auto by_act = [&](auto dk) {
    switch (a.act.kind) {
      case ACT_GEGLU_TANH: go(dk, std::integral_constant<int, ACT_GEGLU_TANH>{}); break;
      case ACT_SITU: go(dk, std::integral_constant<int, ACT_SITU>{}); break;
      case ACT_RELU2: go(dk, std::integral_constant<int, ACT_RELU2>{}); break;
      default: go(dk, std::integral_constant<int, ACT_SWIGLU>{}); break;
    }
  };
  if (ns1 % G1_D == 0) by_act(std::integral_constant<int, G1_D>{});
  else if (ns1 % 2 == 0) by_act(std::integral_constant<int, 2>{});
  else by_act(std::integral_constant<int, 1>{});
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.mark) p.mark(p.mark_ctx, 2);
  // 4 * I/512 K-steps: a multiple of 4
  if (p.atomic) dec_gemm2_kernel<4, true><<<g2, DEC_THREADS, 0, stream>>>(a);
  else dec_gemm2_kernel<4, false><<<g2, DEC_THREADS, 0, stream>>>(a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.mark) p.mark(p.mark_ctx, 3);  // the finalize ran inside GEMM2
  return hipSuccess;
}

}  // namespace moe
