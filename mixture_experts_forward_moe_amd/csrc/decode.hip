// decode.hip -- the W4A16 forward for decode-sized batches in one launch.
//
// At decode sizes (a route or two per active expert) the pass is bound by
// HBM bandwidth on weight bytes: each weight byte meets one or two
// activation rows.  Separate sort / GEMM1 / GEMM2 / finalize launches would
// each pay a launch gap and a cold start (routing ids, then activations,
// then weights: three dependent trips to memory) that cost about as much as
// a kernel's whole weight stream, so the path is one persistent kernel:
//
//  * Every workgroup builds the batch's routing plan in LDS (per-expert
//    counts, 16-slot tiles, stable slots in route order: the plan moe_sort
//    builds).  Workgroup 0 also writes the plan out.
//  * Tasks [0, n1): GEMM1 of one 16-slot tile for 16 columns of I -- 16 gate
//    and 16 up weight rows streamed against the tile's x rows, expert scale,
//    SwiGLU, bf16 y1.  Finishing one bumps the tile's ready count.
//  * Tasks [n1, n1 + n2): GEMM2 of one tile for 64 columns of H.  The
//    workgroup puts its first weight loads in flight, then waits for the
//    tile's ready count (all I/16 GEMM1 tasks of the tile), stages the y1
//    rows and streams the rest.  Finishing one bumps the column group's
//    done count; the task that completes a column group over all tiles
//    applies the deterministic route-order finalize to those 64 columns of
//    every token ("flashinfer.fused_moe.alphamoe_nvfp4_routed_moe",
//    summary: contributions in route order, seeded from the output).
//  * Workgroup b of G takes tasks b, b + G, b + 2G, ...  GEMM1 tasks go
//    round the tiles (task t: tile t % nt), so each tile's tasks spread over
//    all of a CU's workgroup slots and the tiles are ready together; GEMM2
//    tasks likewise, so each column group's tiles finish together.  A
//    shared task counter would cost an atomic per task on one address, and
//    those serialise (about 12 ns each) into a bottleneck of their own.
//
// Forward progress: the launch has no more workgroups than fit on the
// device at once, and each workgroup runs all of its GEMM1 tasks, which
// wait for nothing, before any GEMM2 task; so every GEMM1 task a GEMM2 task
// waits for is run by a workgroup that is (or, once other work on the
// device drains, will be) resident.  Waits are still bounded: one that
// runs out writes NaN for its outputs and bumps a sticky stall count.  The
// workgroup that finalizes the last column group clears the counters for
// the next call.
//
// Inner product without matrix cores: lane (rr, ch) owns weight row rr of
// its wavefront's four and the 16-byte chunks ch, ch+16, ... of that row
// (32 codes, two E4M3 blocks each).  Codes become bf16 pairs with
// v_cvt_scalef32_pk_bf16_fp4 (scale 1: exact E2M1 values), v_dot2_f32_bf16
// multiplies them with bf16 activation pairs read from LDS, and each
// block's partial sum is multiplied by its decoded scale (v_cvt_f32_fp8).
// The 16 chunk lanes of a row reduce with a fixed xor tree, so results are
// reproducible run to run.
#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace moe {

constexpr int DEC_THREADS = 256;
constexpr int DEC_T = 16;                        // plan tile
constexpr int DEC_G1_COLS = 16;                  // GEMM1 task: columns of I
constexpr int DEC_G2_COLS = 64;                  // GEMM2 task: columns of H
constexpr long long DEC_SPIN_LIMIT = 1ll << 19;  // polls before a wait gives up (about a second)

// The counter block: the head slot holds the count of finalized column
// groups and the (sticky) count of stalled waits; then one slot per tile
// (ready count) and one per column group (done count).  One counter per
// 256 bytes: atomics and device-scope polls that share a line queue behind
// each other at the memory side, and with every tile's counter on one line
// that queue held up the whole launch.
constexpr int CTR_FINAL = 0, CTR_STALL = 1;
DEV int* ready_ctr(int* ctr, int pt) { return ctr + DEC_CTR_SLOT * (1 + pt); }
DEV int* done_ctr(int* ctr, int c) { return ctr + DEC_CTR_SLOT * (1 + DEC_MAX_TILES + c); }

struct DecArgs {
  const int32_t* ids;
  int M, top_k, El, offset;
  const uint16_t* x;
  int64_t x_row_stride;  // elements
  const uint8_t* w1;
  const uint8_t* w1_sf;
  const float* w1_alpha;
  const uint8_t* w2;
  const uint8_t* w2_sf;
  const float* w2_alpha;
  int H, I;
  float sw_alpha, sw_beta, sw_limit;
  uint16_t* y1;  // [slots, I]
  uint16_t* y2;  // [slots, H]
  int* ctr;      // counter block, zero between calls
  const float* topk_w;
  float rsf;
  int accumulate;
  uint16_t* out;
  // plan arrays written by workgroup 0
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

// The batch's plan in LDS: counts, tile bases, and every route's slot
// (slots of expert e start at 16 * tbase[e], in ascending route order).
DEV int build_plan(const DecArgs& a, const LocalPlan& P) {
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
  // stable slots: wavefront 0 walks the routes 64 at a time
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
  return nt;
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

// routes of tile pt (owned by expert e) that are in use
DEV int tile_valid(const LocalPlan& P, int e, int pt) { return min(DEC_T, P.tbase[e] * DEC_T + P.cnt[e] - pt * DEC_T); }

// ---------------------------------------------------------------- streaming

// Weight rows are addressed as a wavefront-uniform base (the first of the
// wavefront's rows, in scalar registers) plus a 32-bit lane offset: lane
// (rr, ch) reads row rr of the base, 16-byte chunk ch of each K-step, and
// the matching pair of scale codes.  K-step s is 16 chunks further on.
struct RowPtr {
  const uint8_t* w;  // uniform
  const uint8_t* s;  // uniform
};

struct LaneOff {
  uint32_t w, s;
};

DEV RowPtr row_base(const uint8_t* W, const uint8_t* Wsf, int64_t row, int K) {
  return RowPtr{W + row * (K / 2), Wsf + row * (K / 16)};
}

DEV LaneOff lane_off(int rr, int ch, int K) {
  return LaneOff{(uint32_t)(rr * (K / 2) + ch * 16), (uint32_t)(rr * (K / 16) + ch * 2)};
}

struct Chunk {
  u32x4_t w;
  uint32_t s;
};

DEV Chunk load_step(const RowPtr& p, const LaneOff& o, int step) {
  Chunk c;
  c.w = *reinterpret_cast<const u32x4_t*>(p.w + (o.w + (uint32_t)step * 256u));
  c.s = *reinterpret_cast<const uint16_t*>(p.s + (o.s + (uint32_t)step * 32u));
  return c;
}

// two E2M1 codes (byte B of w) as a bf16 pair, exact
template <int B>
DEV uint32_t e2m1x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}

DEV void decode_chunk(const Chunk& c, uint32_t* wb) {
  // copy the words out: bit-casting an element of a vector register in
  // place is not reliable
  const uint32_t w4[4] = {c.w.x, c.w.y, c.w.z, c.w.w};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    wb[4 * j + 0] = e2m1x2_bf16<0>(w4[j]);
    wb[4 * j + 1] = e2m1x2_bf16<1>(w4[j]);
    wb[4 * j + 2] = e2m1x2_bf16<2>(w4[j]);
    wb[4 * j + 3] = e2m1x2_bf16<3>(w4[j]);
  }
}

// acc + the chunk's 32 products with the activation pairs of chunk kc at xs
// (LDS), each 16-element block's partial sum times its decoded E4M3 scale
DEV float dot_chunk(const Chunk& c, const uint32_t* xs, int kc, float acc) {
  uint32_t wb[16];
  decode_chunk(c, wb);
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(xs + kc * 16);
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const u32x4_t v = xr[j];
    const uint32_t xw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xw[b]);
      const bf16x2_t wp = __builtin_bit_cast(bf16x2_t, wb[4 * j + b]);
      if (j < 2) p0 = __builtin_amdgcn_fdot2_f32_bf16(xp, wp, p0, false);
      else p1 = __builtin_amdgcn_fdot2_f32_bf16(xp, wp, p1, false);
    }
  }
  const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)c.s, 0), s1 = __builtin_amdgcn_cvt_f32_fp8((int)c.s, 1);
  acc = acc + s0 * p0;
  acc = acc + s1 * p1;
  return acc;
}

// gate and up chunks of the same K range against the same activations:
// each activation word is read from LDS once for both rows
DEV void dot_chunk2(const Chunk& cg, const Chunk& cu, const uint32_t* xs, int kc, float& ag, float& au) {
  uint32_t wg[16], wu[16];
  decode_chunk(cg, wg);
  decode_chunk(cu, wu);
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(xs + kc * 16);
  float pg0 = 0.0f, pg1 = 0.0f, pu0 = 0.0f, pu1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const u32x4_t v = xr[j];
    const uint32_t xw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xw[b]);
      const bf16x2_t gp = __builtin_bit_cast(bf16x2_t, wg[4 * j + b]);
      const bf16x2_t up = __builtin_bit_cast(bf16x2_t, wu[4 * j + b]);
      if (j < 2) {
        pg0 = __builtin_amdgcn_fdot2_f32_bf16(xp, gp, pg0, false);
        pu0 = __builtin_amdgcn_fdot2_f32_bf16(xp, up, pu0, false);
      } else {
        pg1 = __builtin_amdgcn_fdot2_f32_bf16(xp, gp, pg1, false);
        pu1 = __builtin_amdgcn_fdot2_f32_bf16(xp, up, pu1, false);
      }
    }
  }
  const float g0 = __builtin_amdgcn_cvt_f32_fp8((int)cg.s, 0), g1 = __builtin_amdgcn_cvt_f32_fp8((int)cg.s, 1);
  const float u0 = __builtin_amdgcn_cvt_f32_fp8((int)cu.s, 0), u1 = __builtin_amdgcn_cvt_f32_fp8((int)cu.s, 1);
  ag = ag + g0 * pg0;
  ag = ag + g1 * pg1;
  au = au + u0 * pu0;
  au = au + u1 * pu1;
}

DEV float sum16(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

// GEMM1 lane work: one gate and one up row over K = H.  g1_prefetch loads
// the first D steps (before the activations are staged); g1_run keeps D
// steps in flight.  Its steady loop issues every load unconditionally (D
// divides the step count), so each step waits only for its own loads.
template <int D>
DEV void g1_prefetch(const RowPtr& pg, const RowPtr& pu, const LaneOff& o, Chunk* bg, Chunk* bu) {
#pragma unroll
  for (int d = 0; d < D; d++) {
    bg[d] = load_step(pg, o, d);
    bu[d] = load_step(pu, o, d);
  }
}

// Issue priority by remaining work: a wavefront that has fallen behind
// (more of its row still to stream) is served first, so the workgroups on
// a CU finish closer together instead of strictly in launch order.
DEV void prio_by_progress(int done, int total) {
  const int left4 = 4 * (total - done);
  if (left4 > 3 * total) __builtin_amdgcn_s_setprio(3);
  else if (left4 > 2 * total) __builtin_amdgcn_s_setprio(2);
  else if (left4 > total) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

template <int D>
DEV void g1_run(const RowPtr& pg, const RowPtr& pu, const LaneOff& o, int nsteps, int ch, Chunk* bg, Chunk* bu,
                const uint32_t* xs, float& ag, float& au) {
  int s0 = 0;
  for (; s0 + D < nsteps; s0 += D) {
    prio_by_progress(s0, nsteps);
#pragma unroll
    for (int d = 0; d < D; d++) {
      dot_chunk2(bg[d], bu[d], xs, ch + 16 * (s0 + d), ag, au);
      bg[d] = load_step(pg, o, s0 + d + D);
      bu[d] = load_step(pu, o, s0 + d + D);
      __builtin_amdgcn_sched_barrier(0);  // keep one step's values live at a time
    }
  }
#pragma unroll
  for (int d = 0; d < D; d++) {
    dot_chunk2(bg[d], bu[d], xs, ch + 16 * (s0 + d), ag, au);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// GEMM2 lane work: rows 4g + rr (g = 0..3) of the wavefront's 16 over
// K = I, the four rows interleaved (flattened step f: row f % 4, K-step
// f / 4) so that all their loads are in flight together.
template <int D>
DEV void g2_prefetch(const RowPtr* pr, const LaneOff& o, Chunk* b) {
#pragma unroll
  for (int d = 0; d < D; d++) b[d] = load_step(pr[d & 3], o, d >> 2);
}

template <int D>
DEV void g2_run(const RowPtr* pr, const LaneOff& o, int nflat, int ch, Chunk* b, const uint32_t* xs, float* acc) {
  static_assert(D % 4 == 0, "row of a flattened step must be d % 4");
  int f0 = 0;
  for (; f0 + D < nflat; f0 += D) {
    prio_by_progress(f0, nflat);
#pragma unroll
    for (int d = 0; d < D; d++) {
      const int f = f0 + d;
      acc[d & 3] = dot_chunk(b[d], xs, ch + 16 * (f >> 2), acc[d & 3]);
      const int fn = f + D;
      b[d] = load_step(pr[d & 3], o, fn >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D; d++) {
    const int f = f0 + d;
    acc[d & 3] = dot_chunk(b[d], xs, ch + 16 * (f >> 2), acc[d & 3]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- sync
//
// Data that crosses workgroups (y1, y2) and the counters are accessed with
// device-scope loads and stores (the scope bits of each instruction: they
// bypass the CU's L1 and stay coherent across the L2s of all XCDs), and
// ordered by waiting for the stores to complete before the counter bump.
// Fences at device scope would do the same with a write-back or invalidate
// of a whole L2 per fence, which at thousands of tasks per launch costs
// more than the weight stream itself.  The stores write through to memory,
// so a task gathers its outputs in LDS first and stores them as whole
// 32- or 128-byte pieces from consecutive lanes of one instruction:
// scattered 2-byte write-throughs clog the memory controllers.

DEV void st_dev(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish this workgroup's device-scope stores: every wavefront waits for
// its stores to complete (vmcnt 0), then after the barrier thread 0 bumps
// *c.  The previous value goes to thread 0.
DEV int publish_bump(int* c) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // keeps the stores above the wait
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0): expcnt and lgkmcnt not waited
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

// thread 0: wait until *c >= target; false if the wait ran out.  Polls
// back off exponentially to about 2 us apart: device-scope loads bypass the
// caches, so hundreds of workgroups polling one line at full rate would
// saturate the memory channel that holds it, and every weight stream with
// bytes on that channel would stall behind the polls.
DEV bool wait_at_least(int* c, int target) {
  int nap = 1;
  for (long long it = 0; it < DEC_SPIN_LIMIT; it++) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    // s_sleep takes an immediate: one branch per step of the backoff
    if (nap <= 1) __builtin_amdgcn_s_sleep(1);
    else if (nap <= 2) __builtin_amdgcn_s_sleep(2);
    else if (nap <= 4) __builtin_amdgcn_s_sleep(4);
    else if (nap <= 8) __builtin_amdgcn_s_sleep(8);
    else if (nap <= 16) __builtin_amdgcn_s_sleep(16);
    else if (nap <= 32) __builtin_amdgcn_s_sleep(32);
    else __builtin_amdgcn_s_sleep(64);
    if (nap < 64) nap *= 2;
  }
  return false;
}

// ---------------------------------------------------------------- finalize

// out[:, c0 : c0 + 64] in route order for every token.  Thread (tt, p) owns
// columns c0 + 2p and c0 + 2p + 1 of tokens tt, tt + 8, ...
DEV void finalize_cols(const DecArgs& a, const int* e2p, int c0) {
  const int tid = threadIdx.x;
  const int p = tid & 31, tt = tid >> 5;
  const int col = c0 + 2 * p;
  for (int m = tt; m < a.M; m += DEC_THREADS / 32) {
    uint32_t* o = reinterpret_cast<uint32_t*>(a.out + (int64_t)m * a.H + col);
    float acc0 = 0.0f, acc1 = 0.0f;
    if (a.accumulate) {
      const uint32_t v = *o;
      acc0 = __uint_as_float(v << 16);
      acc1 = __uint_as_float(v & 0xffff0000u);
    }
    for (int j = 0; j < a.top_k; j++) {
      const int r = m * a.top_k + j;
      const int s = e2p[r];
      if (s < 0) continue;
      const float wf = a.topk_w[r] * a.rsf;
      const uint32_t v = ld_dev(reinterpret_cast<const uint32_t*>(a.y2 + (int64_t)s * a.H + col));
      acc0 = acc0 + wf * __uint_as_float(v << 16);
      acc1 = acc1 + wf * __uint_as_float(v & 0xffff0000u);
    }
    *o = pack_bf16x2(acc0, acc1);
  }
}

// Finalize one column group, then count it.  The workgroup that completes
// the last group clears the counters for the next call: by then every
// GEMM1 task has been counted and every wait of this launch is over.
DEV void finalize_group(const DecArgs& a, const int* e2p, int c0, int* bc) {
  finalize_cols(a, e2p, c0);
  const int old = publish_bump(a.ctr + CTR_FINAL);
  if (threadIdx.x == 0) bc[2] = (old == a.H / DEC_G2_COLS - 1);
  __syncthreads();
  if (bc[2]) {
    for (int i = threadIdx.x; i < DEC_MAX_TILES + DEC_MAX_COL_GROUPS; i += DEC_THREADS)
      __hip_atomic_store(a.ctr + DEC_CTR_SLOT * (1 + i), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(a.ctr + CTR_FINAL, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- kernel

template <int D1, int D2>
__global__ __launch_bounds__(DEC_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void dec_fused_kernel(const DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dsm[];
  const int R = a.M * a.top_k;
  LocalPlan P;
  P.cnt = (int*)dsm;
  P.tbase = P.cnt + a.El;
  P.run = P.tbase + a.El + 1;
  P.tmp = P.run + a.El;
  P.e2p = P.tmp + DEC_THREADS / 64;
  int* rows = P.e2p + R;   // [16] routes of the current tile
  int* bc = rows + DEC_T;  // [4] broadcast words
  uint32_t* ybuf = reinterpret_cast<uint32_t*>(bc + 4);  // [32] a task's outputs of one row, bf16 pairs
  uint16_t* ybuf16 = reinterpret_cast<uint16_t*>(ybuf);
  // staged activation row at the next 16-byte boundary: offset arithmetic
  // on the LDS array itself (an integer round trip would make every read a
  // flat load, and a flat load waits for all weight loads in flight)
  const int xs_word = (3 * a.El + 1 + DEC_THREADS / 64 + R + DEC_T + 4 + 32 + 3) & ~3;
  uint32_t* xs = dsm + xs_word;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // the same, known uniform
  const int rr = lane >> 4, ch = lane & 15;

  const int nt = build_plan(a, P);

  if (blockIdx.x == 0) {
    // the plan, for callers that read it
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

  const int g1_per_tile = a.I / DEC_G1_COLS, g2_per_tile = a.H / DEC_G2_COLS;
  const int n1 = nt * g1_per_tile, n2 = nt * g2_per_tile;
  const int G = gridDim.x;
  int t = blockIdx.x;

  // ---------------- GEMM1 tasks: tile pt, columns [16 cg, 16 cg + 16) of I
  for (; t < n1; t += G) {
    const int cg = t / nt, pt = t - cg * nt;  // tiles interleaved
    const int e = tile_owner(P, a.El, pt);
    const int valid = tile_valid(P, e, pt), slot0 = pt * DEC_T;
    const int col = DEC_G1_COLS * cg + 4 * wave + rr;
    const int64_t rg = (int64_t)e * 2 * a.I + DEC_G1_COLS * cg + 4 * wv;  // wavefront's first gate row
    const RowPtr pg = row_base(a.w1, a.w1_sf, rg, a.H);
    const RowPtr pu = row_base(a.w1, a.w1_sf, rg + a.I, a.H);
    const LaneOff lo = lane_off(rr, ch, a.H);
    const float al = a.w1_alpha[e];
    for (int r = tid; r < R; r += DEC_THREADS) {
      const int s = P.e2p[r];
      if (s >= slot0 && s < slot0 + DEC_T) rows[s - slot0] = r;
    }
    for (int r0 = 0; r0 < valid; r0++) {
      Chunk bg[D1], bu[D1];
      g1_prefetch<D1>(pg, pu, lo, bg, bu);
      __syncthreads();  // rows[] is filled and the previous pass is done with xs
      const int64_t tok = rows[r0] / a.top_k;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.x + tok * a.x_row_stride);
      for (int i = tid; i < a.H / 8; i += DEC_THREADS) reinterpret_cast<u32x4_t*>(xs)[i] = src[i];
      __syncthreads();
      float ag = 0.0f, au = 0.0f;
      g1_run<D1>(pg, pu, lo, a.H / 512, ch, bg, bu, xs, ag, au);
      const float g = sum16(ag), u = sum16(au);
      if (ch == 0) ybuf16[col - DEC_G1_COLS * cg] = f32_to_bf16(swiglu_f32(g * al, u * al, a.sw_alpha, a.sw_beta, a.sw_limit));
      __syncthreads();
      if (tid < DEC_G1_COLS / 2)  // the row's 16 outputs: 32 bytes from 8 lanes
        st_dev(reinterpret_cast<uint32_t*>(a.y1 + (int64_t)(slot0 + r0) * a.I + DEC_G1_COLS * cg) + tid, ybuf[tid]);
    }
    publish_bump(ready_ctr(a.ctr, pt));
  }

  // ---------------- GEMM2 tasks: tile pt, columns [64 c, 64 c + 64) of H
  for (; t < n1 + n2; t += G) {
    const int t2 = t - n1;
    const int c = t2 / nt, pt = t2 - c * nt;  // a column group's tiles together
    const int e = tile_owner(P, a.El, pt);
    const int valid = tile_valid(P, e, pt), slot0 = pt * DEC_T;
    const int c0 = DEC_G2_COLS * c;
    const int64_t row0 = (int64_t)e * a.H + c0 + 16 * wv;  // wavefront's first row
    RowPtr pr[4];
#pragma unroll
    for (int g = 0; g < 4; g++) pr[g] = row_base(a.w2, a.w2_sf, row0 + 4 * g, a.I);
    const LaneOff lo = lane_off(rr, ch, a.I);
    const float al = a.w2_alpha[e];
    bool ok = true;
    for (int r0 = 0; r0 < valid; r0++) {
      Chunk b[D2];
      g2_prefetch<D2>(pr, lo, b);
      if (r0 == 0) {
        // the tile's y1 is complete once all its GEMM1 tasks are
        if (tid == 0) bc[0] = wait_at_least(ready_ctr(a.ctr, pt), g1_per_tile) ? 1 : 0;
        __syncthreads();
        ok = bc[0] != 0;
      } else {
        __syncthreads();  // the previous pass is done with xs
      }
      const uint64_t* src = reinterpret_cast<const uint64_t*>(a.y1 + (int64_t)(slot0 + r0) * a.I);
      for (int i = tid; i < a.I / 4; i += DEC_THREADS) reinterpret_cast<uint64_t*>(xs)[i] = ld_dev(src + i);
      __syncthreads();
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      g2_run<D2>(pr, lo, 4 * (a.I / 512), ch, b, xs, acc);
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const float v = sum16(acc[g]);
        if (ch == 0) ybuf16[16 * wave + 4 * g + rr] = ok ? f32_to_bf16(v * al) : (uint16_t)0x7fc0;
      }
      __syncthreads();
      if (tid < DEC_G2_COLS / 2)  // the row's 64 outputs: one 128-byte line from 32 lanes
        st_dev(reinterpret_cast<uint32_t*>(a.y2 + (int64_t)(slot0 + r0) * a.H + c0) + tid, ybuf[tid]);
    }
    if (tid == 0 && !ok) atomicAdd(a.ctr + CTR_STALL, 1);
    const int old = publish_bump(done_ctr(a.ctr, c));
    if (tid == 0) bc[1] = (old == nt - 1);
    __syncthreads();
    if (bc[1]) finalize_group(a, P.e2p, c0, bc);  // every tile's GEMM2 for these columns is done
  }

  // ---------------- with no local route: the finalize of every column group
  if (nt == 0)
    for (int c = blockIdx.x; c < g2_per_tile; c += G) finalize_group(a, P.e2p, DEC_G2_COLS * c, bc);
}

// ---------------------------------------------------------------- host side

constexpr int DEC_D1 = 2;  // GEMM1 K-steps in flight
constexpr int DEC_D2 = 4;  // GEMM2 flattened steps in flight

static size_t dec_lds(int El, int R, int H, int I) {
  const size_t words = ((size_t)(3 * El + 1 + DEC_THREADS / 64 + R + DEC_T + 4 + 32) + 3) & ~(size_t)3;
  return sizeof(uint32_t) * words + sizeof(uint16_t) * (size_t)(H > I ? H : I);
}

bool decode_supported(int mode, int M, int top_k, int El, int H, int I) {
  const int64_t R = (int64_t)M * top_k;
  // the prefetch depths divide the K-step counts, so no load runs past a row
  return mode == 0 && M > 0 && R <= DEC_MAX_ROUTES && El <= MAX_LOCAL_EXPERTS && H % 512 == 0 && I % 512 == 0 &&
         (H / 512) % DEC_D1 == 0 && (4 * (I / 512)) % DEC_D2 == 0 && H / DEC_G2_COLS <= DEC_MAX_COL_GROUPS &&
         dec_lds(El, (int)R, H, I) <= 65536;
}

// Workgroups that fit on the device at once (cached per device).  The
// launch never uses more: a GEMM2 task waits for GEMM1 tasks of other
// workgroups, which must not be queued behind it.
static int dec_grid(size_t lds) {
  static int cached[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev][0] == 0 || cached[dev][1] != (int)lds) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, dec_fused_kernel<DEC_D1, DEC_D2>, DEC_THREADS, lds) !=
            hipSuccess ||
        per <= 0)
      per = 1;
    cached[dev][0] = cus * per;
    cached[dev][1] = (int)lds;
  }
  return cached[dev][0];
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
  a.w2 = p.w2;
  a.w2_sf = p.w2_sf;
  a.w2_alpha = p.w2_alpha;
  a.H = p.H;
  a.I = p.I;
  a.sw_alpha = p.swiglu_alpha;
  a.sw_beta = p.swiglu_beta;
  a.sw_limit = p.swiglu_limit;
  a.y1 = p.y1;
  a.y2 = p.y2;
  a.ctr = p.counters;
  a.topk_w = p.topk_weights;
  a.rsf = p.routed_scaling_factor;
  a.accumulate = p.accumulate;
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
  if (a.max_tiles > DEC_MAX_TILES) return hipErrorInvalidValue;
  const int R = a.M * a.top_k;
  const size_t lds = dec_lds(a.El, R, a.H, a.I);
  // more workgroups than tasks would only build the plan and leave
  const int64_t tasks = (int64_t)a.max_tiles * (a.I / DEC_G1_COLS + a.H / DEC_G2_COLS);
  int grid = dec_grid(lds);
  if (tasks < grid) grid = (int)(tasks > 0 ? tasks : 1);
  if (p.mark) p.mark(p.mark_ctx, 1);
  dec_fused_kernel<DEC_D1, DEC_D2><<<grid, DEC_THREADS, lds, stream>>>(a);
  hipError_t err = hipGetLastError();
  if (p.mark) {
    p.mark(p.mark_ctx, 2);
    p.mark(p.mark_ctx, 3);
  }
  return err;
}

}  // namespace moe
