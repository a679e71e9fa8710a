// sort.hip -- moe_sort on gfx950: the routing plan of the fused MoE forward.
//
// The plan ("vllm.models.flint.ops.moe_cute", grouped_moe: tile_to_expert,
// tile_to_mn_limit, expanded_to_permuted, permuted_to_expanded, num_tiles)
// puts each local expert's routes into consecutive slots in ascending route
// order r = t*top_k + j, pads every expert's range to a multiple of the tile
// and lists the tiles.  The order inside an expert is stable, so the plan is
// bit-exact and reproducible, and a tile's rows come from a narrow token
// window (the locality FlashInfer pull request 4440 gets from contiguous
// per-CTA route windows).
//
// Two parallelisations give the same plan:
//  - single workgroup (small route counts): histogram -> scan -> scatter in
//    one 1024-thread workgroup, every expert id read once into registers;
//  - spans (large route counts): each workgroup owns one contiguous span of
//    routes; kernel 1 writes per-span expert histograms; in kernel 2 every
//    workgroup scans them across spans and experts (workgroup 0 also writes
//    the tile tables) and scatters its span in order.  Every workgroup stops
//    at its own span end.
// Inside a span, routes are ranked 1024 at a time: wavefront ballots give a
// route's rank among equal experts in its wavefront, and an LDS prefix over
// the 16 wavefronts gives the rest.
#include "device_common.h"
#include "internal.h"

namespace moe {

constexpr int SORT_THREADS = 1024;
constexpr int SORT_WAVES = SORT_THREADS / 64;
constexpr int SORT_FUSED_COUNTS = 8192;  // ints of LDS for the one-pass scatter (32 KiB)

struct SortArgs {
  const int32_t* ids;
  int64_t R;  // routes M * top_k
  int El;
  int offset;
  int tile;
  int nbits;  // bits to hold El (the non-local sentinel)
  int64_t slots;
  int max_tiles;
  int spans;
  int64_t span_len;
  int32_t* e2p;
  int32_t* p2e;
  int32_t* tile_expert;
  int32_t* tile_limit;
  int32_t* num_tiles;
  int32_t* offsets;  // [El+1]
  int32_t* counts;   // [El]
  int32_t* scratch;  // [spans][El] span histograms, then span bases
};

DEV int local_expert(const SortArgs& a, int64_t r) {
  int id = a.ids[r];
  int le = id - a.offset;
  return (id >= a.offset && le < a.El) ? le : -1;
}

// per-span histogram into LDS counters cnt[El] (zeroed by the caller)
DEV void span_histogram(const SortArgs& a, int64_t lo, int64_t hi, int* cnt) {
  for (int64_t r = lo + threadIdx.x; r < hi; r += SORT_THREADS) {
    int le = local_expert(a, r);
    if (le >= 0) atomicAdd(&cnt[le], 1);
  }
}

// Inclusive prefix sum of x over each aligned segment of `seg` lanes (16,
// 32 or 64) of the wavefront, on the VALU: shifts within 16-lane rows, then
// row broadcasts (each step adds 0 where the source lane lies outside the
// segment).
DEV int seg_incl_scan(int x, int seg) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  if (seg >= 32) x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  if (seg >= 64) x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scan over v[0..n) in LDS by one workgroup; returns the total.
// `tmp` holds SORT_WAVES ints.
DEV int block_exclusive_scan(int* v, int n, int* tmp) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + SORT_THREADS - 1) / SORT_THREADS;
  const int lo = tid * per;
  int s = 0;
  for (int i = 0; i < per; i++)
    if (lo + i < n) s += v[lo + i];
  // inclusive scan of s across the wavefront
  const int x = seg_incl_scan(s, 64);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int wbase = 0, total = 0;
  for (int w = 0; w < SORT_WAVES; w++) {
    int t = tmp[w];
    if (w < wave) wbase += t;
    total += t;
  }
  int run = wbase + x - s;
  for (int i = 0; i < per; i++) {
    if (lo + i < n) {
      int c = v[lo + i];
      v[lo + i] = run;
      run += c;
    }
  }
  __syncthreads();
  return total;
}

// Given per-expert counts cnt[El] (LDS), write counts, offsets, tile tables
// and num_tiles.  base/tbase: LDS [El+1].  Leaves base[le] = first slot.
// write = false: only base / tbase (for workgroups that need the slot bases
// but leave the tables to another).
DEV void plan_tables(const SortArgs& a, const int* cnt, int* base, int* tbase, int* tmp, bool write = true) {
  const int T = a.tile;
  for (int le = threadIdx.x; le < a.El; le += SORT_THREADS) {
    int c = cnt[le];
    int nt = (c + T - 1) / T;
    base[le] = nt * T;
    tbase[le] = nt;
    if (write) a.counts[le] = c;
  }
  __syncthreads();
  int total_slots = block_exclusive_scan(base, a.El, tmp);
  int total_tiles = block_exclusive_scan(tbase, a.El, tmp);
  if (threadIdx.x == 0) {
    base[a.El] = total_slots;
    tbase[a.El] = total_tiles;
    if (write) {
      a.offsets[a.El] = total_slots;
      *a.num_tiles = total_tiles;
    }
  }
  if (!write) {
    __syncthreads();
    return;
  }
  for (int le = threadIdx.x; le < a.El; le += SORT_THREADS) a.offsets[le] = base[le];
  __syncthreads();
  for (int i = threadIdx.x; i < a.max_tiles; i += SORT_THREADS) {
    int te = -1, tl = -1;
    if (i < total_tiles) {
      int lo = 0, hi = a.El - 1;  // last expert with tbase <= i
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (tbase[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      te = lo;
      int start = base[lo] + (i - tbase[lo]) * T;
      int lim = base[lo] + cnt[lo];
      tl = min(start + T, lim);
    }
    a.tile_expert[i] = te;
    a.tile_limit[i] = tl;
  }
}

// One chunk of the stable scatter: this thread's route r (r < hi) has local
// expert le (-1: not local).  running[le] (LDS) holds the next slot of
// expert le and is advanced.  wcnt: LDS [SORT_WAVES][El].  Called by the
// whole workgroup.
DEV void scatter_chunk(const SortArgs& a, int64_t r, int le, int64_t hi, int* running, int* wcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = tid; i < SORT_WAVES * a.El; i += SORT_THREADS) wcnt[i] = 0;
  int key = le < 0 ? a.El : le;
  uint64_t m = ~0ull;
  for (int b = 0; b < a.nbits; b++) {
    int bit = (key >> b) & 1;
    uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  int rank = __popcll(m & below);
  int cnt = __popcll(m);
  __syncthreads();
  if (le >= 0 && rank == 0) wcnt[le * SORT_WAVES + wave] = cnt;
  __syncthreads();
  // per expert, an exclusive scan of its 16 wavefront counts on 16 lanes
  static_assert(SORT_WAVES == 16, "one 16-lane group per expert");
  for (int e0 = 0; e0 < a.El; e0 += SORT_THREADS / SORT_WAVES) {
    const int e = e0 + (tid >> 4), w = tid & 15;
    const int c = (e < a.El) ? wcnt[e * SORT_WAVES + w] : 0;
    const int x = seg_incl_scan(c, 16);
    if (e < a.El) {
      const int run = running[e];
      wcnt[e * SORT_WAVES + w] = run + x - c;
      if (w == 15) running[e] = run + x;
    }
  }
  __syncthreads();
  if (r < hi) {
    if (le >= 0) {
      int slot = wcnt[le * SORT_WAVES + wave] + rank;
      a.e2p[r] = slot;
      a.p2e[slot] = (int32_t)r;
    } else {
      a.e2p[r] = -1;
    }
  }
  __syncthreads();
}

// Stable scatter of routes [lo, hi), 1024 at a time, expert ids read as it goes.
DEV void span_scatter(const SortArgs& a, int64_t lo, int64_t hi, int* running, int* wcnt) {
  for (int64_t c0 = lo; c0 < hi; c0 += SORT_THREADS) {
    const int64_t r = c0 + threadIdx.x;
    scatter_chunk(a, r, (r < hi) ? local_expert(a, r) : -1, hi, running, wcnt);
  }
}

// ---------------------------------------------------------------- kernels

// One workgroup: the whole plan.
__global__ __launch_bounds__(SORT_THREADS) void sort_single_kernel(SortArgs a) {
  extern __shared__ int lds[];
  int* cnt = lds;                      // El
  int* base = cnt + a.El;              // El+1
  int* tbase = base + a.El + 1;        // El+1
  int* tmp = tbase + a.El + 1;         // SORT_WAVES
  int* wcnt = tmp + SORT_WAVES;        // SORT_WAVES * El
  for (int i = threadIdx.x; i < a.El; i += SORT_THREADS) cnt[i] = 0;
  for (int64_t s = threadIdx.x; s < a.slots; s += SORT_THREADS) a.p2e[s] = -1;
  if (a.R > SORT_SINGLE_MAX_ROUTES) {  // a one-workgroup order asked for a large batch
    __syncthreads();
    span_histogram(a, 0, a.R, cnt);
    __syncthreads();
    plan_tables(a, cnt, base, tbase, tmp);
    __syncthreads();
    span_scatter(a, 0, a.R, base, wcnt);
    return;
  }
  // every route's expert is read once, up front, and kept in registers
  constexpr int PER = SORT_SINGLE_MAX_ROUTES / SORT_THREADS;
  static_assert(SORT_SINGLE_MAX_ROUTES % SORT_THREADS == 0, "whole chunks per thread");
  int le[PER];
  int id[PER];
#pragma unroll
  for (int c = 0; c < PER; c++)  // all loads in flight at once (routes past R re-read route 0)
    id[c] = a.ids[(c * SORT_THREADS + (int)threadIdx.x < a.R) ? c * SORT_THREADS + threadIdx.x : 0];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < PER; c++) {
    const int l = id[c] - a.offset;
    le[c] = (c * SORT_THREADS + (int)threadIdx.x < a.R && id[c] >= a.offset && l < a.El) ? l : -1;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < PER; c++)
    if (le[c] >= 0) atomicAdd(&cnt[le[c]], 1);
  __syncthreads();
  plan_tables(a, cnt, base, tbase, tmp);
  __syncthreads();
  const int chunks = (int)((a.R + SORT_THREADS - 1) / SORT_THREADS);
  const int cw = chunks <= 1 ? 1 : (chunks <= 2 ? 2 : 4);  // chunk slots per expert, a power of two
  if (chunks > 4 || a.El * cw * SORT_WAVES > SORT_FUSED_COUNTS) {
#pragma unroll
    for (int c = 0; c < PER; c++)
      if ((int64_t)c * SORT_THREADS < a.R)
        scatter_chunk(a, (int64_t)c * SORT_THREADS + threadIdx.x, le[c], a.R, base, wcnt);
    return;
  }
  // Up to 4096 routes: every chunk ranked at once.  wcnt[(e * cw + c) * 16 + w]
  // counts expert e's routes in wavefront w of chunk c (route order is chunk,
  // then wavefront, then lane); one scan per expert over its cw * 16 counts
  // turns them into slots.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = tid; i < a.El * cw * SORT_WAVES; i += SORT_THREADS) wcnt[i] = 0;
  __syncthreads();
  int rank[4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    rank[c] = 0;
    if (c < chunks) {
      const int key = le[c] < 0 ? a.El : le[c];
      uint64_t m = ~0ull;
      for (int b = 0; b < a.nbits; b++) {
        const int bit = (key >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      rank[c] = __popcll(m & below);
      if (le[c] >= 0 && rank[c] == 0) wcnt[(le[c] * cw + c) * SORT_WAVES + wave] = __popcll(m);
    }
  }
  __syncthreads();
  const int n = cw * SORT_WAVES;  // 16, 32 or 64 lanes per expert
  for (int e0 = 0; e0 < a.El; e0 += SORT_THREADS / n) {
    const int e = e0 + tid / n, j = tid % n;
    const int v = (e < a.El) ? wcnt[e * n + j] : 0;
    const int x = seg_incl_scan(v, n);
    if (e < a.El) wcnt[e * n + j] = base[e] + x - v;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int64_t r = (int64_t)c * SORT_THREADS + tid;
    if (c < chunks && r < a.R) {
      if (le[c] >= 0) {
        const int slot = wcnt[(le[c] * cw + c) * SORT_WAVES + wave] + rank[c];
        a.e2p[r] = slot;
        a.p2e[slot] = (int32_t)r;
      } else {
        a.e2p[r] = -1;
      }
    }
  }
}

// Spans, kernel 1: per-span histograms; also fills permuted_to_expanded with -1.
__global__ __launch_bounds__(SORT_THREADS) void sort_span_hist_kernel(SortArgs a) {
  extern __shared__ int lds[];
  int* cnt = lds;
  const int w = blockIdx.x;
  for (int i = threadIdx.x; i < a.El; i += SORT_THREADS) cnt[i] = 0;
  for (int64_t s = (int64_t)w * SORT_THREADS + threadIdx.x; s < a.slots; s += (int64_t)a.spans * SORT_THREADS)
    a.p2e[s] = -1;
  __syncthreads();
  int64_t lo = (int64_t)w * a.span_len;
  int64_t hi = min(lo + a.span_len, a.R);
  span_histogram(a, lo, hi, cnt);
  __syncthreads();
  for (int i = threadIdx.x; i < a.El; i += SORT_THREADS) a.scratch[(int64_t)w * a.El + i] = cnt[i];
}

// Spans, kernel 2: every workgroup reads all span histograms, forms the
// expert totals, the slot bases and its own span's base per expert (the
// scan is small: spans x E_l counts), workgroup 0 writes the tables, and
// each workgroup then scatters its span in order.
__global__ __launch_bounds__(SORT_THREADS) void sort_span_scatter_kernel(SortArgs a) {
  extern __shared__ int lds[];
  int* cnt = lds;                     // El
  int* base = cnt + a.El;             // El+1
  int* tbase = base + a.El + 1;       // El+1
  int* tmp = tbase + a.El + 1;        // SORT_WAVES
  int* running = tmp + SORT_WAVES;    // El
  int* wcnt = running + a.El;         // SORT_WAVES * El
  const int w = blockIdx.x;
  for (int e = threadIdx.x; e < a.El; e += SORT_THREADS) {
    int total = 0, before = 0;
    for (int v = 0; v < a.spans; v++) {
      const int c = a.scratch[(int64_t)v * a.El + e];
      if (v < w) before += c;
      total += c;
    }
    cnt[e] = total;
    running[e] = before;
  }
  __syncthreads();
  plan_tables(a, cnt, base, tbase, tmp, w == 0);
  __syncthreads();
  for (int e = threadIdx.x; e < a.El; e += SORT_THREADS) running[e] += base[e];
  __syncthreads();
  int64_t lo = (int64_t)w * a.span_len;
  int64_t hi = min(lo + a.span_len, a.R);
  span_scatter(a, lo, hi, running, wcnt);
}

// ---------------------------------------------------------------- host side

int sort_max_spans(int64_t routes) {
  int64_t s = (routes + SORT_SPAN_MIN - 1) / SORT_SPAN_MIN;
  if (s < 1) s = 1;
  if (s > SORT_MAX_SPANS) s = SORT_MAX_SPANS;
  return (int)s;
}

hipError_t launch_sort(const int32_t* ids, int M, int top_k, int offset, int route_order, const moe_plan_t* plan,
                       hipStream_t stream) {
  SortArgs a;
  a.ids = ids;
  a.R = (int64_t)M * top_k;
  a.El = plan->num_local_experts;
  a.offset = offset;
  a.tile = plan->tile;
  int nb = 0;
  while ((1 << nb) <= a.El) nb++;
  a.nbits = nb;
  a.slots = plan->route_slots;
  a.max_tiles = plan->max_tiles;
  a.e2p = plan->expanded_to_permuted;
  a.p2e = plan->permuted_to_expanded;
  a.tile_expert = plan->tile_to_expert;
  a.tile_limit = plan->tile_to_mn_limit;
  a.num_tiles = plan->num_tiles;
  a.offsets = plan->expert_offsets;
  a.counts = plan->expert_counts;
  a.scratch = plan->scratch;
  bool span = route_order == MOE_ROUTE_ORDER_SPAN ||
              (route_order == MOE_ROUTE_ORDER_AUTO && a.R > SORT_SINGLE_MAX_ROUTES);
  if (a.R == 0) span = false;
  const size_t lds_tables = sizeof(int) * (3 * (size_t)a.El + 2 + SORT_WAVES);
  const size_t lds_wcnt = sizeof(int) * (size_t)SORT_WAVES * a.El;
  if (!span) {
    a.spans = 1;
    a.span_len = a.R;
    // room for the all-chunks counts of the fused path (up to 4096 routes)
    const size_t lds_fused = sizeof(int) * SORT_FUSED_COUNTS;
    sort_single_kernel<<<1, SORT_THREADS, lds_tables + (lds_wcnt > lds_fused ? lds_wcnt : lds_fused), stream>>>(a);
    return hipGetLastError();
  }
  // spans: as many as the scratch allows, each at least SORT_SPAN_MIN routes
  int spans = plan->max_spans;
  int64_t len = (a.R + spans - 1) / spans;
  len = (len + SORT_THREADS - 1) / SORT_THREADS * SORT_THREADS;
  spans = (int)((a.R + len - 1) / len);
  a.spans = spans;
  a.span_len = len;
  sort_span_hist_kernel<<<spans, SORT_THREADS, sizeof(int) * a.El, stream>>>(a);
  sort_span_scatter_kernel<<<spans, SORT_THREADS, lds_tables + sizeof(int) * a.El + lds_wcnt, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
