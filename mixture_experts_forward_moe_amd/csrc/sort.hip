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
//    one 1024-thread workgroup;
//  - spans (large route counts): each workgroup owns one contiguous span of
//    routes; kernel 1 writes per-span expert histograms, kernel 2 scans them
//    across spans and experts and writes the tile tables, kernel 3 scatters
//    each span in order.  Every workgroup stops at its own span end.
// Inside a span, routes are ranked 1024 at a time: wavefront ballots give a
// route's rank among equal experts in its wavefront, and an LDS prefix over
// the 16 wavefronts gives the rest.
#include "device_common.h"
#include "internal.h"

namespace moe {

constexpr int SORT_THREADS = 1024;
constexpr int SORT_WAVES = SORT_THREADS / 64;

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
  int x = s;
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
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
DEV void plan_tables(const SortArgs& a, const int* cnt, int* base, int* tbase, int* tmp) {
  const int T = a.tile;
  for (int le = threadIdx.x; le < a.El; le += SORT_THREADS) {
    int c = cnt[le];
    int nt = (c + T - 1) / T;
    base[le] = nt * T;
    tbase[le] = nt;
    a.counts[le] = c;
  }
  __syncthreads();
  int total_slots = block_exclusive_scan(base, a.El, tmp);
  int total_tiles = block_exclusive_scan(tbase, a.El, tmp);
  if (threadIdx.x == 0) {
    base[a.El] = total_slots;
    tbase[a.El] = total_tiles;
    a.offsets[a.El] = total_slots;
    *a.num_tiles = total_tiles;
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

// Stable scatter of routes [lo, hi): running[le] (LDS) holds the next slot
// of expert le and is advanced.  wcnt: LDS [SORT_WAVES][El].
DEV void span_scatter(const SortArgs& a, int64_t lo, int64_t hi, int* running, int* wcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = lo; c0 < hi; c0 += SORT_THREADS) {
    for (int i = tid; i < SORT_WAVES * a.El; i += SORT_THREADS) wcnt[i] = 0;
    int64_t r = c0 + tid;
    int le = (r < hi) ? local_expert(a, r) : -1;
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
    if (le >= 0 && rank == 0) wcnt[wave * a.El + le] = cnt;
    __syncthreads();
    for (int e = tid; e < a.El; e += SORT_THREADS) {
      int run = running[e];
      for (int w = 0; w < SORT_WAVES; w++) {
        int c = wcnt[w * a.El + e];
        wcnt[w * a.El + e] = run;
        run += c;
      }
      running[e] = run;
    }
    __syncthreads();
    if (r < hi) {
      if (le >= 0) {
        int slot = wcnt[wave * a.El + le] + rank;
        a.e2p[r] = slot;
        a.p2e[slot] = (int32_t)r;
      } else {
        a.e2p[r] = -1;
      }
    }
    __syncthreads();
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
  __syncthreads();
  span_histogram(a, 0, a.R, cnt);
  __syncthreads();
  plan_tables(a, cnt, base, tbase, tmp);
  __syncthreads();
  span_scatter(a, 0, a.R, base, wcnt);
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

// Spans, kernel 2 (one workgroup): expert totals, per-span bases, tables.
__global__ __launch_bounds__(SORT_THREADS) void sort_span_scan_kernel(SortArgs a) {
  extern __shared__ int lds[];
  int* cnt = lds;
  int* base = cnt + a.El;
  int* tbase = base + a.El + 1;
  int* tmp = tbase + a.El + 1;
  for (int e = threadIdx.x; e < a.El; e += SORT_THREADS) {
    int run = 0;
    for (int w = 0; w < a.spans; w++) {
      int c = a.scratch[(int64_t)w * a.El + e];
      a.scratch[(int64_t)w * a.El + e] = run;  // exclusive prefix over spans
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  plan_tables(a, cnt, base, tbase, tmp);
  __syncthreads();
  // span bases become absolute slots
  for (int64_t i = threadIdx.x; i < (int64_t)a.spans * a.El; i += SORT_THREADS)
    a.scratch[i] += base[i % a.El];
}

// Spans, kernel 3: stable scatter of each span.
__global__ __launch_bounds__(SORT_THREADS) void sort_span_scatter_kernel(SortArgs a) {
  extern __shared__ int lds[];
  int* running = lds;                 // El
  int* wcnt = running + a.El;         // SORT_WAVES * El
  const int w = blockIdx.x;
  for (int e = threadIdx.x; e < a.El; e += SORT_THREADS) running[e] = a.scratch[(int64_t)w * a.El + e];
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
    sort_single_kernel<<<1, SORT_THREADS, lds_tables + lds_wcnt, stream>>>(a);
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
  sort_span_scan_kernel<<<1, SORT_THREADS, lds_tables, stream>>>(a);
  sort_span_scatter_kernel<<<spans, SORT_THREADS, sizeof(int) * a.El + lds_wcnt, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
