// tile_order.h -- heaviest-first order over the tiles of a routing plan,
// shared by the wide-tile GEMMs.
//
// A plan tile of `tile` slots holds between 1 and `tile` routes; its height
// is the number of 16-slot row groups in use.  Workgroups take the tiles in
// order of decreasing height (tiles of one height in plan order), so that
// the short tiles fill the tail of the launch.
#pragma once
#include "device_common.h"

namespace moe {

// Plan tile of rank r (0 <= r < num_tiles) in the heaviest-first order.
// Called by every thread of a workgroup of `nthreads` threads (a multiple of
// 64, at most 1024); the result is uniform.  Uses LDS and barriers.
DEV int tile_of_rank(const int32_t* tile_limit, int num_tiles, int tile, int r, int nthreads) {
  __shared__ int cls_n[17];
  __shared__ int wave_n[16];
  __shared__ int found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = nthreads >> 6;
  const int groups = tile >> 4;
  auto height = [&](int pt) -> int { return (min(tile, tile_limit[pt] - pt * tile) + 15) >> 4; };
  if (tid <= groups) cls_n[tid] = 0;
  __syncthreads();
  for (int pt = tid; pt < num_tiles; pt += nthreads) atomicAdd(&cls_n[height(pt)], 1);
  __syncthreads();
  int c = groups, before = 0;
  while (before + cls_n[c] <= r) before += cls_n[c--];
  const int k = r - before;  // index among the tiles of height c
  int seen = 0;
  for (int base = 0; base < num_tiles; base += nthreads) {
    const int pt = base + tid;
    const bool hit = pt < num_tiles && height(pt) == c;
    const unsigned long long bal = __ballot(hit);
    if (lane == 0) wave_n[wave] = __popcll(bal);
    __syncthreads();
    int off = seen;
    for (int w = 0; w < wave; w++) off += wave_n[w];
    const int idx = off + __popcll(bal & ((1ull << lane) - 1));
    if (hit && idx == k) found = pt;
    for (int w = 0; w < nwaves; w++) seen += wave_n[w];
    __syncthreads();
    if (seen > k) break;
  }
  return __builtin_amdgcn_readfirstlane(found);
}

}  // namespace moe
