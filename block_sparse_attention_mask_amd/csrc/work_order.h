// Work order of the attention kernel, computed by one workgroup from the kv-list
// lengths (of CSR lists, of fixed-stride lists, or counted straight from a mask).
#pragma once
#include "common.h"
#include "launch.h"

namespace bsa {

constexpr int SCHED_RANGES = 8;   // XCD ranges of the attention work order

// The attention kernel's work item is a pair of adjacent query blocks (2p, 2p+1)
// walking the union of their kv lists. The items are cut into 8 contiguous ranges, one
// per XCD (workgroups are dealt to the XCDs round-robin, so workgroup x runs on XCD
// x % 8): neighbouring query blocks keep sharing one L2. Inside a range the items go
// longest first, by cost(item) = max(|list 2p|, |list 2p+1|), clamped to [0, nb]; equal
// keys in arbitrary order (the attention output does not depend on the order). Slot x
// of the order holds the item of position x / 8 in range x % 8, or -1.
// One workgroup of NT threads (512 or 1024) does it all in shared memory: per-range key
// histograms, a descending scan per range, and a scatter with shared-memory atomics.
// sm: 2 * SCHED_RANGES * (nb + 1) ints of shared memory. Every thread of the workgroup
// must call it.
template <int NT, typename Cost>
__device__ __forceinline__ void pair_schedule_block(Cost cost, int BH, int nb, int32_t* __restrict__ order, int* sm) {
  static_assert(NT == 512 || NT == 1024, "one or two waves per range");
  constexpr int TPR = NT / SCHED_RANGES;             // threads per range
  const int nk = nb + 1, npair = (nb + 1) / 2, items = BH * npair;
  const int maxg = (items + SCHED_RANGES - 1) / SCHED_RANGES;
  int* hist = sm;                                    // [ranges][nk]
  int* cur = sm + SCHED_RANGES * nk;                 // [ranges][nk]: descending starts, then cursors
  __shared__ int part[SCHED_RANGES][2];
  __shared__ int gsize[SCHED_RANGES];
  const int t = threadIdx.x;
  for (int x = t; x < 2 * SCHED_RANGES * nk; x += NT) sm[x] = 0;
  __syncthreads();
  constexpr int PER = PAIR_SCHED_MAX_ITEMS / NT;
  int key[PER], grp[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int it = t + r * NT;
    key[r] = -1;
    grp[r] = 0;
    if (it < items) {
      key[r] = min(max(cost(it), 0), nb);
      grp[r] = (int)(((int64_t)it * SCHED_RANGES) / items);
      atomicAdd(&hist[grp[r] * nk + key[r]], 1);
    }
  }
  __syncthreads();
  // descending exclusive scan of each range's histogram: TPR threads per range, each
  // summing a chunk of keys (largest keys first), then a scan of the chunk sums
  {
    const int g = t / TPR, c = t % TPR;
    const int per = (nk + TPR - 1) / TPR;
    const int k1 = nk - 1 - c * per;                 // chunk: k1, k1-1, ..., k1-per+1
    int sum = 0;
    for (int e = 0; e < per; ++e)
      if (k1 - e >= 0) sum += hist[g * nk + k1 - e];
    const int incl = wave_incl_scan_i32(sum);
    int run = incl - sum;
    if constexpr (TPR == 128) {   // two waves per range: the first wave's total goes to the second
      if ((c & 63) == 63) part[g][c >> 6] = incl;
      __syncthreads();
      if (c >= 64) run += part[g][0];
    }
    if (c == TPR - 1) gsize[g] = run + sum;
    for (int e = 0; e < per; ++e)
      if (k1 - e >= 0) { cur[g * nk + k1 - e] = run; run += hist[g * nk + k1 - e]; }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    if (key[r] >= 0) {
      const int pos = atomicAdd(&cur[grp[r] * nk + key[r]], 1);
      order[pos * SCHED_RANGES + grp[r]] = t + r * NT;
    }
  }
  // slots past the end of a range
  for (int x = t; x < maxg * SCHED_RANGES; x += NT)
    if (x / SCHED_RANGES >= gsize[x % SCHED_RANGES]) order[x] = -1;
}

}  // namespace bsa
