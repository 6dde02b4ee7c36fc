// Work orders derived inside a kernel from kv-list lengths (shared by the attention
// forward and backward kernels).
#pragma once
#include "common.h"

namespace bsa {

// Item it = (head, pair p of adjacent rows 2p, 2p+1) costs the longer of the pair's two
// lists, len(row) for rows (it / npair) * nb + 2p (+1), clamped to [0, nb].
// kth_longest_item returns the item at position k of the items [lo, lo + R) ordered by
// decreasing cost, equal costs in ascending item order, so that every workgroup derives
// the same order by itself: a cost histogram in shared memory, a descending scan of it
// by one wave (the cost at position k and the number of items above it), then one
// wave's ballots over the range find the item. sm: nb + 1 + R + 3 ints; the trailing
// barrier lets the caller reuse them at once. All NT threads of the workgroup call it.
template <int NT, typename Len>
__device__ int kth_longest_item(Len len, int nb, int* sm, int lo, int R, int k) {
  const int npair = (nb + 1) / 2;
  const int t = threadIdx.x, lane = t & 63, nk = nb + 1;
  int* hist = sm;
  int* cost = sm + nk;
  int* res = cost + R;
  for (int x = t; x < nk; x += NT) hist[x] = 0;
  __syncthreads();
  for (int i = t; i < R; i += NT) {
    const int it = lo + i, p = it % npair, rA = (it / npair) * nb + 2 * p;
    int c = len(rA);
    if (2 * p + 1 < nb) c = max(c, len(rA + 1));
    c = min(max(c, 0), nb);
    cost[i] = c;
    atomicAdd(&hist[c], 1);
  }
  __syncthreads();
  if (t < 64) {
    // lane chunks of keys in descending order; the chunk holding position k names the
    // cost K there and the number of items with a larger cost
    const int per = (nk + 63) / 64, k1 = nk - 1 - lane * per;
    int sum = 0;
    for (int e = 0; e < per; ++e)
      if (k1 - e >= 0) sum += hist[k1 - e];
    const int incl = wave_incl_scan_i32(sum);
    int run = incl - sum;
    if (run <= k && k < incl) {
      for (int e = 0; e < per; ++e) {
        const int key = k1 - e;
        if (key < 0) break;
        if (k < run + hist[key]) { res[0] = key; res[1] = run; break; }
        run += hist[key];
      }
    }
  }
  __syncthreads();
  const int K = res[0], need = k - res[1];         // the need-th item (ascending) of cost K
  if (t < 64) {
    int base = 0;
    for (int i0 = 0; i0 < R; i0 += 64) {
      const bool f = i0 + lane < R && cost[i0 + lane] == K;
      const uint64_t b = __ballot(f);
      const int n = __popcll(b);
      if (need < base + n) {
        if (f && __popcll(b & ((1ull << lane) - 1ull)) == need - base) res[2] = lo + i0 + lane;
        break;
      }
      base += n;
    }
  }
  __syncthreads();
  const int item = res[2];
  __syncthreads();
  return item;
}

}  // namespace bsa
