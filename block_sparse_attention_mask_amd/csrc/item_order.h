// Work orders derived inside a kernel from kv-list lengths (shared by the attention
// forward and backward kernels).
#pragma once
#include "common.h"

namespace bsa {

// Query blocks of pair p (of ceil(nb / 2)) when a head's blocks are paired at offset d >= 1:
// the blocks are taken in runs of 2d, block a of a run's first half paired with a + d; the
// blocks after the last whole run pair with their neighbour. d = 1: pairs (2p, 2p + 1).
// y = -1 when the pair has one block (odd nb).
__host__ __device__ inline int2 pair_blocks(int p, int d, int nb) {
  const int full = nb / (2 * d) * (2 * d);
  if (2 * p < full) {
    const int r = p / d, a = 2 * r * d + (p - r * d);
    return make_int2(a, a + d);
  }
  const int a = full + 2 * (p - full / 2);
  return make_int2(a, a + 1 < nb ? a + 1 : -1);
}

// Union walk over the bit rows of two kv lists (word w of a row holds the row's blocks
// 64 w .. 64 w + 63): ascending blocks of either row with use flags (bit 0: row a holds
// the block, bit 1: row b), -1 at the end. Wave-uniform scalar state; one scalar load per
// word of each row.
struct BitUnionWalk {
  using CU64 = const uint64_t __attribute__((address_space(4)));
  CU64* ra;
  CU64* rb;   // NULL: no second row
  int nw, wi;
  uint64_t ca, cb;
  __device__ void init(const uint64_t* bits, int64_t row_a, int64_t row_b, int nw_) {
    nw = nw_;
    ra = (CU64*)(uintptr_t)(bits + row_a * nw);
    rb = row_b >= 0 ? (CU64*)(uintptr_t)(bits + row_b * nw) : nullptr;
    wi = -1;
    ca = cb = 0;
  }
  __device__ int next(int& flags) {
    while ((ca | cb) == 0) {
      if (++wi >= nw) { flags = 0; return -1; }
      ca = ra[wi];
      cb = rb ? rb[wi] : 0ull;
    }
    const int t = __builtin_ctzll(ca | cb);
    flags = (int)((ca >> t) & 1ull) | (int)(((cb >> t) & 1ull) << 1);
    ca &= ~(1ull << t);
    cb &= ~(1ull << t);
    return 64 * wi + t;
  }
};

// Item it = (head, pair p) costs the longer of the pair's two lists (rows of
// pair_blocks(p, d) of head it / npair, d = pair_d[head], or 1 without pair_d), clamped
// to [0, nb].
// kth_longest_item returns the item at position k of the items [lo, lo + R) ordered by
// decreasing cost, equal costs in ascending item order, so that every workgroup derives
// the same order by itself: a cost histogram in shared memory, a descending scan of it
// by one wave (the cost at position k and the number of items above it), then one
// wave's ballots over the range find the item. sm: kth_longest_ints(nb, R) ints; the
// trailing barrier lets the caller reuse them at once. All NT threads of the workgroup
// call it. A caller whose shared buffer is smaller (kth_longest_fits false) keeps the
// natural order instead: the order never changes what is computed.
__host__ __device__ constexpr int kth_longest_ints(int nb, int R) { return nb + 1 + R + 3; }
__host__ __device__ constexpr bool kth_longest_fits(int nb, int R, int sm_bytes) {
  return kth_longest_ints(nb, R) <= sm_bytes / 4;
}
template <int NT, typename Len>
__device__ int kth_longest_item(Len len, int nb, int* sm, int lo, int R, int k, const int32_t* pair_d = nullptr) {
  const int npair = (nb + 1) / 2;
  const int t = threadIdx.x, lane = t & 63, nk = nb + 1;
  int* hist = sm;
  int* cost = sm + nk;
  int* res = cost + R;
  for (int x = t; x < nk; x += NT) hist[x] = 0;
  __syncthreads();
  for (int i = t; i < R; i += NT) {
    const int it = lo + i, bh = it / npair;
    const int2 pb = pair_blocks(it - bh * npair, pair_d ? pair_d[bh] : 1, nb);
    int c = len(bh * nb + pb.x);
    if (pb.y >= 0) c = max(c, len(bh * nb + pb.y));
    if (!BSA_CHECK(c >= 0 && c <= nb, CHK_ATTN_LEN)) c = min(max(c, 0), nb);   // (histogram index)
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
