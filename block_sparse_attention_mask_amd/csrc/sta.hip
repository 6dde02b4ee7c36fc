// Static sliding-tile (STA-style) block mask.
//
// Method: blog review "Fast Video Generation with SLIDING TILE ATTENTION", section
// "Observation & Proposed Method": tokens are grouped into 3D tiles and every query
// of a tile attends to the keys of the tiles in a local 3D window around it; with
// tiles equal to the attention block there are no partially used blocks. Here the
// window is centred on the query tile, cut off at the grid border, and a 64-token
// block pair is kept iff some token of one may see some token of the other.
//
// Two kernels: sta_tiles lists the distinct window tiles touched by each block;
// sta_pairs tests every block pair with those lists. When blocks align with the
// tiles, one kernel tests tile distances directly.
#include "common.h"
#include "launch.h"

namespace bsa {

// (t, h, w) of sequence position p under the token order of g.
__device__ __forceinline__ void token_coord(const StaGeom& g, int p, int& t, int& h, int& w) {
  if (g.order == 0) {
    w = p % g.W;
    h = (p / g.W) % g.H;
    t = p / (g.W * g.H);
    return;
  }
  // tile-major: tiles visited row-major; border tiles are smaller
  const int slab = g.ot * g.H * g.W;           // tokens in a full t-slab of tiles
  const int a = p / slab;
  int rem = p - a * slab;
  const int st = min(g.ot, g.T - a * g.ot);    // t-extent of this slab
  const int rowsz = st * g.oh * g.W;
  const int b = rem / rowsz;
  rem -= b * rowsz;
  const int sh = min(g.oh, g.H - b * g.oh);
  const int tilesz = st * sh * g.ow;
  const int c = rem / tilesz;
  rem -= c * tilesz;
  const int sw = min(g.ow, g.W - c * g.ow);
  t = a * g.ot + rem / (sh * sw);
  h = b * g.oh + (rem / sw) % sh;
  w = c * g.ow + rem % sw;
}

__device__ __forceinline__ int32_t pack_tile(int a, int b, int c) { return (a << 20) | (b << 10) | c; }

// One wave per block, one token per lane: the distinct window tiles of the block's
// real tokens, in first-occurrence order.
__global__ __launch_bounds__(256) void sta_tiles_kernel(StaGeom g, int32_t* __restrict__ tiles) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (i >= g.nb) return;
  const int p = i * BSA_N + l;
  const bool real = p < g.S_valid;
  int32_t key = -1;
  if (real) {
    int t, h, w;
    token_coord(g, p, t, h, w);
    key = pack_tile(t / g.tt, h / g.th, w / g.tw);
  }
  // a lane is the first of its key if no lower lane holds the same key
  bool first = real;
  for (int o = 0; o < 63; ++o) {
    const int other = __shfl(key, o, 64);
    if (o < l && other == key) first = false;
  }
  const uint64_t ball = __ballot(first);
  int32_t* out = tiles + (int64_t)i * (STA_MAX_TILES + 1);
  if (first) out[1 + __popcll(ball & ((1ull << l) - 1ull))] = key;
  if (l == 0) out[0] = __popcll(ball);
}

// One workgroup per query block i; threads sweep the key blocks j. Block i's tiles are
// decoded once into shared memory; block j's list is read 8 entries at a time with
// independent loads, so a pair costs about 1 + n_j / 8 memory round trips.
__global__ __launch_bounds__(256) void sta_pairs_kernel(StaGeom g, const int32_t* __restrict__ tiles,
                                                        uint8_t* __restrict__ mask) {
  __shared__ int16_t ta[3][STA_MAX_TILES];
  __shared__ int nti;
  const int i = blockIdx.x;
  const int32_t* src = tiles + (int64_t)i * (STA_MAX_TILES + 1);
  if (threadIdx.x == 0) nti = src[0];
  if (threadIdx.x < STA_MAX_TILES) {
    const int32_t t = src[1 + threadIdx.x];
    ta[0][threadIdx.x] = (int16_t)(t >> 20);
    ta[1][threadIdx.x] = (int16_t)((t >> 10) & 1023);
    ta[2][threadIdx.x] = (int16_t)(t & 1023);
  }
  __syncthreads();
  const int n_i = nti;
  for (int j = threadIdx.x; j < g.nb; j += 256) {
    const int32_t* tj = tiles + (int64_t)j * (STA_MAX_TILES + 1);
    const int n_j = tj[0];
    bool keep = false;
    for (int y0 = 0; y0 < n_j && !keep; y0 += 8) {
      int32_t c[8];
#pragma unroll
      for (int y = 0; y < 8; ++y) c[y] = y0 + y < n_j ? tj[1 + y0 + y] : -1;
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        if (c[y] < 0) continue;
        const int c0 = c[y] >> 20, c1 = (c[y] >> 10) & 1023, c2 = c[y] & 1023;
        for (int x = 0; x < n_i; ++x)
          keep |= abs(ta[0][x] - c0) <= g.rt && abs(ta[1][x] - c1) <= g.rh && abs(ta[2][x] - c2) <= g.rw;
      }
    }
    mask[(int64_t)i * g.nb + j] = keep ? 1 : 0;
  }
}

// Aligned case: tile-major token order whose tile is the window tile, full tiles only
// (every grid extent a multiple of the tile), a tile a whole number of 64-token
// blocks, no padding. Then every block lies inside one tile, block i's tile is i / bpt,
// and the any-pair rule reduces to the tile-distance test; one kernel, O(1) per pair.
__global__ __launch_bounds__(256) void sta_aligned_kernel(StaRule r, int nb, uint8_t* __restrict__ mask) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j < nb; j += 256) mask[(int64_t)i * nb + j] = sta_rule_keep(r, i, j) ? 1 : 0;
}

StaRule sta_rule_of(const StaGeom& g) {
  const int tile_tokens = g.tt * g.th * g.tw;
  const bool aligned = g.order == 1 && g.ot == g.tt && g.oh == g.th && g.ow == g.tw && g.T % g.tt == 0 &&
                       g.H % g.th == 0 && g.W % g.tw == 0 && tile_tokens % BSA_N == 0 &&
                       g.S_valid == g.T * g.H * g.W && g.S_valid == g.nb * BSA_N;
  StaRule r = {0, 0, 0, 0, 0, 0};
  if (aligned) r = {tile_tokens / BSA_N, g.H / g.th, g.W / g.tw, g.rt, g.rh, g.rw};
  return r;
}

hipError_t launch_sta(const StaGeom& g, int32_t* tiles_ws, uint8_t* mask_out, hipStream_t st) {
  const StaRule r = sta_rule_of(g);
  if (r.bpt) {
    hipLaunchKernelGGL(sta_aligned_kernel, dim3(g.nb), dim3(256), 0, st, r, g.nb, mask_out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(sta_tiles_kernel, dim3((g.nb + 3) / 4), dim3(256), 0, st, g, tiles_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sta_pairs_kernel, dim3(g.nb), dim3(256), 0, st, g, (const int32_t*)tiles_ws, mask_out);
  return hipGetLastError();
}

}  // namespace bsa
