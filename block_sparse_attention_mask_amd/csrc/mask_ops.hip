// Mask union and mask -> per-query-block kv index lists (CSR).
//
// The union follows the NABLA review ("What carries the argument": the adaptive mask
// is optionally OR'd with a sliding-tile mask); the index lists are the "skip lists"
// of the CalibAtt page: the attention kernel visits only the listed blocks.
#include "common.h"
#include "launch.h"
#include "item_order.h"
#include "work_order.h"

namespace bsa {

__global__ __launch_bounds__(256) void mask_or_kernel(uint8_t* __restrict__ dst, const uint8_t* a, int64_t n,
                                                      const uint8_t* __restrict__ b, int64_t b_n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += stride)
    dst[x] = (a[x] | b[x % b_n]) ? 1 : 0;
}

hipError_t launch_mask_or(uint8_t* dst, const uint8_t* a, int64_t n, const uint8_t* b, int64_t b_n,
                          hipStream_t st) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(mask_or_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dst, a, n, b, b_n);
  return hipGetLastError();
}

// one wave per row: number of kept blocks
__global__ __launch_bounds__(256) void csr_count_kernel(const uint8_t* __restrict__ mask, int64_t sb,
                                                        int64_t sh, int H, int nb, int rows,
                                                        int32_t* __restrict__ counts) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / nb, i = row % nb;
  const uint8_t* m = mask + (bh / H) * sb + (bh % H) * sh + (int64_t)i * nb;
  int c = 0;
  for (int j = l; j < nb; j += 64) c += m[j] != 0;
  c = wave_sum_i32(c);
  if (l == 0) counts[row] = c;
}

// Exclusive scan of the row counts into row_ptr[0..rows], in two passes:
// csr_block_sum_kernel reduces each 1024-row segment; csr_scan_kernel scans the
// segment sums (in shared memory) and then its own segment.
constexpr int SCAN_SEG = 1024;
__device__ __forceinline__ int block_excl_scan_1024(int v, int* sh, int& total) {
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int incl = wave_incl_scan_i32(v);
  if (l == 63) sh[w] = incl;
  __syncthreads();
  if (t < 16) {
    int x = sh[t];
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(x, o, 16);
      if (t >= o) x += y;
    }
    sh[16 + t] = x;     // inclusive scan of the wave sums
  }
  __syncthreads();
  total = sh[31];
  const int r = incl - v + (w ? sh[16 + w - 1] : 0);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void csr_block_sum_kernel(const int32_t* __restrict__ counts, int rows,
                                                             int32_t* __restrict__ seg_sum) {
  __shared__ int sh[32];
  const int r = blockIdx.x * SCAN_SEG + threadIdx.x;
  int total;
  block_excl_scan_1024(r < rows ? counts[r] : 0, sh, total);
  if (threadIdx.x == 0) seg_sum[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void csr_scan_kernel(const int32_t* __restrict__ counts, int rows,
                                                        const int32_t* __restrict__ seg_sum, int nseg,
                                                        int32_t* __restrict__ row_ptr) {
  __shared__ int sh[32];
  __shared__ int base_sh;
  // offset of this segment: sum of the earlier segment sums
  int part = 0;
  for (int x = threadIdx.x; x < (int)blockIdx.x; x += SCAN_SEG) part += seg_sum[x];
  int tot_part;
  block_excl_scan_1024(part, sh, tot_part);
  if (threadIdx.x == 0) base_sh = tot_part;
  __syncthreads();
  const int base = base_sh;
  const int r = blockIdx.x * SCAN_SEG + threadIdx.x;
  const int v = r < rows ? counts[r] : 0;
  int total;
  const int ex = block_excl_scan_1024(v, sh, total);
  if (r < rows) row_ptr[r] = base + ex;
  if (blockIdx.x == nseg - 1 && threadIdx.x == 0) row_ptr[rows] = base + total;
}

// one wave per row: ascending kept column indices
__global__ __launch_bounds__(256) void csr_fill_kernel(const uint8_t* __restrict__ mask, int64_t sb, int64_t sh,
                                                       int H, int nb, int rows,
                                                       const int32_t* __restrict__ row_ptr,
                                                       int32_t* __restrict__ col_idx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  const int bh = row / nb, i = row % nb;
  const uint8_t* m = mask + (bh / H) * sb + (bh % H) * sh + (int64_t)i * nb;
  int32_t* out = col_idx + row_ptr[row];
  int base = 0;
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + l;
    const bool f = j < nb && m[j] != 0;
    const uint64_t ball = __ballot(f);
    if (f) out[base + __popcll(ball & ((1ull << l) - 1ull))] = j;
    base += __popcll(ball);
  }
}

// Small masks (few rows, nb a multiple of 16, nb <= 512; contiguous [B,H,nb,nb] or
// one [nb,nb] plane for every head) in one launch instead of four. Workgroup x owns rows [64x, 64x + 64). It counts the kept entries of all
// earlier rows itself (16-byte chunks, a row is nb/16 chunks, 16 loads in flight per
// thread, 1024 threads; the mask is small, so the repeated reads stay in L2), stages its own rows
// in shared memory, counts them with wave ballots, scans the counts, and writes
// row_ptr and the ascending kept indices.

constexpr int CSR_SMALL_ROWS = 4096;
constexpr int CSR_SMALL_NB = 512;
constexpr int CSR_SMALL_RPW = 64;                     // rows per workgroup
__global__ __launch_bounds__(1024) void csr_small_kernel(const uint8_t* __restrict__ mask, int64_t sb, int64_t sh,
                                                        int H, int nb, int rows, int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx,
                                                        int32_t* __restrict__ pair_order) {
  __shared__ __attribute__((aligned(16))) uint8_t own[CSR_SMALL_RPW * CSR_SMALL_NB];
  __shared__ int rc[CSR_SMALL_RPW];
  __shared__ int red[16];
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  const int row0 = blockIdx.x * CSR_SMALL_RPW;
  const int nown = min(CSR_SMALL_RPW, rows - row0);
  const int cpr = nb / 16;
  // 16-byte chunk c of the row-major [rows][nb] mask: contiguous, or one plane repeated
  const int plane = nb * nb;
  auto chunk = [&](int c) {
    const int off = sb == 0 ? (c * 16) % plane : c * 16;
    return *(const i32x4_t*)(mask + off);
  };
  auto nz16 = [](i32x4_t v) {                          // nonzero bytes of a chunk
    int n = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned x = (unsigned)v[e];
      n += __popc((((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u);
    }
    return n;
  };
  constexpr int NL = 16;
  if (pair_order && blockIdx.x == gridDim.x - 1) {
    // the extra last workgroup: kept count of every row straight from the mask (in the
    // row buffer), then the attention work order from them, beside the compaction
    int* cnt = (int*)own;
    for (int r = t; r < rows; r += 1024) cnt[r] = 0;
    __syncthreads();
    const int nall = rows * cpr;
    for (int c0 = 0; c0 < nall; c0 += 1024 * NL) {
      i32x4_t v[NL];
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        const int c = c0 + t + k * 1024;
        v[k] = c < nall ? chunk(c) : i32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        const int c = c0 + t + k * 1024, n = nz16(v[k]);
        if (c < nall && n) atomicAdd(&cnt[c / cpr], n);
      }
    }
    __syncthreads();
    extern __shared__ int sched_sm[];
    const int npair = (nb + 1) / 2;
    pair_schedule_block<1024>(
        [&](int it) {
          const int rA = (it / npair) * nb + 2 * (it % npair);
          return max(cnt[rA], 2 * (it % npair) + 1 < nb ? cnt[rA + 1] : 0);
        },
        rows / nb, nb, pair_order, sched_sm);
    return;
  }
  // ---- stage the own rows
  for (int c = t; c < nown * cpr; c += 1024) *(i32x4_t*)(own + c * 16) = chunk(row0 * cpr + c);
  // ---- kept entries before row0
  int part = 0;
  const int nchunk = row0 * cpr;
  for (int c0 = 0; c0 < nchunk; c0 += 1024 * NL) {
    i32x4_t v[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int c = c0 + t + k * 1024;
      v[k] = c < nchunk ? chunk(c) : i32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) part += nz16(v[k]);
  }
  part = wave_sum_i32(part);
  if (l == 0) red[w] = part;
  __syncthreads();
  // ---- own rows: counts by ballot (wave w takes rows w, w + 16, ...)
  for (int r = w; r < nown; r += 16) {
    int cnt = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) cnt += __popcll(__ballot(j0 + l < nb && own[r * nb + j0 + l] != 0));
    if (l == 0) rc[r] = cnt;
  }
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int x = 0; x < 16; ++x) base += red[x];
  if (w == 0) {                                        // exclusive scan of the row counts
    const int x = l < nown ? rc[l] : 0;
    const int incl = wave_incl_scan_i32(x);
    if (l < nown) row_ptr[row0 + l] = base + incl - x;
    if (row0 + l == rows - 1) row_ptr[rows] = base + incl;
    if (l < nown) rc[l] = base + incl - x;
  }
  __syncthreads();
  for (int r = w; r < nown; r += 16) {
    int32_t* out = col_idx + rc[r];
    int pos = 0;
    for (int j0 = 0; j0 < nb; j0 += 64) {
      const bool f = j0 + l < nb && own[r * nb + j0 + l] != 0;
      const uint64_t ball = __ballot(f);
      if (f) out[pos + __popcll(ball & ((1ull << l) - 1ull))] = j0 + l;
      pos += __popcll(ball);
    }
  }
}

hipError_t launch_csr(const uint8_t* mask, int64_t sb, int64_t sh, int B, int H, int nb, int32_t* row_ptr,
                      int32_t* col_idx, int32_t* counts, hipStream_t st, int32_t* pair_order) {
  const int rows = B * H * nb;
  const bool dense = (H == 1 || sh == (int64_t)nb * nb) && (B == 1 || sb == (int64_t)H * nb * nb) && (sb || sh);
  const bool plane = sb == 0 && sh == 0;
  if (nb % 16 == 0 && ((uintptr_t)mask & 15) == 0 && (dense || plane) && rows <= CSR_SMALL_ROWS &&
      nb <= CSR_SMALL_NB) {
    if (dense) sb = 1;                                 // kernel: sb == 0 means one repeated plane
    // with a pair order: one more workgroup, which builds it from the mask's row counts
    const unsigned g = (rows + CSR_SMALL_RPW - 1) / CSR_SMALL_RPW + (pair_order ? 1 : 0);
    const size_t dyn = pair_order ? (size_t)2 * SCHED_RANGES * (nb + 1) * 4 : 0;
    hipLaunchKernelGGL(csr_small_kernel, dim3(g), dim3(1024), dyn, st, mask, sb, sh, H, nb, rows, row_ptr, col_idx,
                       pair_order);
    return hipGetLastError();
  }
  const unsigned g = (unsigned)((rows + 3) / 4);
  hipLaunchKernelGGL(csr_count_kernel, dim3(g), dim3(256), 0, st, mask, sb, sh, H, nb, rows, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nseg = (rows + SCAN_SEG - 1) / SCAN_SEG;
  int32_t* seg_sum = counts + rows;
  hipLaunchKernelGGL(csr_block_sum_kernel, dim3(nseg), dim3(1024), 0, st, (const int32_t*)counts, rows, seg_sum);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_scan_kernel, dim3(nseg), dim3(1024), 0, st, (const int32_t*)counts, rows,
                     (const int32_t*)seg_sum, nseg, row_ptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_fill_kernel, dim3(g), dim3(256), 0, st, mask, sb, sh, H, nb, rows,
                     (const int32_t*)row_ptr, col_idx);
  e = hipGetLastError();
  if (e != hipSuccess || !pair_order) return e;
  return launch_pair_schedule(row_ptr, B * H, nb, pair_order, st);
}

// ---------------------------------------------------------------------------
// Longest-first orders (a work list sorted by decreasing cost, so that the longest
// items start first and the short ones fill the tail).

// Descending exclusive scan of n counters by one block of 1024 threads:
// out[c] = sum of cnt[c'] over c' > c. Thread t handles a contiguous chunk.
__device__ void desc_excl_scan_block(const int32_t* cnt, int n, int32_t* out, int* sh) {
  const int per = (n + 1023) / 1024;
  const int c1 = n - 1 - threadIdx.x * per;          // chunk: c1, c1-1, ..., c1-per+1 (descending)
  int part = 0;
  for (int e = 0; e < per; ++e) {
    const int c = c1 - e;
    if (c >= 0) part += cnt[c];
  }
  int total;
  int run = block_excl_scan_1024(part, sh, total);
  for (int e = 0; e < per; ++e) {
    const int c = c1 - e;
    if (c >= 0) { out[c] = run; run += cnt[c]; }
  }
}

// Rows (b,h,i) sorted by kept count, descending, ties by ascending row index: a
// stable counting sort over blocks of LPT_W waves (64 rows each).
//   lpt_hist_kernel    per-block count histograms hist[blk][c]
//   lpt_scan_kernel    per count c, exclusive scan over the blocks (in place), and
//                      gstart[c] = number of rows with a larger count
//   lpt_scatter_kernel rank inside a block: equal counts of one wave ranked by lane,
//                      earlier waves of the block before later ones
__global__ __launch_bounds__(1024) void lpt_hist_kernel(const int32_t* __restrict__ row_ptr, int rows, int nk,
                                                        int per_blk, int32_t* __restrict__ hist) {
  extern __shared__ int h[];
  for (int c = threadIdx.x; c < nk; c += blockDim.x) h[c] = 0;
  __syncthreads();
  const int r = blockIdx.x * per_blk + threadIdx.x;
  if (threadIdx.x < per_blk && r < rows) atomicAdd(&h[row_ptr[r + 1] - row_ptr[r]], 1);
  __syncthreads();
  int32_t* out = hist + (int64_t)blockIdx.x * nk;
  for (int c = threadIdx.x; c < nk; c += blockDim.x) out[c] = h[c];
}

__global__ __launch_bounds__(1024) void lpt_scan_kernel(int32_t* __restrict__ hist, int nblk, int nk,
                                                        int32_t* __restrict__ tot, int32_t* __restrict__ gstart) {
  __shared__ int sh[32];
  for (int c = threadIdx.x; c < nk; c += 1024) {
    int run = 0;
    int b = 0;
    for (; b + 4 <= nblk; b += 4) {
      const int t0 = hist[(int64_t)b * nk + c], t1 = hist[(int64_t)(b + 1) * nk + c];
      const int t2 = hist[(int64_t)(b + 2) * nk + c], t3 = hist[(int64_t)(b + 3) * nk + c];
      hist[(int64_t)b * nk + c] = run;
      hist[(int64_t)(b + 1) * nk + c] = run + t0;
      hist[(int64_t)(b + 2) * nk + c] = run + t0 + t1;
      hist[(int64_t)(b + 3) * nk + c] = run + t0 + t1 + t2;
      run += t0 + t1 + t2 + t3;
    }
    for (; b < nblk; ++b) {
      const int t = hist[(int64_t)b * nk + c];
      hist[(int64_t)b * nk + c] = run;
      run += t;
    }
    tot[c] = run;
  }
  __threadfence_block();
  __syncthreads();
  desc_excl_scan_block(tot, nk, gstart, sh);
}

__global__ __launch_bounds__(1024) void lpt_scatter_kernel(const int32_t* __restrict__ row_ptr, int rows, int nk,
                                                           const int32_t* __restrict__ hist,
                                                           const int32_t* __restrict__ gstart,
                                                           int32_t* __restrict__ order) {
  extern __shared__ int cnt[];                       // [waves][nk]
  const int nw = blockDim.x >> 6;
  for (int x = threadIdx.x; x < nw * nk; x += blockDim.x) cnt[x] = 0;
  __syncthreads();
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  const int c = r < rows ? row_ptr[r + 1] - row_ptr[r] : -1;
  // rank among the lanes of this wave with the same count and a lower lane
  int rank = 0;
  uint64_t todo = __ballot(c >= 0);
  while (todo) {
    const int lc = __shfl(c, __ffsll((unsigned long long)todo) - 1, 64);
    const uint64_t m = __ballot(c == lc);
    if (c == lc) rank = __popcll(m & ((1ull << l) - 1ull));
    if (l == 0) cnt[w * nk + lc] = __popcll(m);
    todo &= ~m;
  }
  __syncthreads();
  if (c >= 0) {
    int before = 0;
    for (int w2 = 0; w2 < w; ++w2) before += cnt[w2 * nk + c];
    order[gstart[c] + hist[(int64_t)blockIdx.x * nk + c] + before + rank] = r;
  }
}

int lpt_rows_block(int nk) {
  // waves per block: the per-wave count table has to fit in 64 KB of shared memory
  int w = (64 * 1024) / (nk * 4);
  return w > 16 ? 16 : w;
}

size_t lpt_rows_ws_ints(int rows, int nk) {
  const int w = lpt_rows_block(nk);
  if (w < 1) return 0;
  const int nblk = (rows + 64 * w - 1) / (64 * w);
  return (size_t)nblk * nk + 2 * (size_t)nk;
}

hipError_t launch_lpt_rows(const int32_t* row_ptr, int rows, int nb, int32_t* ws, int32_t* order, hipStream_t st) {
  const int nk = nb + 1;
  const int w = lpt_rows_block(nk);
  if (w < 1) return hipErrorInvalidValue;
  const int per_blk = 64 * w;
  const int nblk = (rows + per_blk - 1) / per_blk;
  int32_t* hist = ws;
  int32_t* tot = ws + (size_t)nblk * nk;
  int32_t* gstart = tot + nk;
  hipLaunchKernelGGL(lpt_hist_kernel, dim3(nblk), dim3(per_blk), nk * 4, st, row_ptr, rows, nk, per_blk, hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lpt_scan_kernel, dim3(1), dim3(1024), 0, st, hist, nblk, nk, tot, gstart);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lpt_scatter_kernel, dim3(nblk), dim3(per_blk), w * nk * 4, st, row_ptr, rows, nk,
                     (const int32_t*)hist, (const int32_t*)gstart, order);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void pair_schedule_kernel(const int32_t* __restrict__ row_ptr, int BH, int nb,
                                                             int32_t* __restrict__ order) {
  extern __shared__ int sm[];
  const int npair = (nb + 1) / 2;
  pair_schedule_block<1024>(
      [&](int it) {
        const int bh = it / npair, i = 2 * (it % npair);
        const int rA = bh * nb + i;
        const int cA = row_ptr[rA + 1] - row_ptr[rA];
        const int cB = i + 1 < nb ? row_ptr[rA + 2] - row_ptr[rA + 1] : 0;
        return max(cA, cB);
      },
      BH, nb, order, sm);
}

bool pair_schedule_fits(int BH, int nb) {
  return (int64_t)BH * ((nb + 1) / 2) <= PAIR_SCHED_MAX_ITEMS && nb + 1 <= PAIR_SCHED_MAX_NB + 1;
}

int pair_schedule_slots(int BH, int nb) {
  const int items = BH * ((nb + 1) / 2);
  return ((items + SCHED_RANGES - 1) / SCHED_RANGES) * SCHED_RANGES;
}

__global__ __launch_bounds__(1024) void pair_schedule_len_kernel(const int32_t* __restrict__ kv_len, int BH, int nb,
                                                                 int32_t* __restrict__ order) {
  extern __shared__ int sm[];
  const int npair = (nb + 1) / 2;
  pair_schedule_block<1024>(
      [&](int it) {
        const int p = it % npair, rA = (it / npair) * nb + 2 * p;
        return max(kv_len[rA], 2 * p + 1 < nb ? kv_len[rA + 1] : 0);
      },
      BH, nb, order, sm);
}

hipError_t launch_pair_schedule_len(const int32_t* kv_len, int BH, int nb, int32_t* order, hipStream_t st) {
  hipLaunchKernelGGL(pair_schedule_len_kernel, dim3(1), dim3(1024), 2 * SCHED_RANGES * (nb + 1) * 4, st, kv_len, BH,
                     nb, order);
  return hipGetLastError();
}

hipError_t launch_pair_schedule(const int32_t* row_ptr, int BH, int nb, int32_t* order, hipStream_t st) {
  const int nk = nb + 1;
  hipLaunchKernelGGL(pair_schedule_kernel, dim3(1), dim3(1024), 2 * SCHED_RANGES * nk * 4, st, row_ptr, BH, nb,
                     order);
  return hipGetLastError();
}

static size_t pairing_al256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- pairing offsets
//
// A workgroup walks the union of its two query blocks' kv lists, so each kv tile that only
// one of them keeps costs the other block's waves a step. Adjacent blocks are not always
// the most alike: in row-major video layouts a block's list is often closer to the block
// one frame later. The offset d of each head minimises the number of union steps over the
// pairings pair_blocks(., d): the lists become bit rows, then each candidate d is costed
// by popcounts of ORed rows.

// bits[r][w] = bit j - 64 w set iff row r's list holds key block j (64 w <= j < 64 w + 64).
// One wave per row: the row's words are cleared in shared memory, every list entry ORs its
// bit in (LDS atomics), and the words are written out. Shared memory: 4 rows x nw words.
__global__ __launch_bounds__(256) void row_bits_kernel(const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       const int32_t* __restrict__ row_len, int row_stride,
                                                       int64_t rows, int nw, uint64_t* __restrict__ bits) {
  extern __shared__ unsigned long long row_words[];
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  unsigned long long* w = row_words + wv * nw;
  for (int x = l; x < nw; x += 64) w[x] = 0ull;
  __syncthreads();
  if (r < rows) {
    int lo, hi;
    if (row_len) {
      lo = (int)(r * row_stride);
      hi = lo + row_len[r];
    } else {
      lo = row_ptr[r];
      hi = row_ptr[r + 1];
    }
    for (int e = lo + l; e < hi; e += 64) {
      const int j = col_idx[e];
      if (BSA_CHECK((unsigned)j < (unsigned)(64 * nw), CHK_ROW_BITS)) atomicOr(&w[j >> 6], 1ull << (j & 63));
    }
  }
  __syncthreads();
  if (r < rows)
    for (int x = l; x < nw; x += 64) bits[r * nw + x] = w[x];
}

// cost[bh][d - 1] = sum over the pairs of pair_blocks(., d) of |list(a) u list(b)|; grid (BH, dmax)
__global__ __launch_bounds__(256) void pair_cost_kernel(const uint64_t* __restrict__ bits, int nb, int nw,
                                                        unsigned long long* __restrict__ cost) {
  const int bh = blockIdx.x, d = blockIdx.y + 1;
  const int npair = (nb + 1) / 2;
  const uint64_t* hb = bits + (int64_t)bh * nb * nw;
  unsigned acc = 0;
  for (int x = threadIdx.x; x < npair * nw; x += blockDim.x) {
    const int p = x / nw, w = x - p * nw;
    const int2 pb = pair_blocks(p, d, nb);
    uint64_t m = hb[(int64_t)pb.x * nw + w];
    if (pb.y >= 0) m |= hb[(int64_t)pb.y * nw + w];
    acc += (unsigned)__popcll(m);
  }
  __shared__ unsigned long long part[4];
  unsigned long long v = acc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) cost[(int64_t)bh * PAIR_D_MAX + d - 1] = part[0] + part[1] + part[2] + part[3];
}

// pair_d[bh] = the d of least cost, ties to the smaller d; one wave per head
__global__ __launch_bounds__(64) void pair_pick_kernel(const unsigned long long* __restrict__ cost, int dmax,
                                                       int32_t* __restrict__ pair_d) {
  const int bh = blockIdx.x, l = threadIdx.x;
  unsigned long long c = l < dmax ? cost[(int64_t)bh * PAIR_D_MAX + l] : ~0ull;
  int d = l + 1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long c2 = __shfl_xor(c, o, 64);
    const int d2 = __shfl_xor(d, o, 64);
    if (c2 < c || (c2 == c && d2 < d)) { c = c2; d = d2; }
  }
  if (l == 0) pair_d[bh] = d;
}

size_t pair_bits_ws(int64_t rows, int nb) {
  const int64_t BH = rows / (nb > 0 ? nb : 1);
  return pairing_al256((size_t)rows * ((nb + 63) / 64) * 8) + pairing_al256((size_t)BH * PAIR_D_MAX * 8);
}

hipError_t launch_pair_offsets(const int32_t* row_ptr, const int32_t* col_idx, const int32_t* row_len,
                               int row_stride, int BH, int nb, uint64_t* bits, int32_t* pair_d, hipStream_t st) {
  const int nw = (nb + 63) / 64, dmax = nb / 2 < PAIR_D_MAX ? (nb / 2 > 1 ? nb / 2 : 1) : PAIR_D_MAX;
  const int64_t rows = (int64_t)BH * nb, n = rows * nw;
  unsigned long long* cost = (unsigned long long*)((char*)bits + pairing_al256((size_t)n * 8));
  hipLaunchKernelGGL(row_bits_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 4 * nw * sizeof(uint64_t), st,
                     row_ptr, col_idx, row_len, row_stride, rows, nw, bits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pair_cost_kernel, dim3((unsigned)BH, (unsigned)dmax), dim3(256), 0, st, bits, nb, nw, cost);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pair_pick_kernel, dim3((unsigned)BH), dim3(64), 0, st, cost, dmax, pair_d);
  return hipGetLastError();
}

BSA_CHECK_ACCESSOR(check_flags_mask_ops)

}  // namespace bsa
