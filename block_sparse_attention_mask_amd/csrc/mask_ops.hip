// Mask union and mask -> per-query-block kv index lists (CSR).
//
// The union follows the NABLA review ("What carries the argument": the adaptive mask
// is optionally OR'd with a sliding-tile mask); the index lists are the "skip lists"
// of the CalibAtt page: the attention kernel visits only the listed blocks.
#include "common.h"
#include "launch.h"

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

hipError_t launch_csr(const uint8_t* mask, int64_t sb, int64_t sh, int B, int H, int nb, int32_t* row_ptr,
                      int32_t* col_idx, int32_t* counts, hipStream_t st) {
  const int rows = B * H * nb;
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
  return hipGetLastError();
}

}  // namespace bsa
