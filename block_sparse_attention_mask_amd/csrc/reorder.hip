// Token reordering of [B, H, S, D] tensors between the row-major (t, h, w) layout of a
// T x H x W latent grid and the layouts the block masks prefer (gfx950).
//
// Method: NABLA (Pith review, "Assumptions & free parameters" and Figure 4): fractal
// flattening groups each frame's tokens into P x P spatial patches, so that one
// N-token block is one patch; STA blog review ("Observation & Proposed Method"): tokens
// grouped into 3D tiles, tile = kernel block; SVG (blog review of Sparse VideoGen):
// a layout transformation that makes the tokens of one spatial position across frames
// contiguous. All are permutations of the T*H*W rows:
//   ORDER_TILE     tiles (tt, th, tw) in row-major tile order, tokens row-major inside a
//                  tile; border tiles are smaller (fractal flattening = tile 1 x P x P);
//   ORDER_SPATIAL  (h, w, t): the frames of one spatial position together.
// The source row of each destination row is computed in closed form (no index array):
// tiles along one axis are full except the last, so the first token of tile (a, b, c)
// is a tt HW + st(a) b th W + st(a) sh(b) c tw, with st, sh the tile's extents.
// Rows >= T*H*W (end padding) are written as zeros. Pure data movement: one read and
// one write of every row, 16-byte chunks, all loads of a thread issued before its stores.
#include "common.h"
#include "launch.h"

namespace bsa {

// row-major index of the token at position p of the given order
__device__ __forceinline__ int64_t ordered_to_rowmajor(int64_t p, const ReorderGeom& g) {
  const int64_t HW = (int64_t)g.H * g.W;
  if (g.order == ORDER_SPATIAL) {
    const int64_t hw = p / g.T, t = p % g.T;
    return t * HW + hw;
  }
  if (g.order == ORDER_TILE) {
    const int64_t slab = (int64_t)g.tt * HW;            // tokens of one full row of tiles in t
    const int a = (int)(p / slab);
    int64_t r = p - a * slab;
    const int st = min(g.tt, g.T - a * g.tt);
    const int64_t band = (int64_t)st * g.th * g.W;      // a full row of tiles in h, inside slab a
    const int bb = (int)(r / band);
    r -= bb * band;
    const int sh = min(g.th, g.H - bb * g.th);
    const int64_t tile = (int64_t)st * sh * g.tw;       // a full tile in w
    const int c = (int)(r / tile);
    r -= c * tile;
    const int sw = min(g.tw, g.W - c * g.tw);
    const int it = (int)(r / (sh * sw)), ih = (int)((r / sw) % sh), iw = (int)(r % sw);
    return ((int64_t)(a * g.tt + it) * g.H + (bb * g.th + ih)) * g.W + (c * g.tw + iw);
  }
  return p;
}

// One workgroup of 256 threads per 64 destination rows of one (b, h); CH 16-byte chunks
// per row. inverse = false: dst[p] = src[rowmajor(p)] (row-major -> ordered);
// inverse = true: dst[rowmajor(p)] = src[p] (ordered -> row-major).
template <int CH>
__global__ __launch_bounds__(256) void token_reorder_kernel(const char* __restrict__ src, int64_t s_sb, int64_t s_sh,
                                                            int64_t s_ss, char* __restrict__ dst, int64_t d_sb,
                                                            int64_t d_sh, int64_t d_ss, ReorderGeom g, int H,
                                                            bool inverse) {
  constexpr int PER = 64 * CH / 256;                // chunks per thread
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const char* sbase = src + b * s_sb + h * s_sh;
  char* dbase = dst + b * d_sb + h * d_sh;
  const int64_t valid = (int64_t)g.T * g.H * g.W;
  i32x4_t val[PER];
  int64_t drow[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int x = threadIdx.x + u * 256;
    const int64_t p = (int64_t)blockIdx.x * 64 + x / CH;
    const int c = x % CH;
    int64_t srow, dr;
    if (p < valid) {
      const int64_t rm = ordered_to_rowmajor(p, g);
      srow = inverse ? p : rm;
      dr = inverse ? rm : p;
      val[u] = *(const i32x4_t*)(sbase + srow * s_ss + c * 16);
    } else {
      dr = p;
      val[u] = i32x4_t{0, 0, 0, 0};
    }
    drow[u] = dr;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int x = threadIdx.x + u * 256;
    *(i32x4_t*)(dbase + drow[u] * d_ss + (x % CH) * 16) = val[u];
  }
}

hipError_t launch_token_reorder(const void* src, const int64_t* s_strides_bytes, void* dst,
                                const int64_t* d_strides_bytes, int B, int H, int S, int row_bytes,
                                const ReorderGeom& g, bool inverse, hipStream_t st) {
  dim3 grid(S / 64, B * H);
  const char* s = (const char*)src;
  char* d = (char*)dst;
#define BSA_REORDER(CHN)                                                                                       \
  hipLaunchKernelGGL(token_reorder_kernel<CHN>, grid, dim3(256), 0, st, s, s_strides_bytes[0], s_strides_bytes[1], \
                     s_strides_bytes[2], d, d_strides_bytes[0], d_strides_bytes[1], d_strides_bytes[2], g, H, inverse)
  switch (row_bytes / 16) {
    case 4: BSA_REORDER(4); break;
    case 8: BSA_REORDER(8); break;
    case 16: BSA_REORDER(16); break;
    case 32: BSA_REORDER(32); break;
    default: return hipErrorInvalidValue;
  }
#undef BSA_REORDER
  return hipGetLastError();
}

}  // namespace bsa
