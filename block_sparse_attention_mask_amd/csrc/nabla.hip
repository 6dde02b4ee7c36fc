// Adaptive block mask (NABLA): block pooling, reduced map, row softmax and the
// cumulative-mass threshold, on gfx950.
//
// Method: Pith review of "NABLA: Neighborhood Adaptive Block-Level Attention",
// sections "What carries the argument" and "Core claim": average-pool Q and K over
// N-token blocks, softmax the reduced (S/N)x(S/N) map, sort each row, take the
// cumulative sum and keep the smallest prefix whose mass reaches 1 - thr; the
// referee report (minor comment 2) fixes the sort/cumsum to the key-block axis and
// the final reorder to the original block order.
//
// GPU formulation (no sort is materialised):
//   * pool_kernel streams Q and K once and writes exact fp64 block means
//     (sums of 64 bf16 values are exact in fp64);
//   * select_kernel computes 16 rows of L = scale * Qbar Kbar^T per workgroup in
//     fp64 registers, softmaxes them, and finds for each row the "pivot": the
//     first entry, in descending (p, -index) order, at which the cumulative mass
//     reaches 1 - thr. Entries before it and the pivot itself are kept. The pivot
//     is found by a radix select on the fp64 bit pattern of p (monotone for p >= 0)
//     using per-bucket mass histograms. Masses are accumulated in 2^-60 fixed
//     point, so the sums are exact integers and the result does not depend on the
//     order of the atomic additions (run-to-run deterministic).
#include "common.h"
#include "launch.h"

namespace bsa {

// ----------------------------------------------------------------------------
// Pooling: Qbar[bh][i][d] = (1/64) sum_r Q[bh][64 i + r][d];  KbarT[bh][d][i] likewise.
// One workgroup per (block i, bh, tensor). Each thread loads 16 bytes per row.
// ----------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, int64_t q_sb, int64_t q_sh,
                                                   int64_t q_ss, const T* __restrict__ k, int64_t k_sb,
                                                   int64_t k_sh, int64_t k_ss, int H, int nb,
                                                   double* __restrict__ qbar, double* __restrict__ kbarT) {
  constexpr int E = 16 / sizeof(T);        // elements per 16-byte load
  constexpr int TPR = D / E;               // threads per row
  constexpr int RPP = 256 / TPR;           // rows per pass
  constexpr int PASSES = BSA_N / RPP;
  __shared__ double part[RPP][D];

  const int i = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int b = bh / H, h = bh % H;
  const T* src = which == 0 ? q + b * q_sb + h * q_sh + (int64_t)i * BSA_N * q_ss
                            : k + b * k_sb + h * k_sh + (int64_t)i * BSA_N * k_ss;
  const int64_t ss = which == 0 ? q_ss : k_ss;
  const int t = threadIdx.x, cg = t % TPR, r0 = t / TPR;

  double acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0;
  // issue all loads first, then convert
  i32x4_t raw[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps)
    raw[ps] = *(const i32x4_t*)(src + (int64_t)(r0 + ps * RPP) * ss + cg * E);
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned u = (unsigned)raw[ps][w];
        acc[2 * w] += (double)__uint_as_float(u << 16);
        acc[2 * w + 1] += (double)__uint_as_float(u & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] += (double)__int_as_float(raw[ps][w]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) part[r0][cg * E + e] = acc[e];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += part[r][t];
    s *= (1.0 / BSA_N);
    if (which == 0)
      qbar[((int64_t)bh * nb + i) * D + t] = s;
    else
      kbarT[((int64_t)bh * D + t) * nb + i] = s;
  }
}

// ----------------------------------------------------------------------------
// Row selection.
// ----------------------------------------------------------------------------
constexpr int SEL_ROWS = 16;
constexpr int SEL_WAVES = 4;

enum : int { ROW_ACTIVE = 0, ROW_PIVOT = 1, ROW_ALL = 2, ROW_TIE = 3, ROW_SKIP = 4 };

struct SelRowState {
  uint64_t lo;         // current key range [lo, lo + 2^span)
  uint64_t mass_above; // fixed-point mass of all keys above the range
  int span;            // bits of the range (-1 before the exponent pass)
  int status;
  int cnt;             // candidates in the range
  int tie_keep;        // number of tied entries kept (ROW_TIE)
};

__device__ __forceinline__ uint64_t fixed_mass(double p) {
  // p in [0, 1]  ->  floor(p * 2^60)
  return (uint64_t)(p * 0x1p60);
}

// digit of key for the current pass; returns -1 when the key is outside the range
__device__ __forceinline__ int sel_digit(uint64_t key, const SelRowState& st) {
  if (st.span < 0) {               // exponent pass: 256 buckets over the fp64 exponent
    int e = (int)(key >> 52);      // sign bit is 0
    int d = e - 768;
    return d < 0 ? 0 : (d > 255 ? 255 : d);
  }
  if (key < st.lo || key - st.lo >= (1ull << st.span)) return -1;
  int db = st.span < 8 ? st.span : 8;
  return (int)((key - st.lo) >> (st.span - db));
}

template <int C>   // C = column chunks of 64 per wave
__global__ __launch_bounds__(256) void select_kernel(const double* __restrict__ qbar,
                                                     const double* __restrict__ kbarT, int nb, int D,
                                                     double scale, uint64_t T_fixed,
                                                     const uint8_t* __restrict__ or_mask, int64_t or_sb,
                                                     int64_t or_sh, int H, uint8_t* __restrict__ mask_out) {
  __shared__ double qs[SEL_ROWS][128];
  __shared__ uint64_t hmass[SEL_ROWS][256];
  __shared__ uint32_t hcnt[SEL_ROWS][256];
  __shared__ uint32_t tiebits[SEL_ROWS][64];
  __shared__ double red[SEL_ROWS][SEL_WAVES];
  __shared__ uint64_t redu[SEL_ROWS][SEL_WAVES];
  __shared__ SelRowState st[SEL_ROWS];
  __shared__ int any_active;

  const int bh = blockIdx.y, row0 = blockIdx.x * SEL_ROWS;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;

  for (int x = tid; x < SEL_ROWS * D; x += 256) {
    int r = x / D, d = x % D;
    qs[r][d] = (row0 + r < nb) ? qbar[((int64_t)bh * nb + row0 + r) * D + d] : 0.0;
  }
  __syncthreads();

  // ---- reduced map rows: acc[r][c] = <Qbar_row, Kbar_j>, j = (c*4 + w)*64 + l
  double acc[SEL_ROWS][C];
#pragma unroll
  for (int r = 0; r < SEL_ROWS; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[r][c] = 0.0;
  bool valid[C];
  int col[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    col[c] = (c * SEL_WAVES + w) * 64 + l;
    valid[c] = col[c] < nb;
  }
  const double* kb = kbarT + (int64_t)bh * D * nb;
  for (int d = 0; d < D; d += 2) {
    double k0[C], k1[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      k0[c] = valid[c] ? kb[(int64_t)d * nb + col[c]] : 0.0;
      k1[c] = valid[c] ? kb[(int64_t)(d + 1) * nb + col[c]] : 0.0;
    }
#pragma unroll
    for (int r = 0; r < SEL_ROWS; ++r) {
      double q0 = qs[r][d], q1 = qs[r][d + 1];
#pragma unroll
      for (int c = 0; c < C; ++c) acc[r][c] = fma(q1, k1[c], fma(q0, k0[c], acc[r][c]));
    }
  }

  // ---- softmax of each row (fp64), max and sum reduced across the 4 waves
#pragma unroll
  for (int r = 0; r < SEL_ROWS; ++r) {
    double m = -INFINITY;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      acc[r][c] *= scale;
      if (valid[c]) m = fmax(m, acc[r][c]);
    }
    m = wave_max_f64(m);
    if (l == 0) red[r][w] = m;
  }
  __syncthreads();
  double rowmax[SEL_ROWS];
#pragma unroll
  for (int r = 0; r < SEL_ROWS; ++r)
    rowmax[r] = fmax(fmax(red[r][0], red[r][1]), fmax(red[r][2], red[r][3]));
  __syncthreads();
#pragma unroll
  for (int r = 0; r < SEL_ROWS; ++r) {
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      double e = valid[c] ? exp(acc[r][c] - rowmax[r]) : 0.0;
      acc[r][c] = e;
      s += e;
    }
    s = wave_sum_f64(s);
    if (l == 0) red[r][w] = s;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < SEL_ROWS; ++r) {
    double tot = ((red[r][0] + red[r][1]) + red[r][2]) + red[r][3];
    uint64_t ms = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      acc[r][c] = acc[r][c] / tot;           // p >= 0; its bits are the sort key
      ms += fixed_mass(acc[r][c]);
    }
    ms = wave_sum_u64(ms);
    if (l == 0) redu[r][w] = ms;
  }
  __syncthreads();
  if (tid < SEL_ROWS) {
    int r = tid;
    uint64_t total = redu[r][0] + redu[r][1] + redu[r][2] + redu[r][3];
    SelRowState s;
    s.lo = 0;
    s.mass_above = 0;
    s.span = -1;
    s.cnt = 0;
    s.tie_keep = 0;
    if (row0 + r >= nb) s.status = ROW_SKIP;
    else if (total < T_fixed) s.status = ROW_ALL;   // every entry is reached before the mass 1 - thr
    else s.status = ROW_ACTIVE;
    st[r] = s;
  }
  if (tid == 0) any_active = 1;
  __syncthreads();

  // ---- radix select of the pivot, all rows in lock step
  for (int pass = 0; pass < 9; ++pass) {
    if (!any_active) break;
    for (int x = tid; x < SEL_ROWS * 256; x += 256) {
      hmass[x / 256][x % 256] = 0;
      hcnt[x / 256][x % 256] = 0;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SEL_ROWS; ++r) {
      SelRowState s = st[r];
      if (s.status != ROW_ACTIVE) continue;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (!valid[c]) continue;
        uint64_t key = (uint64_t)__double_as_longlong(acc[r][c]);
        int dg = sel_digit(key, s);
        if (dg >= 0) {
          atomicAdd((unsigned long long*)&hmass[r][dg], (unsigned long long)fixed_mass(acc[r][c]));
          atomicAdd(&hcnt[r][dg], 1u);
        }
      }
    }
    __syncthreads();
    // each wave scans 4 rows: lane l owns buckets 255-4l .. 252-4l (descending keys)
    for (int r = w; r < SEL_ROWS; r += SEL_WAVES) {
      SelRowState s = st[r];
      if (s.status != ROW_ACTIVE) continue;
      uint64_t mb[4];
      uint32_t cb[4];
      uint64_t lt = 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        mb[x] = hmass[r][255 - 4 * l - x];
        cb[x] = hcnt[r][255 - 4 * l - x];
        lt += mb[x];
      }
      uint64_t incl = wave_incl_scan_u64(lt);
      uint64_t before = s.mass_above + (incl - lt);
      bool cross = before + lt >= T_fixed;
      uint64_t ball = __ballot(cross);
      int L = ball ? __builtin_ctzll(ball) : 63;   // the invariant guarantees ball != 0
      if (l == L) {
        uint64_t cum = before;
        int xs = 3;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          if (cum + mb[x] >= T_fixed) { xs = x; break; }
          cum += mb[x];
        }
        int dg = 255 - 4 * l - xs;
        SelRowState n = s;
        n.mass_above = cum;
        n.cnt = (int)cb[xs];
        if (s.span < 0) {
          n.lo = (uint64_t)(dg + 768) << 52;
          n.span = 52;
        } else {
          int db = s.span < 8 ? s.span : 8;
          n.span = s.span - db;
          n.lo = s.lo + ((uint64_t)dg << n.span);
        }
        if (n.cnt <= 1) n.status = ROW_PIVOT;
        else if (n.span == 0) {
          // identical keys: visited by ascending index, each adds the same mass
          uint64_t wq = fixed_mass(__longlong_as_double((long long)n.lo));
          uint64_t need = T_fixed - n.mass_above;          // > 0
          uint64_t t = wq ? (need + wq - 1) / wq : (uint64_t)n.cnt;
          n.tie_keep = (int)(t < (uint64_t)n.cnt ? t : (uint64_t)n.cnt);
          n.status = ROW_TIE;
        }
        st[r] = n;
      }
    }
    __syncthreads();
    if (tid == 0) {
      int a = 0;
      for (int r = 0; r < SEL_ROWS; ++r) a |= st[r].status == ROW_ACTIVE;
      any_active = a;
    }
    __syncthreads();
  }

  // ---- ties: rank tied entries by ascending column index
  bool need_ties = false;
#pragma unroll
  for (int r = 0; r < SEL_ROWS; ++r) need_ties |= st[r].status == ROW_TIE;
  if (need_ties) {
    for (int x = tid; x < SEL_ROWS * 64; x += 256) tiebits[x / 64][x % 64] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SEL_ROWS; ++r) {
      if (st[r].status != ROW_TIE) continue;
      uint64_t lo = st[r].lo;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (valid[c] && (uint64_t)__double_as_longlong(acc[r][c]) == lo)
          atomicOr(&tiebits[r][col[c] >> 5], 1u << (col[c] & 31));
    }
    __syncthreads();
  }

  // ---- write the mask rows (OR'd with the optional mask)
  const int b = bh / H, h = bh % H;
#pragma unroll
  for (int r = 0; r < SEL_ROWS; ++r) {
    SelRowState s = st[r];
    if (s.status == ROW_SKIP) continue;
    const int row = row0 + r;
    uint8_t* dst = mask_out + ((int64_t)bh * nb + row) * nb;
    const uint8_t* om = or_mask ? or_mask + b * or_sb + h * or_sh + (int64_t)row * nb : nullptr;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (!valid[c]) continue;
      uint64_t key = (uint64_t)__double_as_longlong(acc[r][c]);
      bool keep;
      if (s.status == ROW_ALL) keep = true;
      else if (s.status == ROW_PIVOT) keep = key >= s.lo;
      else {   // ROW_TIE
        if (key != s.lo) keep = key > s.lo;
        else {
          int j = col[c], rank = 0;
          for (int x = 0; x < (j >> 5); ++x) rank += __popc(tiebits[r][x]);
          rank += __popc(tiebits[r][j >> 5] & ((1u << (j & 31)) - 1u));
          keep = rank < s.tie_keep;
        }
      }
      if (om && om[col[c]]) keep = true;
      dst[col[c]] = keep ? 1 : 0;
    }
  }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <typename T, int D>
static hipError_t launch_pool_t(const void* q, const int64_t* qs, const void* k, const int64_t* ks, int B,
                                int H, int nb, double* qbar, double* kbarT, hipStream_t st) {
  dim3 grid(nb, B * H, 2);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, st, (const T*)q, qs[0], qs[1], qs[2],
                     (const T*)k, ks[0], ks[1], ks[2], H, nb, qbar, kbarT);
  return hipGetLastError();
}

hipError_t launch_pool(bool f32, int D, const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                       int B, int H, int nb, double* qbar, double* kbarT, hipStream_t st) {
  if (f32) return D == 64 ? launch_pool_t<float, 64>(q, qs, k, ks, B, H, nb, qbar, kbarT, st)
                          : launch_pool_t<float, 128>(q, qs, k, ks, B, H, nb, qbar, kbarT, st);
  return D == 64 ? launch_pool_t<u16, 64>(q, qs, k, ks, B, H, nb, qbar, kbarT, st)
                 : launch_pool_t<u16, 128>(q, qs, k, ks, B, H, nb, qbar, kbarT, st);
}

template <int C>
static hipError_t launch_select_c(const double* qbar, const double* kbarT, int B, int H, int nb, int D,
                                  double scale, uint64_t T_fixed, const uint8_t* or_mask, int64_t or_sb,
                                  int64_t or_sh, uint8_t* mask_out, hipStream_t st) {
  dim3 grid((nb + SEL_ROWS - 1) / SEL_ROWS, B * H);
  hipLaunchKernelGGL((select_kernel<C>), grid, dim3(256), 0, st, qbar, kbarT, nb, D, scale, T_fixed, or_mask,
                     or_sb, or_sh, H, mask_out);
  return hipGetLastError();
}

hipError_t launch_select(const double* qbar, const double* kbarT, int B, int H, int nb, int D, double scale,
                         uint64_t T_fixed, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                         uint8_t* mask_out, hipStream_t st) {
  const int chunks = (nb + 63) / 64;
  const int C = (chunks + SEL_WAVES - 1) / SEL_WAVES;
#define BSA_SEL_CASE(n) \
  case n: return launch_select_c<n>(qbar, kbarT, B, H, nb, D, scale, T_fixed, or_mask, or_sb, or_sh, mask_out, st);
  switch (C) {
    BSA_SEL_CASE(1) BSA_SEL_CASE(2) BSA_SEL_CASE(3) BSA_SEL_CASE(4)
    BSA_SEL_CASE(5) BSA_SEL_CASE(6) BSA_SEL_CASE(7) BSA_SEL_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef BSA_SEL_CASE
}

}  // namespace bsa
