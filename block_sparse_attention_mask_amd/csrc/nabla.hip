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
//   * select_kernel computes 16 rows of L = scale * Qbar Kbar^T per workgroup on the
//     fp64 MFMA, softmaxes them, and finds for each row the "pivot": the
//     first entry, in descending (p, -index) order, at which the cumulative mass
//     reaches 1 - thr. Entries before it and the pivot itself are kept. The pivot
//     is found by a radix select on the 2^-60 fixed-point mass w = floor(p 2^60) of
//     each entry (monotone in p; distinct for distinct p >= 2^-8, so only entries
//     closer than 2^-60 to each other are ordered by index), with per-bucket
//     histograms of count and mass. The sums are exact integers, so the result does
//     not depend on the order of the atomic additions (run-to-run deterministic).
//     For short rows (nb <= 256) select_rows_kernel does the same per row with one
//     wave per row after the map is formed, without workgroup barriers.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace bsa {

// ----------------------------------------------------------------------------
// Pooled vectors are stored in the operand order of v_mfma_f64_16x16x4_f64: for a
// tile of 16 blocks (rows of Qbar, or columns of Kbar^T) and k-step s (channels
// 4s..4s+3), lane l of the MFMA holds block 16*tile + l%16, channel 4s + l/16, so
// each operand is one coalesced 512-byte load. The layout is [bh][tile][D/4][64].
// ----------------------------------------------------------------------------
__device__ __forceinline__ int64_t mf_index(int bh, int nb, int D, int blk, int d) {
  const int ntile = (nb + 15) / 16;
  return (((int64_t)bh * ntile + blk / 16) * (D / 4) + d / 4) * 64 + (blk % 16) + 16 * (d % 4);
}

// ----------------------------------------------------------------------------
// fp8 e4m3fn encoding (OCP 8-bit floating point: bias 7, 3 mantissa bits, subnormals
// m/8 * 2^-6, no infinities, largest finite 448; FlashAttention-3 abstract, Daily Papers
// listing: block quantisation). v_cvt_pk_fp8_f32 of gfx950 rounds fp32 to this format,
// nearest even; it agrees with the reference encoder (nearest code of the format's value
// table) on 1.1e6 values covering every tie between adjacent codes and their neighbours,
// the subnormal range and values just above and below 448. The quotients fed to it never
// exceed 448 by more than an fp32 rounding, which rounds back to 448.
// ----------------------------------------------------------------------------
__device__ __forceinline__ unsigned pack_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// One cross-lane butterfly of the fast Walsh-Hadamard transform on chunk bit X of the
// rotated pool's lane map: the lower lane of the pair keeps a + b, the upper a - b (a the
// lower lane's value, b the upper's), each as one fma with the lane's sign su = +1 / -1:
// fma(+-1, b, a) is a +- b rounded once, signed zeros included. Partners 1 or 2 lanes apart
// come from a DPP quad permute ([1,0,3,2], [2,3,0,1]): there the own value is b in the
// upper lane, so the lower lane's fma(1, y, o) = y + o and the upper's fma(-1, y, o) = o - y.
// Partners 16 or 32 apart come from a permlane swap, which leaves a in r[0] and b in r[1]
// in both lanes of the pair; 4 apart from a shuffle.
template <int X>
__device__ __forceinline__ float wht_lane_stage(float y, float su) {
  const unsigned u = __float_as_uint(y);
  if constexpr (X < 2) {
    const float o = __uint_as_float((unsigned)__builtin_amdgcn_mov_dpp((int)u, X == 0 ? 0xB1 : 0x4E, 0xF, 0xF, true));
    return __builtin_fmaf(su, y, o);
  } else if constexpr (X == 2 || X == 3) {
    const auto r = X == 2 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                          : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_fmaf(su, __uint_as_float(r[1]), __uint_as_float(r[0]));
  } else {
    return __builtin_fmaf(su, y, __shfl_xor(y, 4, 64));
  }
}

// ----------------------------------------------------------------------------
// Pooling: Qbar[bh][i][d] = (1/64) sum_r Q[bh][64 i + r][d], and Kbar likewise.
// One workgroup per two consecutive blocks of one (bh, tensor); each thread issues
// all of its 16-byte loads (8 rows x 2 blocks) before converting any. NT: streaming
// (non-temporal) loads, for inputs much larger than the last-level cache.
// Q8: from the same registers, the block's fp8 quantisation (scale = amax / 448 in
// fp32, codes = e4m3(x / scale)), so a run with fp8 Q/K reads Q and K once.
// POOL = false skips the means (quantisation alone, of the tensor in q).
// ROT (with Q8): incoherent processing (FlashAttention-3 abstract, Daily Papers listing:
// named beside block quantisation) before the quantisation: each row x becomes
// y = H (s . x), H the Sylvester Hadamard matrix and s the caller's random signs, by the
// fast Walsh-Hadamard transform in fp32, butterflies (a, b) -> (a + b, a - b) at strides
// 1, 2, ..., D/2 in that order (strides below E inside a thread, the others between the
// lanes of the row); the amax, scale and codes are then those of y, and the stored scale
// is multiplied by f8.smul (1/D on the key side, exact), so that dequantised codes give
// q . k of the unrotated rows. The means are still those of the unrotated rows.
// ----------------------------------------------------------------------------
constexpr int POOL_BPW = 2;   // blocks per workgroup
template <typename T, int D, bool NT, bool POOL, bool Q8, bool ROT = false>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, int64_t q_sb, int64_t q_sh,
                                                   int64_t q_ss, const T* __restrict__ k, int64_t k_sb,
                                                   int64_t k_sh, int64_t k_ss, int H, int nb,
                                                   double* __restrict__ qbar, double* __restrict__ kbarT,
                                                   Fp8Out f8) {
  constexpr int E = 16 / sizeof(T);        // elements per 16-byte load
  constexpr int TPR = D / E;               // threads per row
  constexpr int RPP = 256 / TPR;           // rows per pass
  constexpr int PASSES = BSA_N / RPP;
  __shared__ double part[POOL_BPW][RPP][D];

  const int i0 = blockIdx.x * POOL_BPW, bh = blockIdx.y, which = blockIdx.z;
  const int b = bh / H, h = bh % H;
  const T* base = which == 0 ? q + b * q_sb + h * q_sh : k + b * k_sb + h * k_sh;
  const int64_t ss = which == 0 ? q_ss : k_ss;
  const int t = threadIdx.x;
  // (row, 16-byte column chunk) of this thread. ROT: the chunk's bits sit on lane bits 0, 1,
  // 4, 5 (then 2, 3), so that the butterfly partners of the cross-lane stages are 1 or 2
  // lanes apart (DPP quad permutes) or 16 or 32 apart (permlane swaps); the other lane bits
  // and the wave index give the row. Either map is a bijection of the threads onto the
  // (row, chunk) pairs of a pass, and a wave still covers whole rows.
  int cg, r0;
  if constexpr (ROT) {
    constexpr int LB[6] = {0, 1, 4, 5, 2, 3};
    constexpr int NCB = TPR == 8 ? 3 : TPR == 16 ? 4 : 5;   // chunk bits
    const int l = t & 63;
    cg = 0;
    int rl = 0, nr = 0;
#pragma unroll
    for (int x = 0; x < 6; ++x) {
      const int bit = (l >> LB[x]) & 1;
      if (x < NCB) cg |= bit << x;
    }
#pragma unroll
    for (int lb = 0; lb < 6; ++lb) {
      bool is_chunk = false;
#pragma unroll
      for (int x = 0; x < NCB; ++x) is_chunk |= LB[x] == lb;
      if (!is_chunk) rl |= ((l >> lb) & 1) << nr++;
    }
    r0 = (t >> 6) * (64 / TPR) + rl;
  } else {
    cg = t % TPR;
    r0 = t / TPR;
  }

  i32x4_t raw[POOL_BPW][PASSES];
#pragma unroll
  for (int bb = 0; bb < POOL_BPW; ++bb) {
    const int i = min(i0 + bb, nb - 1);     // a missing last block re-reads block nb-1 (not stored)
    const T* src = base + (int64_t)i * BSA_N * ss;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const i32x4_t* ptr = (const i32x4_t*)(src + (int64_t)(r0 + ps * RPP) * ss + cg * E);
      if constexpr (NT) raw[bb][ps] = __builtin_nontemporal_load(ptr);
      else raw[bb][ps] = *ptr;
    }
  }
  // element e of 16-byte word w as fp32
  auto elem = [&](const i32x4_t& wv, int e) -> float {
    if constexpr (sizeof(T) == 2) {
      const unsigned u = (unsigned)wv[e / 2];
      return __uint_as_float(e & 1 ? (u & 0xFFFF0000u) : (u << 16));
    } else {
      return __int_as_float(wv[e]);
    }
  };
  // fp64 partial sums of the block means: part[bb][r][d] = sum over this thread's rows
  auto pool_partials = [&]() {
#pragma unroll
    for (int bb = 0; bb < POOL_BPW; ++bb) {
      double acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = 0.0;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            unsigned u = (unsigned)raw[bb][ps][w];
            acc[2 * w] += (double)__uint_as_float(u << 16);
            acc[2 * w + 1] += (double)__uint_as_float(u & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[w] += (double)__int_as_float(raw[bb][ps][w]);
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) part[bb][r0][cg * E + e] = acc[e];
    }
  };
  // ROT: the sums come first, so that the loaded words can die as they are rotated
  if constexpr (POOL && ROT) pool_partials();
  if constexpr (Q8) {
    __shared__ float wmax[POOL_BPW][4];
    const int lane = t & 63, wave = t >> 6;
    // the values quantised: x itself, or its rotation y = H (s . x)
    float rv[ROT ? POOL_BPW : 1][ROT ? PASSES : 1][ROT ? E : 1];
    if constexpr (ROT) {
      const int d0 = cg * E;   // first channel of this thread
      const unsigned sgn = (unsigned)(f8.sbits[d0 >> 6] >> (d0 & 63)) & ((1u << E) - 1u);
#pragma unroll
      for (int bb = 0; bb < POOL_BPW; ++bb)
#pragma unroll
        for (int ps = 0; ps < PASSES; ++ps) {
          float* y = rv[bb][ps];
#pragma unroll
          for (int e = 0; e < E; ++e)
            y[e] = __uint_as_float(__float_as_uint(elem(raw[bb][ps], e)) ^ (((sgn >> e) & 1u) << 31));
#pragma unroll
          for (int hs = 1; hs < E; hs *= 2)
#pragma unroll
            for (int e = 0; e < E; ++e)
              if (!(e & hs)) {
                const float a0 = y[e], b0 = y[e + hs];
                y[e] = a0 + b0;
                y[e + hs] = a0 - b0;
              }
          // stride E 2^X: chunk bit X, the partner lane 1, 2, 16, 32 or 4 apart
          auto stage = [&](auto xc) {
            constexpr int X = decltype(xc)::value;
            if constexpr ((1 << X) < TPR) {
              const float su = (cg >> X) & 1 ? -1.f : 1.f;
#pragma unroll
              for (int e = 0; e < E; ++e) y[e] = wht_lane_stage<X>(y[e], su);
            }
          };
          stage(std::integral_constant<int, 0>{});
          stage(std::integral_constant<int, 1>{});
          stage(std::integral_constant<int, 2>{});
          stage(std::integral_constant<int, 3>{});
          stage(std::integral_constant<int, 4>{});
        }
    }
    auto qval = [&](int bb, int ps, int e) -> float {
      if constexpr (ROT) return rv[bb][ps][e];
      else return elem(raw[bb][ps], e);
    };
#pragma unroll
    for (int bb = 0; bb < POOL_BPW; ++bb) {
      float m = 0.f;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps)
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(qval(bb, ps, e)));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) wmax[bb][wave] = m;
    }
    __syncthreads();
#pragma unroll
    for (int bb = 0; bb < POOL_BPW; ++bb) {
      const int i = i0 + bb;
      if (i >= nb) continue;
      const float amax = fmaxf(fmaxf(wmax[bb][0], wmax[bb][1]), fmaxf(wmax[bb][2], wmax[bb][3]));
      const float sc = amax > 0.f ? amax / 448.f : 1.f;
      // The codes are those of the correctly rounded quotient x / sc. For bf16 inputs with
      // 2^-100 <= amax <= 2^100 the quotient is formed as q = x r with r = 1 / sc and one FMA
      // correction q + (x - q sc) r (Markstein), which gives the same code for every bf16 x <= amax
      // (checked exhaustively on the host: 4.2e8 pairs); elsewhere the division itself is used.
      // (Rotated values are fp32 sums, not bf16: they always take the division.)
      const bool recip = !ROT && sizeof(T) == 2 && amax >= 0x1p-100f && amax <= 0x1p100f;
      const float r = 1.f / sc;
      auto quot = [&](float x) -> float {
        if (!recip) return x / sc;
        const float q0 = __fmul_rn(x, r);
        return __builtin_fmaf(__builtin_fmaf(-q0, sc, x), r, q0);
      };
      uint8_t* cbase = f8.codes[which] + b * f8.sb[which] + h * f8.sh[which];
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        unsigned w[E / 4];
#pragma unroll
        for (int x = 0; x < E / 4; ++x)
          w[x] = pack_e4m3x4(quot(qval(bb, ps, 4 * x)), quot(qval(bb, ps, 4 * x + 1)),
                             quot(qval(bb, ps, 4 * x + 2)), quot(qval(bb, ps, 4 * x + 3)));
        uint8_t* dst = cbase + ((int64_t)i * BSA_N + r0 + ps * RPP) * f8.ss[which] + cg * E;
        if constexpr (E == 8) *(uint2*)dst = make_uint2(w[0], w[1]);
        else *(unsigned*)dst = w[0];
      }
      if (t == 0) f8.scale[which][(int64_t)bh * nb + i] = ROT ? sc * f8.smul[which] : sc;
    }
  }
  if constexpr (POOL && !ROT) pool_partials();
  if constexpr (!POOL) return;
  __syncthreads();
  for (int x = t; x < POOL_BPW * D; x += 256) {
    const int bb = x / D, d = x % D, i = i0 + bb;
    if (i >= nb) continue;
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += part[bb][r][d];
    s *= (1.0 / BSA_N);
    double* dst = which == 0 ? qbar : kbarT;
    dst[mf_index(bh, nb, D, i, d)] = s;
  }
}

// ----------------------------------------------------------------------------
// Row selection.
// ----------------------------------------------------------------------------
constexpr int SEL_ROWS = 16;
constexpr int SEL_WAVES = 8;

enum : int { ROW_ACTIVE = 0, ROW_PIVOT = 1, ROW_ALL = 2, ROW_TIE = 3, ROW_SKIP = 4, ROW_NONE = 5 };

struct SelRowState {
  uint64_t lo;         // current key range [lo, lo + 2^span)
  uint64_t mass_above; // fixed-point mass (Top-k: number) of all keys above the range
  int span;            // bits of the range (-1 before the exponent pass)
  int status;
  int cnt;             // candidates in the range
  int tie_keep;        // number of tied entries kept (ROW_TIE)
};

// State of a row before its radix select for one target: every entry is kept when the row's
// total fixed-point mass stays below the target (Top-k: nb <= topk), none when the target
// is 0 (no entry has an exclusive mass below 0), else the pivot is searched.
__device__ __forceinline__ SelRowState sel_init(bool skip, uint64_t total, uint64_t target, bool by_count, int nb,
                                                int topk) {
  SelRowState n;
  n.lo = 0;
  n.mass_above = 0;
  n.span = -1;
  n.cnt = 0;
  n.tie_keep = 0;
  if (skip) n.status = ROW_SKIP;
  else if (by_count ? nb <= topk : total < target) n.status = ROW_ALL;
  else if (!by_count && target == 0) n.status = ROW_NONE;
  else n.status = ROW_ACTIVE;
  return n;
}

// Whether an entry with this key is kept once its row's state is final; tied: the key
// equals the row's tied key value (ROW_TIE), rank: its position among those by index.
__device__ __forceinline__ bool sel_keep(const SelRowState& sr, uint64_t key, bool tied, int rank) {
  if (sr.status == ROW_ALL) return true;
  if (sr.status == ROW_PIVOT) return key >= sr.lo;
  if (sr.status == ROW_TIE) return tied ? rank < sr.tie_keep : key > sr.lo;
  return false;   // ROW_NONE, ROW_SKIP
}

__device__ __forceinline__ uint64_t fixed_mass(double p) {
  // p in [0, 1]  ->  floor(p * 2^60)
  return (uint64_t)(p * 0x1p60);
}

// Radix digits of a fixed-point mass w (the sort key). The first pass is logarithmic:
// w < 4 gets bucket w; otherwise, with e the position of the leading one, bucket
// 4 + 4 (e - 2) + (the two bits below the leading one), i.e. the range
// [(4 + m) << (e - 2), (5 + m) << (e - 2)). Later passes split the current range
// [lo, lo + 2^span) by its top 8 bits. Returns -1 when w is outside the range.
__device__ __forceinline__ int first_digit(uint64_t w) {
  if (w < 4) return (int)w;
  const int e = 63 - __builtin_clzll(w);
  return 4 + 4 * (e - 2) + (int)((w >> (e - 2)) & 3);
}
__device__ __forceinline__ void first_range(int dg, uint64_t& lo, int& span) {
  if (dg < 4) { lo = (uint64_t)dg; span = 0; return; }
  const int e = (dg - 4) / 4 + 2, m = (dg - 4) % 4;
  lo = (uint64_t)(4 + m) << (e - 2);
  span = e - 2;
}
__device__ __forceinline__ int sel_digit(uint64_t key, const SelRowState& st) {
  if (st.span < 0) return first_digit(key);
  if (key < st.lo || key - st.lo >= (1ull << st.span)) return -1;
  const int db = st.span < 8 ? st.span : 8;
  return (int)((key - st.lo) >> (st.span - db));
}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// The reduced map of 16 query-block rows row0 = 16 rt ..: acc[c] = Qbar(16 rows) .
// Kbar^T(column tile w + SEL_WAVES c) on v_mfma_f64_16x16x4f64. In the result layout
// lane l holds rows {4v + l/16 : v = 0..3} of column 16*tile + l%16. All KS operands of
// a column tile are loaded before its MFMAs (one latency per tile); columns past nb
// hold unspecified values. Ends with the rows' operands staged in qa_lds (after a
// workgroup barrier).
template <int NCT, int KS>
__device__ __forceinline__ void reduced_map_strip(const double* __restrict__ qmf, const double* __restrict__ kmf,
                                                  int bh, int rt, int ntile, int nb, double BSA_LDS* qa_lds,
                                                  f64x4_t (&acc)[NCT]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, row0 = rt * SEL_ROWS;
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  const double* qa = qmf + ((int64_t)bh * ntile + rt) * KS * 64;
  for (int x = tid; x < KS * 64; x += SEL_WAVES * 64) qa_lds[x] = row0 + (x & 15) < nb ? qa[x] : 0.0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int ct = w + SEL_WAVES * c;
    if (ct >= ntile) break;
    const double* kb = kmf + ((int64_t)bh * ntile + ct) * KS * 64 + l;
    double bv[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) bv[s] = kb[s * 64];
    f64x4_t a4 = acc[c];
#pragma unroll
    for (int s = 0; s < KS; ++s) a4 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa_lds[s * 64 + l], bv[s], a4, 0, 0, 0);
    acc[c] = a4;
  }
}

// One workgroup of SEL_WAVES waves per tile of 16 query-block rows of one head.
// The reduced map of the 16 rows is an MFMA f64 product (16 rows) x (16-column
// tiles); wave w owns column tiles w, w + SEL_WAVES, ... (NCT of them). In the
// result layout lane l holds rows {4v + l/16 : v = 0..3} of column 16*tile + l%16,
// so a row lives in one 16-lane group of every wave.
// topk > 0 selects the Top-k alternative (NABLA review, Appendix C: a fixed number of
// blocks per row): the same descending order, the radix passes search the key at which
// the COUNT of entries reaches topk instead of the mass reaching 1 - thr.
// NEAR: the near-threshold flags too. An entry's exclusive mass E lies in the band
// [T_lo, T_hi) iff it is kept under target T_hi and not under T_lo, so the radix select
// runs for those two targets as well (on the same keys) and the row's write ORs nothing
// into the flags.
template <int NCT, int KS, bool NEAR>   // KS = D / 4 k-steps of the f64 MFMA
__global__ __launch_bounds__(SEL_WAVES * 64) void select_kernel(const double* __restrict__ qmf,
                                                               const double* __restrict__ kmf, int nb, int D,
                                                               double scale, uint64_t T_fixed, int topk,
                                                               const uint8_t* __restrict__ or_mask, int64_t or_sb,
                                                               int64_t or_sh, StaRule sta, int H,
                                                               uint8_t* __restrict__ mask_out, SelNear nr) {
  constexpr int NTG = NEAR ? 3 : 1;   // targets: the rule; with NEAR also T_lo, T_hi
  const bool by_count = topk > 0;
  __shared__ uint64_t hmass[SEL_ROWS][256];
  __shared__ uint32_t hcnt[SEL_ROWS][256];
  __shared__ uint32_t tiebits[NTG][SEL_ROWS][64];
  __shared__ double red[SEL_ROWS][SEL_WAVES];
  __shared__ uint64_t redu[SEL_ROWS][SEL_WAVES];
  __shared__ uint64_t row_total[SEL_ROWS];
  __shared__ SelRowState st[NTG][SEL_ROWS];
  __shared__ int any_active;
  __shared__ double qa_lds[32 * 64];   // the 16 rows' Qbar operands, MFMA order

  const int bh = blockIdx.y, rt = blockIdx.x, row0 = rt * SEL_ROWS;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, lc = l & 15;
  const int ntile = (nb + 15) / 16;

  // ---- reduced map (columns past nb are masked below)
  f64x4_t acc[NCT];
  reduced_map_strip<NCT, KS>(qmf, kmf, bh, rt, ntile, nb, (double BSA_LDS*)qa_lds, acc);

  // column of value (c) in this lane, its validity; rows of value slot v: 4v + g
  auto colof = [&](int c) { return (w + SEL_WAVES * c) * 16 + lc; };

  // ---- softmax of each row in fp64: max and sum over the 16-lane group, then the waves
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    double m = -INFINITY;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      acc[c][v] *= scale;
      if (colof(c) < nb) m = fmax(m, acc[c][v]);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmax(m, __shfl_xor(m, o, 64));
    if (lc == 0) red[4 * v + g][w] = m;
  }
  __syncthreads();
  double rowmax[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    double m = red[4 * v + g][0];
#pragma unroll
    for (int x = 1; x < SEL_WAVES; ++x) m = fmax(m, red[4 * v + g][x]);
    rowmax[v] = m;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    double sum = 0.0;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const double e = colof(c) < nb ? exp(acc[c][v] - rowmax[v]) : 0.0;
      acc[c][v] = e;
      sum += e;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 64);
    if (lc == 0) red[4 * v + g][w] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    double tot = red[4 * v + g][0];
#pragma unroll
    for (int x = 1; x < SEL_WAVES; ++x) tot += red[4 * v + g][x];    // fixed order: deterministic
    const double inv = 1.0 / tot;
    uint64_t ms = 0;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      // from here on the slot holds the fixed-point mass w = floor(p 2^60), the sort key
      const uint64_t wq = fixed_mass(acc[c][v] * inv);
      acc[c][v] = __longlong_as_double((long long)wq);
      ms += wq;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) ms += __shfl_xor(ms, o, 64);
    if (lc == 0) redu[4 * v + g][w] = ms;
  }
  __syncthreads();
  if (tid < SEL_ROWS) {
    uint64_t total = 0;
    for (int x = 0; x < SEL_WAVES; ++x) total += redu[tid][x];
    row_total[tid] = total;
  }

  for (int t = 0; t < NTG; ++t) {
    const uint64_t target = by_count ? (uint64_t)topk : (t == 0 ? T_fixed : t == 1 ? nr.t_lo : nr.t_hi);
    __syncthreads();   // row totals written; every wave is done with the previous target's state
    if (tid < SEL_ROWS) st[t][tid] = sel_init(row0 + tid >= nb, row_total[tid], target, by_count, nb, topk);
    if (tid == 0) any_active = 1;
    __syncthreads();

    // ---- radix select of the pivot, all rows in lock step
    for (int pass = 0; pass < 9; ++pass) {
      if (!any_active) break;
      for (int x = tid; x < SEL_ROWS * 256; x += SEL_WAVES * 64) {
        hmass[x / 256][x % 256] = 0;
        hcnt[x / 256][x % 256] = 0;
      }
      __syncthreads();
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * v + g;
        const SelRowState sr = st[t][r];
        if (sr.status != ROW_ACTIVE) continue;
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          if (colof(c) >= nb) continue;
          const uint64_t key = (uint64_t)__double_as_longlong(acc[c][v]);
          const int dg = sel_digit(key, sr);
          if (dg >= 0) {
            atomicAdd((unsigned long long*)&hmass[r][dg], (unsigned long long)key);
            atomicAdd(&hcnt[r][dg], 1u);
          }
        }
      }
      __syncthreads();
      // each wave scans SEL_ROWS / SEL_WAVES rows: lane l owns buckets 255-4l .. 252-4l
      for (int r = w; r < SEL_ROWS; r += SEL_WAVES) {
        const SelRowState sr = st[t][r];
        if (sr.status != ROW_ACTIVE) continue;
        uint64_t mb[4];
        uint32_t cb[4];
        uint64_t lt = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          cb[x] = hcnt[r][255 - 4 * l - x];
          mb[x] = by_count ? (uint64_t)cb[x] : hmass[r][255 - 4 * l - x];   // what the target counts
          lt += mb[x];
        }
        const uint64_t incl = wave_incl_scan_u64(lt);
        const uint64_t before = sr.mass_above + (incl - lt);
        const uint64_t ball = __ballot(before + lt >= target);
        const int L = ball ? __builtin_ctzll(ball) : 63;   // the invariant guarantees ball != 0
        if (l == L) {
          uint64_t cum = before;
          int xs = 3;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            if (cum + mb[x] >= target) { xs = x; break; }
            cum += mb[x];
          }
          const int dg = 255 - 4 * l - xs;
          SelRowState n = sr;
          n.mass_above = cum;
          n.cnt = (int)cb[xs];
          if (sr.span < 0) {
            first_range(dg, n.lo, n.span);
          } else {
            const int db = sr.span < 8 ? sr.span : 8;
            n.span = sr.span - db;
            n.lo = sr.lo + ((uint64_t)dg << n.span);
          }
          if (n.cnt <= 1) n.status = ROW_PIVOT;
          else if (n.span == 0) {
            // identical keys: visited by ascending index, each adds the same mass (Top-k: one)
            const uint64_t wq = by_count ? 1 : n.lo;
            const uint64_t need = target - n.mass_above;           // > 0
            const uint64_t tk = wq ? (need + wq - 1) / wq : (uint64_t)n.cnt;
            n.tie_keep = (int)(tk < (uint64_t)n.cnt ? tk : (uint64_t)n.cnt);
            n.status = ROW_TIE;
          }
          st[t][r] = n;
        }
      }
      __syncthreads();
      if (tid == 0) {
        int act = 0;
        for (int r = 0; r < SEL_ROWS; ++r) act |= st[t][r].status == ROW_ACTIVE;
        any_active = act;
      }
      __syncthreads();
    }

    // ---- ties: rank tied entries by ascending column index
    bool need_ties = false;
    for (int r = 0; r < SEL_ROWS; ++r) need_ties |= st[t][r].status == ROW_TIE;
    if (need_ties) {
      for (int x = tid; x < SEL_ROWS * 64; x += SEL_WAVES * 64) tiebits[t][x / 64][x % 64] = 0;
      __syncthreads();
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * v + g;
        if (st[t][r].status != ROW_TIE) continue;
        const uint64_t lo = st[t][r].lo;
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          const int j = colof(c);
          if (j < nb && (uint64_t)__double_as_longlong(acc[c][v]) == lo)
            atomicOr(&tiebits[t][r][j >> 5], 1u << (j & 31));
        }
      }
      __syncthreads();
    }
  }

  // ---- write the mask rows (OR'd with the optional mask and the sliding-tile rule;
  // the rule's tile coordinates of this lane's columns are formed once); with NEAR the
  // flags of the band [T_lo, T_hi) (never OR'd)
  const int b = bh / H, h = bh % H;
  StaCoord cc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) cc[c] = sta.bpt ? sta_rule_coord(sta, min(colof(c), nb - 1)) : StaCoord{0, 0, 0};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * v + g;
    SelRowState srs[NTG];
#pragma unroll
    for (int t = 0; t < NTG; ++t) srs[t] = st[t][r];
    if (srs[0].status == ROW_SKIP) continue;
    const int row = row0 + r;
    const StaCoord rc = sta.bpt ? sta_rule_coord(sta, row) : StaCoord{0, 0, 0};
    uint8_t* dst = mask_out + ((int64_t)bh * nb + row) * nb;
    uint8_t* ndst = NEAR ? nr.flags + ((int64_t)bh * nb + row) * nb : nullptr;
    const uint8_t* om = or_mask ? or_mask + b * or_sb + h * or_sh + (int64_t)row * nb : nullptr;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int j = colof(c);
      if (j >= nb) continue;
      const uint64_t key = (uint64_t)__double_as_longlong(acc[c][v]);
      bool kt[NTG];
#pragma unroll
      for (int t = 0; t < NTG; ++t) {
        const bool tied = srs[t].status == ROW_TIE && key == srs[t].lo;
        int rank = 0;
        if (tied) {
          for (int x = 0; x < (j >> 5); ++x) rank += __popc(tiebits[t][r][x]);
          rank += __popc(tiebits[t][r][j >> 5] & ((1u << (j & 31)) - 1u));
        }
        kt[t] = sel_keep(srs[t], key, tied, rank);
      }
      bool keep = kt[0];
      if constexpr (NEAR) ndst[j] = kt[2] && !kt[1] ? 1 : 0;
      if ((om && om[j]) || (sta.bpt && sta_rule_near(sta, rc, cc[c]))) keep = true;
      dst[j] = keep ? 1 : 0;
    }
  }
}

// ----------------------------------------------------------------------------
// Row selection for short rows (nb <= 256). The same reduced map, fixed-point keys,
// radix digits and tie rule as select_kernel; once the map is formed it is written to
// shared memory, and each wave then owns whole rows: softmax, radix select, tie
// ranking and the row's write use wave reductions, ballots and wave-uniform state only,
// with no workgroup barrier. Column j of a row is entry e = j / 64 of lane j % 64. A
// wave's histogram lives in its own part of shared memory; the shared-memory
// operations of one wave are processed in program order, so a clear, the atomic
// updates and the reads that follow need no wait between them.
// Optionally the kept blocks of each row also go to a fixed-stride kv list (the
// compaction the attention kernel consumes, without a pass of its own over the mask).
// ----------------------------------------------------------------------------

// value of x in lane L (L wave-uniform)
__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int L) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, L);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), L);
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

// Radix digits of the wave-per-row selection, with NBK = 64 << SUB buckets per pass (SUB
// = 2: 256 buckets, 8-bit digits, the scheme of select_kernel). The first pass is
// logarithmic: w < 4 gets bucket w; otherwise, with e the position of the leading one,
// bucket 4 + (e - 2) 2^SUB + (the SUB bits below the leading one), i.e. the range
// [(2^SUB + m) << (e - SUB), (2^SUB + m + 1) << (e - SUB)). Later passes split the current
// range [lo, lo + 2^span) by its top DB = 6 + SUB bits. -1: w is outside the range.
template <int SUB>
__device__ __forceinline__ int row_digit(uint64_t key, const SelRowState& st) {
  constexpr int DB = 6 + SUB;
  if (st.span < 0) {
    if (key < 4) return (int)key;
    const int e = 63 - __builtin_clzll(key);
    return 4 + ((e - 2) << SUB) + (int)((key >> (e - SUB)) & ((1u << SUB) - 1));
  }
  if (key < st.lo || key - st.lo >= (1ull << st.span)) return -1;
  const int db = st.span < DB ? st.span : DB;
  return (int)((key - st.lo) >> (st.span - db));
}

// The selection of one row by one wave: the row's reduced-map values (scaled) are in
// shared memory at mrow[0 .. nb); lane l holds columns j = 64 e + l. Softmax in fp64, the
// fixed-point keys w = floor(p 2^60), a radix select of the pivot for each target with the
// wave's own histograms hm, hc (NBK buckets; the shared-memory operations of one wave are
// processed in program order, so a clear, the atomic updates and the reads that follow
// need no wait between them), ties ranked by ascending index with ballots; then the mask
// row (OR'd with or_row and the sliding-tile rule), the optional near-threshold flags and
// the optional kv list. Every value is wave-uniform except the per-lane entries.
template <int E, int SUB, bool NEAR>
__device__ __forceinline__ void select_row(const double* mrow, int nb, int row, int64_t grow,
                                           uint64_t T_fixed, int topk, const uint8_t* or_row, const StaRule& sta,
                                           uint8_t* __restrict__ mask_out,
                                           const SelLists& lists, const SelNear& nr, uint64_t* hm, uint32_t* hc) {
  constexpr int NBK = 64 << SUB, BPL = NBK / 64, DB = 6 + SUB;
  constexpr int NTG = NEAR ? 3 : 1;                 // targets: the rule; with NEAR also T_lo, T_hi
  const int l = threadIdx.x & 63;
  const bool by_count = topk > 0;
  const StaCoord rc = sta.bpt ? sta_rule_coord(sta, row) : StaCoord{0, 0, 0};
  // ---- softmax of the row in fp64, then the fixed-point mass w = floor(p 2^60) (the key)
  bool valid[E];
  double x[E];
  double m = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 64 * e + l;
    valid[e] = j < nb;
    x[e] = valid[e] ? mrow[j] : -INFINITY;
    m = fmax(m, x[e]);
  }
  m = wave_max_f64(m);
  double sum = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    x[e] = valid[e] ? exp(x[e] - m) : 0.0;
    sum += x[e];
  }
  const double inv = 1.0 / wave_sum_f64(sum);
  uint64_t key[E];
  uint64_t ms = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    key[e] = valid[e] ? fixed_mass(x[e] * inv) : 0;
    ms += key[e];
  }
  const uint64_t total = wave_sum_u64(ms);

  // ---- radix select of the pivot for each target (the row state is wave-uniform), then
  // the target's decision for each of the lane's entries as bit e of kbits[t]; tied keys
  // are ranked by ascending index
  static_assert(E <= 32, "one bit per entry of a lane");
  uint32_t kb_rule = 0, kb_lo = 0, kb_hi = 0;
#pragma unroll 1
  for (int t = 0; t < NTG; ++t) {
    const uint64_t target = by_count ? (uint64_t)topk : (t == 0 ? T_fixed : t == 1 ? nr.t_lo : nr.t_hi);
    SelRowState sr = sel_init(false, total, target, by_count, nb, topk);
    for (int pass = 0; pass < 12 && sr.status == ROW_ACTIVE; ++pass) {
#pragma unroll
      for (int x4 = 0; x4 < BPL; ++x4) {
        hm[BPL * l + x4] = 0;
        hc[BPL * l + x4] = 0;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (!valid[e]) continue;
        const int dg = row_digit<SUB>(key[e], sr);
        if (dg >= 0) {
          atomicAdd((unsigned long long*)&hm[dg], (unsigned long long)key[e]);
          atomicAdd(&hc[dg], 1u);
        }
      }
      __builtin_amdgcn_wave_barrier();
      // lane l owns buckets NBK-1-BPL l .. NBK-BPL(l+1) (descending keys)
      uint64_t mb[BPL];
      uint32_t cb[BPL];
      uint64_t lt = 0;
#pragma unroll
      for (int x4 = 0; x4 < BPL; ++x4) {
        cb[x4] = hc[NBK - 1 - BPL * l - x4];
        mb[x4] = by_count ? (uint64_t)cb[x4] : hm[NBK - 1 - BPL * l - x4];   // what the target counts
        lt += mb[x4];
      }
      const uint64_t incl = wave_incl_scan_u64(lt);
      const uint64_t before = sr.mass_above + (incl - lt);
      const uint64_t ball = __ballot(before + lt >= target);
      const int L = ball ? __builtin_ctzll(ball) : 63;   // the invariant guarantees ball != 0
      // the crossing bucket of lane L, found by every lane from lane L's values
      uint64_t cum = readlane_u64(before, L);
      int xs = BPL - 1, cnt = 0;
#pragma unroll
      for (int x4 = 0; x4 < BPL; ++x4) {
        const uint64_t mbl = readlane_u64(mb[x4], L);
        const int cbl = __builtin_amdgcn_readlane((int)cb[x4], L);
        if (xs == BPL - 1 && x4 < BPL - 1) {
          if (cum + mbl >= target) { xs = x4; cnt = cbl; }
          else cum += mbl;
        } else if (x4 == BPL - 1 && xs == BPL - 1) {
          cnt = cbl;
        }
      }
      const int dg = NBK - 1 - BPL * L - xs;
      SelRowState n = sr;
      n.mass_above = cum;
      n.cnt = cnt;
      if (sr.span < 0) {
        if (dg < 4) {
          n.lo = (uint64_t)dg;
          n.span = 0;
        } else {
          const int e = ((dg - 4) >> SUB) + 2, mm = (dg - 4) & ((1 << SUB) - 1);
          n.lo = (uint64_t)((1 << SUB) + mm) << (e - SUB);
          n.span = e - SUB;
        }
      } else {
        const int db = sr.span < DB ? sr.span : DB;
        n.span = sr.span - db;
        n.lo = sr.lo + ((uint64_t)dg << n.span);
      }
      if (n.cnt <= 1) n.status = ROW_PIVOT;
      else if (n.span == 0) {
        // identical keys: visited by ascending index, each adds the same mass (Top-k: one)
        const uint64_t wq = by_count ? 1 : n.lo;
        const uint64_t need = target - n.mass_above;           // > 0
        const uint64_t tk = wq ? (need + wq - 1) / wq : (uint64_t)n.cnt;
        n.tie_keep = (int)(tk < (uint64_t)n.cnt ? tk : (uint64_t)n.cnt);
        n.status = ROW_TIE;
      }
      sr = n;
    }
    uint32_t bits = 0;
    int tie_base = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool tied = sr.status == ROW_TIE && valid[e] && key[e] == sr.lo;
      const uint64_t tb = __ballot(tied);
      const int rank = tie_base + __popcll(tb & ((1ull << l) - 1ull));
      tie_base += __popcll(tb);
      if (valid[e] && sel_keep(sr, key[e], tied, rank)) bits |= 1u << e;
    }
    if (t == 0) kb_rule = bits;
    else if (t == 1) kb_lo = bits;
    else kb_hi = bits;
  }

  // ---- write the row (OR'd with the optional mask and the sliding-tile rule); with lists,
  // the kept blocks also go to the row's kv list in ascending order; with NEAR the flags
  // of the band [T_lo, T_hi) (never OR'd)
  uint8_t* dst = mask_out + grow * nb;
  uint8_t* ndst = NEAR ? nr.flags + grow * nb : nullptr;
  int32_t* lst = lists.kv_idx ? lists.kv_idx + grow * nb : nullptr;
  const uint32_t nbits = kb_hi & ~kb_lo;
  int nkept = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 64 * e + l;
    bool keep = (kb_rule >> e) & 1u;
    if (valid[e]) {
      if ((or_row && or_row[j]) || (sta.bpt && sta_rule_near(sta, rc, sta_rule_coord(sta, j)))) keep = true;
      dst[j] = keep ? 1 : 0;
      if constexpr (NEAR) ndst[j] = (nbits >> e) & 1u;
    }
    if (lst) {
      const uint64_t kb = __ballot(keep);
      if (keep) lst[nkept + __popcll(kb & ((1ull << l) - 1ull))] = j;
      nkept += __popcll(kb);
    }
  }
  if (lists.kv_len && l == 0) lists.kv_len[grow] = nkept;
}

// ----------------------------------------------------------------------------
// Row selection for short rows (nb <= 256). The same reduced map, fixed-point keys,
// radix digits and tie rule as select_kernel; once the map is formed it is written to
// shared memory, and each wave then owns whole rows (select_row): softmax, radix select,
// tie ranking and the row's write use wave reductions, ballots and wave-uniform state
// only, with no workgroup barrier. Optionally the kept blocks of each row also go to a
// fixed-stride kv list (the compaction the attention kernel consumes, without a pass of
// its own over the mask).
// Each 16-row strip of the map is formed by SELR_SPLIT workgroups (the same small fp64
// product, recomputed), each taking SEL_ROWS / SELR_SPLIT of its rows: more workgroups
// and fewer rows one after the other in a wave.
// ----------------------------------------------------------------------------
constexpr int SELR_SPLIT = 2;
template <int NCT, int KS, bool NEAR>   // NCT = column tiles per wave (nb <= 128 NCT)
__global__ __launch_bounds__(SEL_WAVES * 64) void select_rows_kernel(const double* __restrict__ qmf,
                                                                    const double* __restrict__ kmf, int nb,
                                                                    double scale, uint64_t T_fixed, int topk,
                                                                    const uint8_t* __restrict__ or_mask,
                                                                    int64_t or_sb, int64_t or_sh, StaRule sta,
                                                                    int H, uint8_t* __restrict__ mask_out,
                                                                    SelLists lists, SelNear nr) {
  constexpr int E = 2 * NCT;                        // entries per lane per row
  constexpr int NBP = SEL_WAVES * 16 * NCT;         // map row length
  __shared__ double qa_lds[32 * 64];
  __shared__ double map[SEL_ROWS][NBP];
  __shared__ uint64_t hmass[SEL_WAVES][256];
  __shared__ uint32_t hcnt[SEL_WAVES][256];

  // strip rt of 16 rows; part `part` of its rows is this workgroup's
  const int bh = blockIdx.y, rt = blockIdx.x / SELR_SPLIT, part = blockIdx.x % SELR_SPLIT, row0 = rt * SEL_ROWS;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, lc = l & 15;
  const int ntile = (nb + 15) / 16;

  f64x4_t acc[NCT];
  reduced_map_strip<NCT, KS>(qmf, kmf, bh, rt, ntile, nb, (double BSA_LDS*)qa_lds, acc);
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int ct = w + SEL_WAVES * c;
    if (ct >= ntile) break;
#pragma unroll
    for (int v = 0; v < 4; ++v) map[4 * v + g][ct * 16 + lc] = acc[c][v] * scale;
  }
  __syncthreads();

  const int b = bh / H, h = bh % H;
  constexpr int RPW = SEL_ROWS / SEL_WAVES / SELR_SPLIT;   // rows per wave
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = part * (SEL_ROWS / SELR_SPLIT) + RPW * w + rr, row = row0 + r;
    if (row >= nb) break;                            // wave-uniform
    const uint8_t* om = or_mask ? or_mask + b * or_sb + h * or_sh + (int64_t)row * nb : nullptr;
    select_row<E, 2, NEAR>(&map[r][0], nb, row, (int64_t)bh * nb + row, T_fixed, topk, om, sta, mask_out, lists, nr,
                           &hmass[w][0], &hcnt[w][0]);
  }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <typename T, int D, bool NT>
static void launch_pool_v(dim3 grid, hipStream_t st, const void* q, const int64_t* qs, const void* k,
                          const int64_t* ks, int H, int nb, double* qbar, double* kbarT, const Fp8Out* f8) {
  const Fp8Out none = {};
  if (!f8)
    hipLaunchKernelGGL((pool_kernel<T, D, NT, true, false>), grid, dim3(256), 0, st, (const T*)q, qs[0], qs[1],
                       qs[2], (const T*)k, ks[0], ks[1], ks[2], H, nb, qbar, kbarT, none);
  else if (f8->rot && qbar)
    hipLaunchKernelGGL((pool_kernel<T, D, NT, true, true, true>), grid, dim3(256), 0, st, (const T*)q, qs[0],
                       qs[1], qs[2], (const T*)k, ks[0], ks[1], ks[2], H, nb, qbar, kbarT, *f8);
  else if (f8->rot)
    hipLaunchKernelGGL((pool_kernel<T, D, NT, false, true, true>), grid, dim3(256), 0, st, (const T*)q, qs[0],
                       qs[1], qs[2], (const T*)q, qs[0], qs[1], qs[2], H, nb, nullptr, nullptr, *f8);
  else if (qbar)
    hipLaunchKernelGGL((pool_kernel<T, D, NT, true, true>), grid, dim3(256), 0, st, (const T*)q, qs[0], qs[1],
                       qs[2], (const T*)k, ks[0], ks[1], ks[2], H, nb, qbar, kbarT, *f8);
  else
    hipLaunchKernelGGL((pool_kernel<T, D, NT, false, true>), grid, dim3(256), 0, st, (const T*)q, qs[0], qs[1],
                       qs[2], (const T*)q, qs[0], qs[1], qs[2], H, nb, nullptr, nullptr, *f8);
}

template <typename T, int D>
static hipError_t launch_pool_t(const void* q, const int64_t* qs, const void* k, const int64_t* ks, int B,
                                int H, int nb, double* qbar, double* kbarT, const Fp8Out* f8, hipStream_t st) {
  const int tensors = qbar ? 2 : 1;
  dim3 grid((nb + POOL_BPW - 1) / POOL_BPW, B * H, tensors);
  // inputs far larger than the 256 MB last-level cache are streamed past it
  const bool nt = (double)tensors * B * H * nb * BSA_N * D * sizeof(T) > 512.0 * (1 << 20);
  if (nt) launch_pool_v<T, D, true>(grid, st, q, qs, k, ks, H, nb, qbar, kbarT, f8);
  else launch_pool_v<T, D, false>(grid, st, q, qs, k, ks, H, nb, qbar, kbarT, f8);
  return hipGetLastError();
}

hipError_t launch_pool(bool f32, int D, const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                       int B, int H, int nb, double* qbar, double* kbarT, const Fp8Out* f8, hipStream_t st) {
  if (f32) return D == 64 ? launch_pool_t<float, 64>(q, qs, k, ks, B, H, nb, qbar, kbarT, f8, st)
                          : launch_pool_t<float, 128>(q, qs, k, ks, B, H, nb, qbar, kbarT, f8, st);
  return D == 64 ? launch_pool_t<u16, 64>(q, qs, k, ks, B, H, nb, qbar, kbarT, f8, st)
                 : launch_pool_t<u16, 128>(q, qs, k, ks, B, H, nb, qbar, kbarT, f8, st);
}

template <int NCT, bool NEAR>
static hipError_t launch_select_c(const double* qmf, const double* kmf, int B, int H, int nb, int D,
                                  double scale, uint64_t T_fixed, int topk, const uint8_t* or_mask, int64_t or_sb,
                                  int64_t or_sh, StaRule sta, uint8_t* mask_out, hipStream_t st, const SelNear& nr) {
  dim3 grid((nb + SEL_ROWS - 1) / SEL_ROWS, B * H);
  if (D == 64)
    hipLaunchKernelGGL((select_kernel<NCT, 16, NEAR>), grid, dim3(SEL_WAVES * 64), 0, st, qmf, kmf, nb, D, scale,
                       T_fixed, topk, or_mask, or_sb, or_sh, sta, H, mask_out, nr);
  else
    hipLaunchKernelGGL((select_kernel<NCT, 32, NEAR>), grid, dim3(SEL_WAVES * 64), 0, st, qmf, kmf, nb, D, scale,
                       T_fixed, topk, or_mask, or_sb, or_sh, sta, H, mask_out, nr);
  return hipGetLastError();
}

template <int NCT, bool NEAR>
static hipError_t launch_select_rows(const double* qmf, const double* kmf, int B, int H, int nb, int D, double scale,
                                     uint64_t T_fixed, int topk, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                                     StaRule sta, uint8_t* mask_out, hipStream_t st, const SelLists& lists,
                                     const SelNear& nr) {
  dim3 grid((nb + SEL_ROWS - 1) / SEL_ROWS * SELR_SPLIT, B * H);
  if (D == 64)
    hipLaunchKernelGGL((select_rows_kernel<NCT, 16, NEAR>), grid, dim3(SEL_WAVES * 64), 0, st, qmf, kmf, nb, scale,
                       T_fixed, topk, or_mask, or_sb, or_sh, sta, H, mask_out, lists, nr);
  else
    hipLaunchKernelGGL((select_rows_kernel<NCT, 32, NEAR>), grid, dim3(SEL_WAVES * 64), 0, st, qmf, kmf, nb, scale,
                       T_fixed, topk, or_mask, or_sb, or_sh, sta, H, mask_out, lists, nr);
  return hipGetLastError();
}

template <bool NEAR>
static hipError_t launch_select_n(const double* qmf, const double* kmf, int B, int H, int nb, int D, double scale,
                                  uint64_t T_fixed, int topk, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                                  StaRule sta, uint8_t* mask_out, hipStream_t st, const SelLists& lists,
                                  const SelNear& nr) {
  const int ntile = (nb + 15) / 16;
  const int nct = (ntile + SEL_WAVES - 1) / SEL_WAVES;
  if (nb <= SELR_MAX_NB) {
    if (nct == 1)
      return launch_select_rows<1, NEAR>(qmf, kmf, B, H, nb, D, scale, T_fixed, topk, or_mask, or_sb, or_sh, sta,
                                         mask_out, st, lists, nr);
    return launch_select_rows<2, NEAR>(qmf, kmf, B, H, nb, D, scale, T_fixed, topk, or_mask, or_sb, or_sh, sta,
                                       mask_out, st, lists, nr);
  }
  if (lists.kv_idx || lists.kv_len) return hipErrorInvalidValue;   // short rows only
#define BSA_SEL_CASE(n)                                                                                         \
  case n:                                                                                                      \
    return launch_select_c<n, NEAR>(qmf, kmf, B, H, nb, D, scale, T_fixed, topk, or_mask, or_sb, or_sh, sta, \
                                    mask_out, st, nr);
  switch (nct) {   // nb > SELR_MAX_NB: 17 .. 128 column tiles
    BSA_SEL_CASE(3) BSA_SEL_CASE(4) BSA_SEL_CASE(5) BSA_SEL_CASE(6) BSA_SEL_CASE(7) BSA_SEL_CASE(8)
    BSA_SEL_CASE(9) BSA_SEL_CASE(10) BSA_SEL_CASE(11) BSA_SEL_CASE(12) BSA_SEL_CASE(13) BSA_SEL_CASE(14)
    BSA_SEL_CASE(15) BSA_SEL_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef BSA_SEL_CASE
}

hipError_t launch_select(const double* qmf, const double* kmf, int B, int H, int nb, int D, double scale,
                         uint64_t T_fixed, int topk, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                         StaRule sta, uint8_t* mask_out, hipStream_t st, const SelLists& lists,
                         const SelNear& near) {
  if (near.flags)
    return launch_select_n<true>(qmf, kmf, B, H, nb, D, scale, T_fixed, topk, or_mask, or_sb, or_sh, sta, mask_out, st,
                                 lists, near);
  return launch_select_n<false>(qmf, kmf, B, H, nb, D, scale, T_fixed, topk, or_mask, or_sb, or_sh, sta, mask_out, st,
                                lists, near);
}

}  // namespace bsa
