// Gradients of block-sparse attention on gfx950 (bf16 MFMA, fp32 accumulation).
//
// Method: FlashAttention (Daily Papers listing) trains with exact tiled attention and
// extends it to block-sparse attention over the listed blocks; the NABLA review (Pith
// review, "Editorial extensions") trains a DiT with the NABLA block mask. The pages
// print no backward formulas; the kernels compute the derivative of the forward
// definition, tile by tile over the kept 64 x 64 blocks, recomputing the
// probabilities from the forward's log-sum-exp instead of storing them:
//   P = exp(scale S - lse),  dV = P^T dO,  dP = dO V^T,  delta = rowsum(dO * O),
//   dS = P * (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q.
//
// Kernels:
//   bwd_prep_kernel   delta and the log-sum-exp in log2 units, one pass over O and dO;
//   mask_transpose_kernel  the block mask transposed, whose compaction gives each key
//                     block its list of query blocks;
//   bwd_dkdv_kernel   one 8-wave workgroup per pair of key blocks, walking the union of
//                     their query-block lists: dK and dV stay in registers, K and V in LDS;
//   bwd_dq_kernel     one 4-wave workgroup per pair of query blocks walking the union of
//                     their kv lists (the forward's decomposition): dQ stays in registers.
// No atomics: every output element is written once, so results are run-to-run exact.
#include "common.h"
#include "item_order.h"
#include "launch.h"
#include "lds_tile.h"

namespace bsa {

// ---- delta_p = <dO_p, O_p> and lse2_p = lse_p log2(e) -----------------------------
// One workgroup of 256 threads per 64 rows. Rows that carry no gradient (padded rows,
// rows with no allowed key: lse = -inf) get lse2 = +inf, so that exp2(x - lse2) = 0.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a, float2* __restrict__ ld) {
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int RPP = 256 / CH;             // rows per pass
  const int t = threadIdx.x, c = t % CH;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const char* ob = (const char*)a.o + (b * a.o_sb + h * a.o_sh) * 2;
  const char* gb = (const char*)a.d_o + (b * a.do_sb + h * a.do_sh) * 2;
#pragma unroll
  for (int p = 0; p < 64 / RPP; ++p) {
    const int r = blockIdx.x * 64 + p * RPP + t / CH;
    const i32x4_t x = *(const i32x4_t*)(ob + (int64_t)r * a.o_ss * 2 + c * 16);
    const i32x4_t y = *(const i32x4_t*)(gb + (int64_t)r * a.do_ss * 2 + c * 16);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(__uint_as_float((unsigned)x[e] << 16), __uint_as_float((unsigned)y[e] << 16), s);
      s = fmaf(__uint_as_float((unsigned)x[e] & 0xffff0000u), __uint_as_float((unsigned)y[e] & 0xffff0000u), s);
    }
#pragma unroll
    for (int o = CH / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (c == 0) {
      const int64_t row = (int64_t)bh * a.S + r;
      const float lse = a.lse[row];
      const bool live = r < a.S_valid && lse > -INFINITY;
      ld[row] = make_float2(live ? lse * 1.4426950408889634f : INFINITY, s);
    }
  }
}

// ---- transposed block mask: mt[bh][j][i] = m[b*sb + h*sh + i*nb + j] -------------
__global__ __launch_bounds__(256) void mask_transpose_kernel(const uint8_t* __restrict__ m, int64_t sb, int64_t sh,
                                                             int H, int nb, uint8_t* __restrict__ mt) {
  __shared__ uint8_t tile[64][65];
  const int bh = blockIdx.z, b = bh / H, h = bh % H;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const uint8_t* src = m + b * sb + h * sh;
  uint8_t* dst = mt + (int64_t)bh * nb * nb;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64;
    tile[r][c] = (i0 + r < nb && j0 + c < nb) ? src[(int64_t)(i0 + r) * nb + j0 + c] : 0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64;             // output row j0 + r, column i0 + c
    if (j0 + r < nb && i0 + c < nb) dst[(int64_t)(j0 + r) * nb + i0 + c] = tile[c][r];
  }
}

// ---- output stores ----------------------------------------------------------------
// Accumulator acc[dt] holds X^T for one 32-column group: rows d = 32 dt + 8 (v/4) +
// 4 hi + v%4, column = this lane's token. Writes token row `tok` of X (times mul).
template <int D, bool F32>
__device__ __forceinline__ void store_rows(void* base, int64_t tok_off, const f32x16_t* acc, float mul, int hi) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * hi;
      if constexpr (F32) {
        *(f32x4_t*)((float*)base + tok_off + d) =
            f32x4_t{acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul, acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul};
      } else {
        uint2 w;
        w.x = pk_bf16(acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul);
        w.y = pk_bf16(acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul);
        *(uint2*)((u16*)base + tok_off + d) = w;
      }
    }
}

// Eight consecutive accumulator values (base, base + 1, ...) -> one bf16x8 operand
__device__ __forceinline__ bf16x8_t pack8(const float* x) {
  i32x4_t w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (int)pk_bf16(x[2 * e], x[2 * e + 1]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// Natural item of this workgroup, or -1: one contiguous range of the items per XCD, or
// (shared) the plain order, in which all eight XCDs walk one head together, so that its
// tiles stay in the last-level cache. The kernels share where the heads pair blocks at an
// offset above 1 (scattered lists; the forward shares ranges between pairs of XCDs there,
// the backward gains more from sharing among all eight).
__device__ __forceinline__ int xcd_range_item(int total, bool shared) {
  if (shared) return (int)blockIdx.x < total ? (int)blockIdx.x : -1;
  const int chunk = (total + BSA_NXCD - 1) / BSA_NXCD;
  const int lin = (int)(blockIdx.x % BSA_NXCD) * chunk + (int)(blockIdx.x / BSA_NXCD);
  return lin < total ? lin : -1;
}

// ---- dK, dV -------------------------------------------------------------------------
// One workgroup of eight waves per PAIR of adjacent key blocks (2p, 2p+1). Wave w works
// on key block 2p + (w >> 2); inside it, it owns keys 32 (w & 1) .. +32 (its MFMA
// columns) and the query half (w >> 1) & 1 of every query tile. K and V of both key
// blocks stay in LDS for the whole walk (K-swizzled: read by rows as B operands). The
// workgroup walks the union of the two blocks' query-block lists in ascending order;
// per query block i (used by the key blocks whose list holds it):
//   * the Q and dO tiles of i (64 x D each) and (lse2, delta) of its 64 queries are
//     copied global -> LDS (direct-to-LDS loads split over the eight waves,
//     double-buffered, one barrier per step); the tiles are V-swizzled: they are read
//     both by rows and transposed;
//   * S = Q K^T -> P = exp2(S scale log2e - lse2) -> dV^T += dO^T P, then
//     dP = dO V^T -> dS = P (dP - delta) -> dK^T += Q^T dS, for the wave's 32 x 32
//     block; P and dS are packed to bf16 as B operands and the A operands dO^T, Q^T
//     are read with transposing LDS reads (the forward's P V step with the query
//     index contracted).
// The two query halves' partial dK^T, dV^T are summed through LDS at the end.
template <int D, bool F32, bool BITS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a, const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx,
                     const float2* __restrict__ ld) {
  constexpr int RB = D * 2, KT = 64 * RB, DT = D / 32, KS = D / 16;
  constexpr int SLOT = 2 * KT + 1024;               // Q tile, dO tile, 128 (lse2, delta) pairs
  constexpr int KV0 = 2 * SLOT;                     // K0, V0, K1, V1 after the two slots
  __shared__ __attribute__((aligned(1024))) char smem[2 * SLOT + 4 * KT];
  static_assert(2 * SLOT + 4 * KT >= 8 * DT * 16 * 64 * 4, "LDS too small for the final exchange");
  char BSA_LDS* lds = (char BSA_LDS*)smem;

  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = wave >> 2, kh = wave & 1, qh = (wave >> 1) & 1;
  const int l32 = l & 31, hi = l >> 5, g16 = l & 15, mbase = 16 * ((l >> 4) & 1);

  const int npair = (a.nb + 1) / 2;
  const int total = a.B * a.H * npair;
  int lin = xcd_range_item(total, a.derive_order && a.pair_dk && a.pair_dk[0] > 1);
  if (lin < 0) return;
  if (a.derive_order && kth_longest_fits(a.nb, npair, sizeof(smem))) {
    // the same ranges, longest first inside each head (natural order where its tables
    // would not fit in smem)
    const int head0 = lin / npair * npair;
    lin = kth_longest_item<512>([&](int r) { return col_ptr[r + 1] - col_ptr[r]; }, a.nb, (int*)smem, head0,
                                npair, lin - head0, a.pair_dk);
  }
  const int bh = lin / npair;
  const int b = bh / a.H, h = bh % a.H;
  // the pair's two key blocks: adjacent, or at the head's pairing offset
  const int2 pb = pair_blocks(lin % npair, a.pair_dk ? a.pair_dk[bh] : 1, a.nb);
  const int jA = pb.x, jB = pb.y;
  const bool hasB = jB >= 0;
  const int sA = col_ptr[bh * a.nb + jA], eA = col_ptr[bh * a.nb + jA + 1];
  const int sB = hasB ? col_ptr[bh * a.nb + jB] : 0, eB = hasB ? col_ptr[bh * a.nb + jB + 1] : 0;
  const bool mine_valid = kb == 0 || hasB;
  const int j = mine_valid && kb ? jB : jA;         // this wave's key block

  const char* qbase = (const char*)a.q + (b * a.q_sb + h * a.q_sh) * 2;
  const char* dobase = (const char*)a.d_o + (b * a.do_sb + h * a.do_sh) * 2;
  const unsigned q_rs = (unsigned)(a.q_ss * 2), do_rs = (unsigned)(a.do_ss * 2);
  const float2* ldb = ld + (int64_t)bh * a.S;

  // K and V of both key blocks into LDS once (a missing second block copies the first)
  {
    const char* kbase = (const char*)a.k + (b * a.k_sb + h * a.k_sh) * 2;
    const char* vbase = (const char*)a.v + (b * a.v_sb + h * a.v_sh) * 2;
    const unsigned k_rs = (unsigned)(a.k_ss * 2), v_rs = (unsigned)(a.v_ss * 2);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int jx = x && hasB ? jB : jA;
      load_tile_part<RB, false, 8>(kbase + (int64_t)jx * 64 * k_rs, k_rs, (unsigned)(uintptr_t)(lds + KV0 + 2 * x * KT),
                                   l, wave);
      load_tile_part<RB, false, 8>(vbase + (int64_t)jx * 64 * v_rs, v_rs,
                                   (unsigned)(uintptr_t)(lds + KV0 + (2 * x + 1) * KT), l, wave);
    }
  }
  // lane bases of the operand reads (an XOR swizzle moves only offset bits below log2 RB,
  // so the offset of byte column cb in a row is the row's offset ^ cb; slot offsets are
  // multiples of 1024 and leave those bits alone): Q / dO rows 32 qh + l32, K / V rows
  // 32 kh + l32 of this wave's key block, transposed dO / Q reads at rows
  // 32 qh + 16 sp + {0, 8} + 4 hi + g16 / 4 and d tile dt
  const int q_row = voff<RB>(qh * 32 + l32, 16 * hi);
  const int kv_row = KV0 + 2 * kb * KT + koff<RB>(kh * 32 + l32, 16 * hi);
  const int q_tr = voff<RB>(32 * qh + 4 * hi + (g16 >> 2), (mbase + 4 * (g16 & 3)) * 2);
  const int key = j * 64 + kh * 32 + l32;
  const bool kvalid = key < a.S_valid;
  const float c2 = a.scale_log2;

  auto dma = [&](int st, int i) {
    char BSA_LDS* sl = lds + st * SLOT;
    load_tile_part<RB, true, 8>(qbase + (int64_t)i * 64 * q_rs, q_rs, (unsigned)(uintptr_t)sl, l, wave);
    load_tile_part<RB, true, 8>(dobase + (int64_t)i * 64 * do_rs, do_rs, (unsigned)(uintptr_t)(sl + KT), l, wave);
    // (lse2, delta) of queries 64 i .. 64 i + 127 (the array is padded by 64 entries)
    if (wave == 0) dma16((const char*)(ldb + (int64_t)i * 64), (unsigned)l * 16u, (unsigned)(uintptr_t)(sl + 2 * KT));
  };

  // union walk over the two query-block lists (wave-uniform scalar state), or over their
  // bit rows
  int ia = sA, ib = sB, cbA = sA, cbB = sB, cacheA = 0, cacheB = 0;
  auto fetch = [&](int base, int e, int& cache) { cache = row_idx[min(base + l, e - 1)]; };
  BitUnionWalk bw;
  if constexpr (BITS) {
    bw.init(a.bits_k, (int64_t)bh * a.nb + jA, hasB ? (int64_t)bh * a.nb + jB : -1, a.nw);
  } else {
    if (sA < eA) fetch(cbA, eA, cacheA);
    if (sB < eB) fetch(cbB, eB, cacheB);
  }
  __builtin_amdgcn_s_waitcnt(0);
  auto next_entry = [&](int& flags) -> int {
    if constexpr (BITS) return bw.next(flags);
    const int BIG = 0x7fffffff;
    if (ia < eA && ia - cbA == 64) { cbA += 64; fetch(cbA, eA, cacheA); __builtin_amdgcn_s_waitcnt(0); }
    if (ib < eB && ib - cbB == 64) { cbB += 64; fetch(cbB, eB, cacheB); __builtin_amdgcn_s_waitcnt(0); }
    const int ja = ia < eA ? __builtin_amdgcn_readlane(cacheA, ia - cbA) : BIG;
    const int jb = ib < eB ? __builtin_amdgcn_readlane(cacheB, ib - cbB) : BIG;
    const int jm = min(ja, jb);
    if (jm == BIG) { flags = 0; return -1; }
    if (!BSA_CHECK(jm >= 0 && jm < a.nb, CHK_BWD_ENTRY)) { flags = 0; return -1; }
    flags = (ja == jm ? 1 : 0) | (jb == jm ? 2 : 0);
    ia += ja == jm;
    ib += jb == jm;
    return jm;
  };

  f32x16_t dvT[DT], dkT[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dvT[dt][v] = dkT[dt][v] = 0.f;

  int f0 = 0, f1 = 0;
  int i0 = next_entry(f0);
  int i1 = i0 >= 0 ? next_entry(f1) : -1;
  if (i0 >= 0) dma(0, i0);
  for (int u = 0; i0 >= 0; ++u) {
    const int st = u & 1;
    wait_vm<0>();
    wg_barrier();                      // tile u (and K, V) everywhere; step u-1 done with slot st ^ 1
    if (i1 >= 0) dma(st ^ 1, i1);
    if (((f0 >> kb) & 1) && i0 * 64 < a.S_valid) {
      const char BSA_LDS* sq = lds + st * SLOT;
      const float BSA_LDS* sld = (const float BSA_LDS*)(sq + 2 * KT);
      const f32x16_t zero16 = {};
      const int qr = opaque(q_row + st * SLOT), qt = opaque(q_tr + st * SLOT), kvr = opaque(kv_row);
      // S = Q K^T: rows q = 32 qh + 8 (v/4) + 4 hi + v%4, column = key
      f32x16_t acc = zero16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t aq = *(const bf16x8_t BSA_LDS*)(lds + (qr ^ (32 * s)));
        const bf16x8_t bk = *(const bf16x8_t BSA_LDS*)(lds + (kvr ^ (32 * s)));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, acc, 0, 0, 0);
      }
      // P; (lse2, delta) of the 4 consecutive rows of group v/4 in two 16-byte reads
      float p[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q0 = qh * 32 + 8 * g + 4 * hi;
        const f32x4_t x0 = *(const f32x4_t BSA_LDS*)(sld + 2 * q0);
        const f32x4_t x1 = *(const f32x4_t BSA_LDS*)(sld + 2 * q0 + 4);
        const float lse2[4] = {x0[0], x0[2], x1[0], x1[2]};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p[4 * g + e] = kvalid ? __builtin_amdgcn_exp2f(fmaf(acc[4 * g + e], c2, -lse2[e])) : 0.f;
      }
      // dV^T += dO^T P (contraction over the wave's 32 queries; A read transposed)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const bf16x8_t pb = pack8(p + 8 * sp);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const char BSA_LDS* o = lds + KT + (qt ^ (64 * dt)) + 16 * sp * RB;
          const s16x4_t o0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)o);
          const s16x4_t o1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)(o + 8 * RB));
          dvT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(o0, o1), pb, dvT[dt], 0, 0, 0);
        }
      }
      // dP = dO V^T, then dS = P (dP - delta)
      acc = zero16;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t ad = *(const bf16x8_t BSA_LDS*)(lds + KT + (qr ^ (32 * s)));
        const bf16x8_t bv = *(const bf16x8_t BSA_LDS*)(lds + KT + (kvr ^ (32 * s)));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, bv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q0 = qh * 32 + 8 * g + 4 * hi;
        const f32x4_t x0 = *(const f32x4_t BSA_LDS*)(sld + 2 * q0);
        const f32x4_t x1 = *(const f32x4_t BSA_LDS*)(sld + 2 * q0 + 4);
        const float dl[4] = {x0[1], x0[3], x1[1], x1[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * g + e] *= acc[4 * g + e] - dl[e];
      }
      // dK^T += Q^T dS
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const bf16x8_t db = pack8(p + 8 * sp);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const char BSA_LDS* o = lds + (qt ^ (64 * dt)) + 16 * sp * RB;
          const s16x4_t q0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)o);
          const s16x4_t q1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)(o + 8 * RB));
          dkT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(q0, q1), db, dkT[dt], 0, 0, 0);
        }
      }
    }
    wait_lgkm0();                      // reads of slot st done before the next barrier
    int f2 = 0;
    const int i2 = i1 >= 0 ? next_entry(f2) : -1;
    i0 = i1; f0 = f1;
    i1 = i2; f1 = f2;
  }

  // ---- sum the two query halves: half 1 hands over its dV^T, half 0 its dK^T
  wait_vm<0>();
  wg_barrier();                        // every wave is past its last read of LDS
  float BSA_LDS* xch = (float BSA_LDS*)lds;
  constexpr int REG = DT * 16 * 64;    // floats of one wave's accumulator set
  {
    float BSA_LDS* mine = xch + wave * REG;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mine[(dt * 16 + v) * 64 + l] = qh ? dvT[dt][v] : dkT[dt][v];
  }
  wait_lgkm0();
  wg_barrier();
  {
    const float BSA_LDS* other = xch + (wave ^ 2) * REG;   // same key block and keys, other query half
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x = other[(dt * 16 + v) * 64 + l];
        if (qh) dkT[dt][v] += x; else dvT[dt][v] += x;
      }
  }
  if (!mine_valid) return;
  if (qh == 0)
    store_rows<D, F32>(a.dv, b * a.dv_sb + h * a.dv_sh + (int64_t)key * a.dv_ss, dvT, 1.f, hi);
  else
    store_rows<D, F32>(a.dk, b * a.dk_sb + h * a.dk_sh + (int64_t)key * a.dk_ss, dkT, a.scale, hi);
}

// ---- dQ -----------------------------------------------------------------------------
// The forward's decomposition: one workgroup of four waves per pair of adjacent query
// blocks (2p, 2p+1), waves 0-1 on block 2p and 2-3 on block 2p+1, 32 queries each,
// walking the union of the two kv lists in ascending order. Per kv tile (K and V
// double-buffered in LDS, one barrier per step):
//   * S^T = K Q^T and dP^T = V dO^T, Q and dO of the wave's queries being the B
//     operands in registers; each lane owns one query, so lse2 and delta are scalars;
//   * P^T = exp2(S^T scale log2e - lse2), dS^T = P^T (dP^T - delta), packed to bf16;
//   * dQ^T += K^T dS^T with K^T read by transposing LDS reads (the K tile is
//     V-swizzled for that; V is read by rows only and is K-swizzled).
template <int D, bool F32, bool BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                   const float2* __restrict__ ld) {
  constexpr int RB = D * 2, KT = 64 * RB, DT = D / 32, KS = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[4 * KT];     // [stage][K, V]
  char BSA_LDS* lds = (char BSA_LDS*)smem;

  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pr = wave >> 1, wv = wave & 1;
  const int l32 = l & 31, hi = l >> 5, g16 = l & 15, mbase = 16 * ((l >> 4) & 1);

  const int npair = (a.nb + 1) / 2;
  const int total = a.B * a.H * npair;
  int lin = xcd_range_item(total, a.derive_order && a.pair_dq && a.pair_dq[0] > 1);
  if (lin < 0) return;
  if (a.derive_order && kth_longest_fits(a.nb, npair, sizeof(smem))) {
    // the same ranges, longest first inside each head (natural order where its tables
    // would not fit in smem)
    const int head0 = lin / npair * npair;
    lin = kth_longest_item<256>([&](int r) { return row_ptr[r + 1] - row_ptr[r]; }, a.nb, (int*)smem, head0,
                                npair, lin - head0, a.pair_dq);
  }
  const int bh = lin / npair, pidx = lin % npair;
  const int b = bh / a.H, h = bh % a.H;
  // the pair's two query blocks: adjacent, or at the head's pairing offset
  const int2 pb = pair_blocks(pidx, a.pair_dq ? a.pair_dq[bh] : 1, a.nb);
  const int iA = pb.x, iB = pb.y;
  const bool hasB = iB >= 0;
  const int rowA = bh * a.nb + iA, rowB = bh * a.nb + iB;
  const int sA = row_ptr[rowA], eA = row_ptr[rowA + 1];
  const int sB = hasB ? row_ptr[rowB] : 0, eB = hasB ? row_ptr[rowB + 1] : 0;
  const int i = pr ? iB : iA;
  const bool mine_valid = pr == 0 || hasB;

  const char* kbase = (const char*)a.k + (b * a.k_sb + h * a.k_sh) * 2;
  const char* vbase = (const char*)a.v + (b * a.v_sb + h * a.v_sh) * 2;
  const unsigned k_rs = (unsigned)(a.k_ss * 2), v_rs = (unsigned)(a.v_ss * 2);
  auto k_lds = [&](int st) { return lds + st * 2 * KT; };
  auto v_lds = [&](int st) { return lds + st * 2 * KT + KT; };
  auto dma = [&](int st, int jt) {
    load_tile_part<RB, true, 4>(kbase + (int64_t)jt * 64 * k_rs, k_rs, (unsigned)(uintptr_t)k_lds(st), l, wave);
    load_tile_part<RB, false, 4>(vbase + (int64_t)jt * 64 * v_rs, v_rs, (unsigned)(uintptr_t)v_lds(st), l, wave);
  };

  // Q and dO of this lane's query as B operands (inner d = 16 s + 8 hi + e)
  const int qtok = (mine_valid ? i : iA) * 64 + wv * 32 + l32;
  bf16x8_t qop[KS], dop[KS];
  {
    const char* qr = (const char*)a.q + (b * a.q_sb + h * a.q_sh + (int64_t)qtok * a.q_ss) * 2;
    const char* gr = (const char*)a.d_o + (b * a.do_sb + h * a.do_sh + (int64_t)qtok * a.do_ss) * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qop[s] = *(const bf16x8_t*)(qr + (16 * s + 8 * hi) * 2);
      dop[s] = *(const bf16x8_t*)(gr + (16 * s + 8 * hi) * 2);
    }
  }
  const float2 lq = ld[(int64_t)bh * a.S + qtok];
  const float lse2 = lq.x, delta = lq.y, c2 = a.scale_log2;

  // union walk over the two kv lists (the forward's), or over their bit rows
  int ia = sA, ib = sB, cbA = sA, cbB = sB, cacheA = 0, cacheB = 0;
  auto fetch = [&](int base, int e, int& cache) { cache = col_idx[min(base + l, e - 1)]; };
  BitUnionWalk bw;
  if constexpr (BITS) {
    bw.init(a.bits_q, rowA, hasB ? (int64_t)rowB : -1, a.nw);
  } else {
    if (sA < eA) fetch(cbA, eA, cacheA);
    if (sB < eB) fetch(cbB, eB, cacheB);
  }
  __builtin_amdgcn_s_waitcnt(0);
  auto next_entry = [&](int& flags) -> int {
    if constexpr (BITS) return bw.next(flags);
    const int BIG = 0x7fffffff;
    if (ia < eA && ia - cbA == 64) { cbA += 64; fetch(cbA, eA, cacheA); __builtin_amdgcn_s_waitcnt(0); }
    if (ib < eB && ib - cbB == 64) { cbB += 64; fetch(cbB, eB, cacheB); __builtin_amdgcn_s_waitcnt(0); }
    const int ja = ia < eA ? __builtin_amdgcn_readlane(cacheA, ia - cbA) : BIG;
    const int jb = ib < eB ? __builtin_amdgcn_readlane(cacheB, ib - cbB) : BIG;
    const int jm = min(ja, jb);
    if (jm == BIG) { flags = 0; return -1; }
    if (!BSA_CHECK(jm >= 0 && jm < a.nb, CHK_BWD_ENTRY)) { flags = 0; return -1; }
    flags = (ja == jm ? 1 : 0) | (jb == jm ? 2 : 0);
    ia += ja == jm;
    ib += jb == jm;
    return jm;
  };

  f32x16_t dqT[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dqT[dt][v] = 0.f;
  // lane bases of the operand reads (offset of byte column cb = row offset ^ cb): K rows
  // (V-swizzled) and V rows (K-swizzled) t*32 + l32, transposed K reads as in the forward
  const int k_row = voff<RB>(l32, 16 * hi), v_row = KT + koff<RB>(l32, 16 * hi);
  const int k_tr = voff<RB>(4 * hi + (g16 >> 2), (mbase + 4 * (g16 & 3)) * 2);

  int f0 = 0, f1 = 0;
  int j0 = next_entry(f0);
  int j1 = j0 >= 0 ? next_entry(f1) : -1;
  if (j0 >= 0) dma(0, j0);
  for (int u = 0; j0 >= 0; ++u) {
    const int st = u & 1;
    wait_vm<0>();
    wg_barrier();
    if (j1 >= 0) dma(st ^ 1, j1);
    const int kv0 = j0 * 64;
    if (((f0 >> pr) & 1) && kv0 < a.S_valid) {
      const int so = st * 2 * KT;
      const int kr = opaque(k_row + so), vr = opaque(v_row + so), ktr = opaque(k_tr + so);
      const f32x16_t zero16 = {};
      // MFMA list: n < 4 KS: S^T = K Q^T and dP^T = V dO^T for (s, t) = (n / 4, (n / 2) % 2),
      // n even S, n odd dP (four independent accumulator chains, one row read each); then
      // 4 DT MFMAs dQ^T += K^T dS^T (the forward's P V step with K in place of V), sp = m / DT,
      // dt = m % DT, one pair of transposing reads each. Operand reads run PD MFMAs ahead
      // (across the switch to dQ, while dS is formed); scheduling fences keep the order.
      constexpr int NSD = 4 * KS, NM = NSD + 4 * DT, PD = 4;
      auto rd = [&](int n) -> bf16x8_t {
        if (n < NSD) {
          const int sm = n >> 2, t = (n >> 1) & 1;
          return *(const bf16x8_t BSA_LDS*)(lds + (((n & 1) ? vr : kr) ^ (32 * sm)) + t * 32 * RB);
        }
        const int m = n - NSD, sp = m / DT, dt = m % DT;
        const char BSA_LDS* o = lds + (ktr ^ (64 * dt)) + (32 * (sp >> 1) + 16 * (sp & 1)) * RB;
        const s16x4_t k0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)o);
        const s16x4_t k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)(o + 8 * RB));
        return join_bf16x8(k0, k1);
      };
      bf16x8_t op[NM];
#pragma unroll
      for (int n = 0; n < PD; ++n) op[n] = rd(n);
      f32x16_t sacc[2], dpacc[2];
#pragma unroll
      for (int n = 0; n < NSD; ++n) {
        __builtin_amdgcn_sched_barrier(0);
        const int sm = n >> 2, t = (n >> 1) & 1;
        if (n & 1)
          dpacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n], dop[sm], sm ? dpacc[t] : zero16, 0, 0, 0);
        else
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n], qop[sm], sm ? sacc[t] : zero16, 0, 0, 0);
        op[n + PD] = rd(n + PD);
      }
      // P^T and dS^T: rows kv = 32 t + 8 (v/4) + 4 hi + v%4, column = this lane's query
      __builtin_amdgcn_sched_barrier(0);
      float ds[2][16];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kv = t * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
          const float pv = kv0 + kv < a.S_valid ? __builtin_amdgcn_exp2f(fmaf(sacc[t][v], c2, -lse2)) : 0.f;
          ds[t][v] = pv * (dpacc[t][v] - delta);
        }
      bf16x8_t db[4];
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) db[sp] = pack8(&ds[sp >> 1][8 * (sp & 1)]);
#pragma unroll
      for (int n = NSD; n < NM; ++n) {
        __builtin_amdgcn_sched_barrier(0);
        const int m = n - NSD;
        dqT[m % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[n], db[m / DT], dqT[m % DT], 0, 0, 0);
        if (n + PD < NM) op[n + PD] = rd(n + PD);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkm0();
    int f2 = 0;
    const int j2 = j1 >= 0 ? next_entry(f2) : -1;
    j0 = j1; f0 = f1;
    j1 = j2; f1 = f2;
  }
  if (!mine_valid) return;
  // padded and gradient-free queries hold dQ = 0 already (P = 0)
  store_rows<D, F32>(a.dq, b * a.dq_sb + h * a.dq_sh + (int64_t)qtok * a.dq_ss, dqT, a.scale, hi);
}

// ---- launchers ----------------------------------------------------------------------
hipError_t launch_bwd_prep(const BwdArgs& a, float2* ld, hipStream_t st) {
  dim3 grid(a.S / 64, a.B * a.H);
  if (a.D == 64) hipLaunchKernelGGL(bwd_prep_kernel<64>, grid, dim3(256), 0, st, a, ld);
  else hipLaunchKernelGGL(bwd_prep_kernel<128>, grid, dim3(256), 0, st, a, ld);
  return hipGetLastError();
}

hipError_t launch_mask_transpose(const uint8_t* m, int64_t sb, int64_t sh, int B, int H, int nb, uint8_t* mt,
                                 hipStream_t st) {
  const int t = (nb + 63) / 64;
  hipLaunchKernelGGL(mask_transpose_kernel, dim3(t, t, B * H), dim3(256), 0, st, m, sb, sh, H, nb, mt);
  return hipGetLastError();
}

template <int D, bool F32>
static hipError_t launch_bwd_t(const BwdArgs& a, const int32_t* row_ptr, const int32_t* col_idx,
                               const int32_t* col_ptr, const int32_t* row_idx, const float2* ld, hipStream_t st) {
  const int npair = a.B * a.H * ((a.nb + 1) / 2);
  const dim3 grid((npair + BSA_NXCD - 1) / BSA_NXCD * BSA_NXCD);
  if (a.bits_k) hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32, true>), grid, dim3(512), 0, st, a, col_ptr, row_idx, ld);
  else hipLaunchKernelGGL((bwd_dkdv_kernel<D, F32, false>), grid, dim3(512), 0, st, a, col_ptr, row_idx, ld);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.bits_q) hipLaunchKernelGGL((bwd_dq_kernel<D, F32, true>), grid, dim3(256), 0, st, a, row_ptr, col_idx, ld);
  else hipLaunchKernelGGL((bwd_dq_kernel<D, F32, false>), grid, dim3(256), 0, st, a, row_ptr, col_idx, ld);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, bool f32_out, const int32_t* row_ptr, const int32_t* col_idx,
                      const int32_t* col_ptr, const int32_t* row_idx, const float2* ld, hipStream_t st) {
  if (a.D == 64)
    return f32_out ? launch_bwd_t<64, true>(a, row_ptr, col_idx, col_ptr, row_idx, ld, st)
                   : launch_bwd_t<64, false>(a, row_ptr, col_idx, col_ptr, row_idx, ld, st);
  return f32_out ? launch_bwd_t<128, true>(a, row_ptr, col_idx, col_ptr, row_idx, ld, st)
                 : launch_bwd_t<128, false>(a, row_ptr, col_idx, col_ptr, row_idx, ld, st);
}

BSA_CHECK_ACCESSOR(check_flags_bwd)

}  // namespace bsa
