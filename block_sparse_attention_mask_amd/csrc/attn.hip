// Block-sparse attention forward on gfx950 (bf16 MFMA; fp32 inputs via a hi/lo bf16
// split; fp8 e4m3 Q/K with per-block scales).
//
// Method: FlashAttention (Daily Papers listing): exact attention computed tile by tile
// with an online softmax (running maximum and normaliser), extended to block-sparse
// attention by visiting only listed key blocks; FlashAttention-2: parallelise over
// query blocks, keep the work of one query block inside one wave so that no
// cross-wave communication is needed; NABLA (Pith review, "What carries the
// argument"): the binary block mask tells the operator which N x N blocks to compute.
//
// Work decomposition: one 4-wave workgroup per pair of adjacent query blocks, two
// waves (32 queries each) per block; the workgroup walks the union of the two kv
// lists. Per kv block:
//   * the 64 x D K and V tiles are copied global -> LDS with direct-to-LDS 16-byte
//     loads, each 1 KB instruction fully coalesced; 16-byte chunks are XOR-swizzled
//     inside a row so that the MFMA operand reads below are bank-conflict free;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K rows are the A operand read with
//     ds_read_b128, Q^T the B operand kept in registers for the whole block); in
//     this transposed form each lane owns the scores of ONE query (its column), so
//     the row max and the row sum need only a swap with the lane 32 apart;
//   * online softmax in fp32 with exp2 and the scale folded into one multiply;
//   * O^T += V^T P^T: P^T is the B operand straight from the S^T accumulators
//     (converted to bf16, no data movement), V^T the A operand read from the
//     row-major V tile with ds_read_b64_tr_b16 (transposing LDS read of gfx950).
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "item_order.h"
#include "lds_tile.h"

namespace bsa {

// The running maximum is only moved when a tile's maximum exceeds it by more than
// RESCALE_TAU (log2 units): the probabilities then stay below 2^TAU, far inside the
// fp32 range, and the rescale of the output accumulators is skipped on most tiles.
constexpr float RESCALE_TAU = 8.f;

// MODE: ATTN_BF16, ATTN_SPLIT_F32, ATTN_FP8.  D: 64 or 128.
//
// One workgroup of four waves per PAIR of adjacent query blocks (2p, 2p+1): waves 0-1
// take the 64 queries of block 2p (32 each), waves 2-3 those of block 2p+1. The
// workgroup walks the union of the two blocks' kv lists in ascending order; every kv
// tile is copied to LDS once and used by each block whose list holds it (adjacent
// blocks share most of their kv blocks, so most tiles serve both). A block visits
// exactly its own tiles, in the same ascending order as it would alone.
//
// Buffers: two K slots and one V slot (48 KB at D = 128 bf16), so that three
// workgroups share a CU (168 VGPRs) and a third wave per SIMD hides latency. Step u:
// each wave waits for its own part of K(u), then the barrier that opens the step (every
// wave has finished step u-1, so the V slot and the other K slot are free); V(u) and
// K(u+1) are copied next; S and the softmax of tile u run while V(u) lands; a second
// barrier makes all parts of V(u) visible before PV. K(u+1) has a whole step to land.
// Each wave issues a quarter of every tile copy.
// BITS: the union walk reads the pair's lists as bit rows (a.row_bits) instead of entries.
template <int MODE, int D, bool BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_fwd_kernel(AttnArgs a, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                     const float* __restrict__ q_scale, const float* __restrict__ k_scale) {
  constexpr int QK_ES = MODE == ATTN_FP8 ? 1 : 2;   // bytes per Q/K element
  constexpr int RBK = D * QK_ES;                    // K tile row bytes
  constexpr int RBV = D * 2;                        // V tile row bytes (bf16)
  constexpr int KT_BYTES = 64 * RBK, VT_BYTES = 64 * RBV;
  constexpr int NSPLIT = MODE == ATTN_SPLIT_F32 ? 2 : 1;
  constexpr int STAGE = NSPLIT * (KT_BYTES + VT_BYTES);
  constexpr int DT = D / 32;                        // 32-wide d tiles of the output
  constexpr int KS = MODE == ATTN_FP8 ? D / 64 : D / 16;   // k-steps of S = K Q^T
  using KOp = typename std::conditional<MODE == ATTN_FP8, i32x8_t, bf16x8_t>::type;

  // two K slots, one V slot
  __shared__ __attribute__((aligned(1024))) char smem[NSPLIT * (2 * KT_BYTES + VT_BYTES)];
  char BSA_LDS* lds = (char BSA_LDS*)smem;
  auto k_lds = [&](int st, int x) { return lds + (st * NSPLIT + x) * KT_BYTES; };
  auto v_lds = [&](int st, int x) { (void)st; return lds + 2 * NSPLIT * KT_BYTES + x * VT_BYTES; };

  const int l = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pr = wave >> 1, wv = wave & 1;        // block of the pair, query half
  const int l32 = l & 31, hi = l >> 5;

  // Work item (head, pair) of this workgroup. Workgroups are dealt to the 8 XCDs
  // round-robin; XCD x runs a contiguous range of items: neighbouring query blocks
  // share most kv tiles, and then share one L2. With a work order, workgroup x takes
  // item order[x] (or none, -1): the order puts each range longest first, and
  // workgroups start in index order as slots free up, so short items fill the tail.
  // Without one: the range of XCD x is [x*chunk, (x+1)*chunk) in natural order, or
  // derived in the kernel from the list lengths: longest first in each range (few
  // rounds), or longest first inside each head (many rounds of long rows: workgroups that
  // run together have lists of similar length, start together and move through the kv
  // blocks at the same pace, so they keep sharing tiles in L2).
  const int npair = (a.nb + 1) / 2;
  const int total = a.B * a.H * npair;
  auto list_len = [&](int r) { return a.row_len ? a.row_len[r] : row_ptr[r + 1] - row_ptr[r]; };
  int lin, cidx = 0;
  // (the in-kernel orders keep their tables in smem; where they would not fit, the
  // workgroups keep the natural order of the same ranges)
  if (a.kv_chunk) {
    // kv-chunked walk: items (head, chunk, pair) in per-XCD ranges of their natural order,
    // so that the ~96 workgroups running on one XCD take the pairs of one chunk of one head
    // and read the same few K/V tiles, which stay in that XCD's L2
    const int per_bh = a.nch * npair;
    const int64_t totc = (int64_t)a.B * a.H * per_bh;
    const int64_t chunk = (totc + BSA_NXCD - 1) / BSA_NXCD;
    const int64_t lc = (int64_t)(blockIdx.x % BSA_NXCD) * chunk + blockIdx.x / BSA_NXCD;
    if (lc >= totc) return;
    const int bh0 = (int)(lc / per_bh), rem = (int)(lc - (int64_t)bh0 * per_bh);
    cidx = rem / npair;
    lin = bh0 * npair + (rem - cidx * npair);
  } else if (a.pair_order) {
    if ((int)blockIdx.x >= a.n_slots) return;
    lin = a.pair_order[blockIdx.x];
    if (lin < 0 || lin >= total) return;   // -1 = no item; larger entries belong to another shape
  } else if (a.derive_order == 1 && kth_longest_fits(a.nb, (total + BSA_NXCD - 1) / BSA_NXCD, sizeof(smem))) {
    // the longest-first order of XCD range x % 8 (as pair_schedule_block cuts the ranges)
    const int g = blockIdx.x % BSA_NXCD, k = blockIdx.x / BSA_NXCD;
    const int lo = (int)(((int64_t)g * total + BSA_NXCD - 1) / BSA_NXCD);
    const int hi = (int)(((int64_t)(g + 1) * total + BSA_NXCD - 1) / BSA_NXCD);
    if (k >= hi - lo) return;
    lin = kth_longest_item<256>(list_len, a.nb, (int*)smem, lo, hi - lo, k, a.pair_d);
  } else if (a.derive_order == 1) {
    // the same ranges as above in natural order (a grid of n_slots workgroups)
    const int g = blockIdx.x % BSA_NXCD, k = blockIdx.x / BSA_NXCD;
    const int lo = (int)(((int64_t)g * total + BSA_NXCD - 1) / BSA_NXCD);
    const int hi = (int)(((int64_t)(g + 1) * total + BSA_NXCD - 1) / BSA_NXCD);
    if (k >= hi - lo) return;
    lin = lo + k;
  } else if (a.derive_order == 2 && a.pair_d && a.pair_d[0] > 1) {
    // Scattered lists (the heads pair blocks at an offset > 1, e.g. one frame apart in a
    // row-major video layout): neighbouring items share few kv tiles, so what counts is that
    // the heads being walked keep their K and V in the last-level cache. XCDs 2g and 2g+1
    // share range g of four and take its items alternately: four heads live at a time
    // instead of eight. (Where blocks pair adjacently, each XCD's own contiguous range keeps
    // the tiles that neighbouring items share in its L2, which matters more.)
    constexpr int NG = BSA_NXCD / 2;
    const int x = blockIdx.x % BSA_NXCD, p = blockIdx.x / BSA_NXCD, g = x >> 1;
    const int chunk = (total + NG - 1) / NG;
    lin = g * chunk + 2 * p + (x & 1);
    if (lin >= min((g + 1) * chunk, total)) return;
    if (kth_longest_fits(a.nb, npair, sizeof(smem))) {
      // longest first inside each head
      const int head0 = lin / npair * npair;
      lin = kth_longest_item<256>(list_len, a.nb, (int*)smem, head0, npair, lin - head0, a.pair_d);
    }
  } else {
    const int chunk = (total + BSA_NXCD - 1) / BSA_NXCD;
    lin = (int)(blockIdx.x % BSA_NXCD) * chunk + (int)(blockIdx.x / BSA_NXCD);
    if (lin >= total) return;
    if (a.derive_order == 2 && kth_longest_fits(a.nb, npair, sizeof(smem))) {
      // the same ranges, longest first inside each head
      const int head0 = lin / npair * npair;
      lin = kth_longest_item<256>(list_len, a.nb, (int*)smem, head0, npair, lin - head0, a.pair_d);
    }
  }
  const int bh = lin / npair, pidx = lin % npair;
  const int b = bh / a.H, h = bh % a.H;
  // the pair's two query blocks: adjacent, or at the head's pairing offset
  const int2 pb = pair_blocks(pidx, a.pair_d ? a.pair_d[bh] : 1, a.nb);
  const int iA = pb.x, iB = pb.y;
  const bool hasB = iB >= 0;
  const int rowA = bh * a.nb + iA, rowB = bh * a.nb + iB;
  int sA, eA, sB = 0, eB = 0;
  if (a.kv_chunk) {   // the part of each list inside chunk cidx
    const int32_t* co = a.cofs + (int64_t)rowA * (a.nch + 1) + cidx;
    sA = co[0];
    eA = co[1];
    if (hasB) {
      const int32_t* cb = a.cofs + (int64_t)rowB * (a.nch + 1) + cidx;
      sB = cb[0];
      eB = cb[1];
    }
    if (sA == eA && sB == eB) return;   // nothing of this pair in the chunk (uniform over the workgroup)
  } else if (a.row_len) {   // fixed-stride lists
    sA = rowA * a.row_stride;
    eA = sA + a.row_len[rowA];
    if (hasB) { sB = rowB * a.row_stride; eB = sB + a.row_len[rowB]; }
  } else {
    sA = row_ptr[rowA];
    eA = row_ptr[rowA + 1];
    if (hasB) { sB = row_ptr[rowB]; eB = row_ptr[rowB + 1]; }
  }
  if (!BSA_CHECK(sA <= eA && eA - sA <= a.nb && sB <= eB && eB - sB <= a.nb, CHK_ATTN_LEN)) {
    eA = sA;   // (checked build: a bad list is walked as empty)
    eB = sB;
  }
  const int i = pr ? iB : iA;                      // this wave's query block
  const bool mine_valid = pr == 0 || hasB;
  const int row = bh * a.nb + i;

  const char* qbase[NSPLIT];
  const char* kbase[NSPLIT];
  const char* vbase[NSPLIT];
  int64_t q_rs, k_rs, v_rs;
  if constexpr (MODE == ATTN_SPLIT_F32) {
    const int64_t off = (int64_t)bh * a.S * D * 2;
    qbase[0] = (const char*)a.q + off; qbase[1] = (const char*)a.q_lo + off;
    kbase[0] = (const char*)a.k + off; kbase[1] = (const char*)a.k_lo + off;
    vbase[0] = (const char*)a.v + off; vbase[1] = (const char*)a.v_lo + off;
    q_rs = k_rs = v_rs = D * 2;
  } else {
    qbase[0] = (const char*)a.q + (b * a.q_sb + h * a.q_sh) * QK_ES;
    kbase[0] = (const char*)a.k + (b * a.k_sb + h * a.k_sh) * QK_ES;
    vbase[0] = (const char*)a.v + (b * a.v_sb + h * a.v_sh) * 2;
    q_rs = a.q_ss * QK_ES; k_rs = a.k_ss * QK_ES; v_rs = a.v_ss * 2;
  }
  const unsigned k_rs32 = (unsigned)k_rs, v_rs32 = (unsigned)v_rs;

  // this wave's quarter of the copy of kv tile jt into stage st
  auto dma_k = [&](int st, int jt) {
#pragma unroll
    for (int x = 0; x < NSPLIT; ++x)
      load_tile_part<RBK, false, 4>(kbase[x] + (int64_t)jt * 64 * k_rs, k_rs32, (unsigned)(uintptr_t)k_lds(st, x), l, wave);
  };
  auto dma_v = [&](int jt) {
#pragma unroll
    for (int x = 0; x < NSPLIT; ++x)
      load_tile_part<RBV, true, 4>(vbase[x] + (int64_t)jt * 64 * v_rs, v_rs32, (unsigned)(uintptr_t)v_lds(0, x), l, wave);
  };
  constexpr int NK_W = NSPLIT * KT_BYTES / 1024 / 4;

  // ---- Q^T as the B operand: lane holds query 32 wv + l32 of block i
  KOp qop[NSPLIT][KS];
  {
    const int64_t qrow = (int64_t)(mine_valid ? i : iA) * 64 + wv * 32 + l32;
#pragma unroll
    for (int x = 0; x < NSPLIT; ++x)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if constexpr (MODE == ATTN_FP8) {
          const char* p = qbase[0] + qrow * q_rs + 64 * s + 32 * hi;
          i32x4_t x0 = *(const i32x4_t*)p, x1 = *(const i32x4_t*)(p + 16);
          qop[x][s] = i32x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        } else {
          qop[x][s] = *(const bf16x8_t*)(qbase[x] + qrow * q_rs + (16 * s + 8 * hi) * 2);
        }
      }
  }
  const float qsc = MODE == ATTN_FP8 && mine_valid ? q_scale[row] : 1.f;

  // ---- union walk over the two kv lists (wave-uniform scalar state). Each list is
  // fetched 64 entries at a time into one register (lane e holds entry base + e) and
  // read with readlane; the fp8 key scale of an entry comes along the same way.
  int ia = sA, ib = sB, cbA = sA, cbB = sB;
  int cacheA = 0, cacheB = 0;
  float kscA = 1.f, kscB = 1.f;
  auto fetch = [&](int base, int e, int& cache, float& ksc) {
    const int x = min(base + l, e - 1);
    cache = col_idx[x];
    if constexpr (MODE == ATTN_FP8) ksc = k_scale[bh * a.nb + cache];
  };
  // BITS: word w of a bit row holds the list's blocks 64 w .. 64 w + 63; the word being
  // walked is in scalar registers with its visited bits cleared, the next one a scalar
  // load away (no vector registers, one load per 64 key blocks)
  using CU64 = const uint64_t __attribute__((address_space(4)));
  CU64* bitsA = BITS ? (CU64*)(uintptr_t)(a.row_bits + (int64_t)rowA * a.nw) : nullptr;
  CU64* bitsB = BITS && hasB ? (CU64*)(uintptr_t)(a.row_bits + (int64_t)rowB * a.nw) : nullptr;
  uint64_t curA = 0, curB = 0;
  int wi = -1;
  if constexpr (!BITS) {
    if (sA < eA) fetch(cbA, eA, cacheA, kscA);
    if (sB < eB) fetch(cbB, eB, cacheB, kscB);
  }
  __builtin_amdgcn_s_waitcnt(0);            // Q and the first list chunks are in registers

  // next union entry: returns the kv block (or -1 when both lists are done), the use
  // flags (bit 0: block 2p, bit 1: block 2p+1) and the fp8 key scale
  auto next_entry = [&](int& flags, float& ksc) -> int {
    if constexpr (BITS) {
      while ((curA | curB) == 0) {   // the next word holding a block of either list
        if (++wi >= a.nw) { flags = 0; return -1; }
        curA = bitsA[wi];
        curB = bitsB ? bitsB[wi] : 0ull;
      }
      const int t = __builtin_ctzll(curA | curB);
      flags = (int)((curA >> t) & 1ull) | (int)(((curB >> t) & 1ull) << 1);
      curA &= ~(1ull << t);
      curB &= ~(1ull << t);
      if (!BSA_CHECK(64 * wi + t < a.nb, CHK_ATTN_ENTRY)) { flags = 0; return -1; }
      // the fp8 key scale of the entry, a scalar load used two steps later
      if constexpr (MODE == ATTN_FP8) ksc = ((const float __attribute__((address_space(4)))*)(uintptr_t)k_scale)[bh * a.nb + 64 * wi + t];
      return 64 * wi + t;
    }
    const int BIG = 0x7fffffff;
    if (ia < eA && ia - cbA == 64) { cbA += 64; fetch(cbA, eA, cacheA, kscA); __builtin_amdgcn_s_waitcnt(0); }
    if (ib < eB && ib - cbB == 64) { cbB += 64; fetch(cbB, eB, cacheB, kscB); __builtin_amdgcn_s_waitcnt(0); }
    const int ja = ia < eA ? __builtin_amdgcn_readlane(cacheA, ia - cbA) : BIG;
    const int jb = ib < eB ? __builtin_amdgcn_readlane(cacheB, ib - cbB) : BIG;
    const int j = min(ja, jb);
    if (j == BIG) { flags = 0; return -1; }
    if (!BSA_CHECK(j >= 0 && j < a.nb && max(ja, jb) >= 0, CHK_ATTN_ENTRY)) { flags = 0; return -1; }
    flags = (ja == j ? 1 : 0) | (jb == j ? 2 : 0);
    if constexpr (MODE == ATTN_FP8)
      ksc = __int_as_float(ja == j ? __builtin_amdgcn_readlane(__float_as_int(kscA), ia - cbA)
                                   : __builtin_amdgcn_readlane(__float_as_int(kscB), ib - cbB));
    ia += ja == j;
    ib += jb == j;
    return j;
  };

  f32x16_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int g16 = l & 15, mbase = 16 * ((l >> 4) & 1);
  // lane bases of the operand reads (bf16 K rows 32 kt + l32, chunk 2 s + hi: base ^ 32 s;
  // V^T rows 32 (sp >> 1) + 16 (sp & 1) + {0, 8} + 4 hi + g16 / 4, d tile dt: base ^ 64 dt)
  const int k_lane = koff_lane<RBK>(l32, hi);
  const int v_lane = voff<RBV>(4 * hi + (g16 >> 2), (mbase + 4 * (g16 & 3)) * 2);

  // two-entry look-ahead ring: (j, flags, scale) of steps u and u+1
  int f0 = 0, f1 = 0;
  float s0 = 1.f, s1 = 1.f;
  int j0 = next_entry(f0, s0);
  int j1 = j0 >= 0 ? next_entry(f1, s1) : -1;
  if (j0 >= 0) dma_k(0, j0);

  for (int u = 0; j0 >= 0; ++u) {
    const int st = u & 1;
    wait_vm<0>();                                        // own share of K(u) landed
    wg_barrier();                                        // everybody's share; step u-1 done everywhere
    dma_v(j0);                                           // V(u) into the V slot (read by step u-1)
    if (j1 >= 0) dma_k(st ^ 1, j1);                      // K(u+1) into the K slot step u-1 used

    const int kv0 = j0 * 64;
    const bool use = ((f0 >> pr) & 1) && kv0 < a.S_valid;
    f32x16_t sacc[2];
    bf16x8_t pop[4];
    if (use) {
      const int ka = opaque(k_lane + st * NSPLIT * KT_BYTES);   // offset of this step's K slot
      // ---- S^T = K Q^T for this wave's 32 queries: sacc[kt], kv = kt*32 + 8(v/4) + 4 hi + v%4
      const f32x16_t zero16 = {};
      if constexpr (MODE == ATTN_BF16) {
        // MFMA m = (s, kt) = (m / 2, m % 2): the two accumulator chains alternate and the
        // operand reads run PD MFMAs ahead. Scheduling fences keep this order; left alone,
        // the compiler runs the chains one after the other and reads each operand right
        // before its MFMA.
        constexpr int NM = 2 * KS, PD = BITS ? 5 : 6;
        auto kread = [&](int m) {
          return *(const bf16x8_t BSA_LDS*)(lds + (ka ^ (32 * (m >> 1))) + (m & 1) * 32 * RBK);
        };
        bf16x8_t kq[NM];
#pragma unroll
        for (int m = 0; m < PD; ++m) kq[m] = kread(m);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          __builtin_amdgcn_sched_barrier(0);
          const int sm = m >> 1, kt = m & 1;
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[m], qop[0][sm], sm ? sacc[kt] : zero16, 0, 0, 0);
          if (m + PD < NM) kq[m + PD] = kread(m + PD);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // fp8 and the f32 split: all K operands of the tile, then the MFMAs
        char BSA_LDS* kt0 = k_lds(st, 0);
        KOp kk[2][KS];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            if constexpr (MODE == ATTN_FP8) {
              const int r = kt * 32 + l32, cb = 64 * s + 32 * hi;
              i32x4_t x0 = *(const i32x4_t BSA_LDS*)(kt0 + koff<RBK>(r, cb));
              i32x4_t x1 = *(const i32x4_t BSA_LDS*)(kt0 + koff<RBK>(r, cb + 16));
              kk[kt][s] = i32x8_t{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            } else {
              kk[kt][s] = *(const bf16x8_t BSA_LDS*)(lds + (ka ^ (32 * s)) + kt * 32 * RBK);
            }
          }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            if constexpr (MODE == ATTN_FP8) {
              sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kk[kt][s], qop[0][s], s ? sacc[kt] : zero16, 0,
                                                                         0, 0, 127, 0, 127);
            } else {
              const bf16x8_t k1 = *(const bf16x8_t BSA_LDS*)(lds + KT_BYTES + (ka ^ (32 * s)) + kt * 32 * RBK);
              sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[kt][s], qop[0][s], s ? sacc[kt] : zero16, 0, 0, 0);
              sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[kt][s], qop[1][s], sacc[kt], 0, 0, 0);
              sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qop[0][s], sacc[kt], 0, 0, 0);
            }
          }
      }
      // ---- mask padded keys of the last block
      if (kv0 + 64 > a.S_valid) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kv = kt * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
            if (kv0 + kv >= a.S_valid) sacc[kt][v] = -INFINITY;
          }
      }
      // ---- online softmax (log2 domain, lazily rescaled)
      const float c = a.scale_log2 * qsc * s0;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kt][v]);
      mx = fmaxf(mx, partner(mx)) * c;
      if (__ballot(mx > m_run + RESCALE_TAU)) {
        const float mnew = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
        m_run = mnew;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
      }
      // The normaliser sums the probabilities as rounded to bf16 for the PV product, so
      // that O is an exact convex combination of those weights: the rounding then moves
      // O by 2^-8 sum_k w_k |V_k - O| at most (bf16's unit roundoff: 8 significant bits),
      // instead of 2^-8 |O|.
      const float mr = m_run;
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        i32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 8 * (sp & 1) + 2 * e;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[sp >> 1][v], c, -mr));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[sp >> 1][v + 1], c, -mr));
          const unsigned pk = pk_bf16(p0, p1);
          w[e] = (int)pk;
          if (e & 1) ls1 = add_bf16_pair(pk, ls1);
          else ls0 = add_bf16_pair(pk, ls0);
        }
        pop[sp] = __builtin_bit_cast(bf16x8_t, w);
      }
      l_run += ls0 + ls1;
    }
    if (j1 >= 0) wait_vm<NK_W>(); else wait_vm<0>();    // own share of V(u) landed
    wg_barrier();                                        // everybody's share
    if (use) {
      // ---- O^T += V^T P^T, V^T read from the row-major V tile with transposing reads
      const int va = opaque(v_lane);
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        const int rofs = (32 * (sp >> 1) + 16 * (sp & 1)) * RBV;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int x = 0; x < NSPLIT; ++x) {
            char BSA_LDS* vt = v_lds(st, x) + (va ^ (64 * dt)) + rofs;
            s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)vt);
            s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t BSA_LDS*)(vt + 8 * RBV));
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x8(v0, v1), pop[sp], oacc[dt], 0, 0, 0);
          }
        }
      }
      if constexpr (MODE != ATTN_SPLIT_F32) pipeline_reads<4 * DT, 2, 4>();
    }
    wait_lgkm0();                                        // reads of this step's slots done before the next barrier
    int f2 = 0;
    float s2 = 1.f;
    const int j2 = j1 >= 0 ? next_entry(f2, s2) : -1;
    j0 = j1; f0 = f1; s0 = s1;
    j1 = j2; f1 = f2; s1 = s2;
  }

  // ---- epilogue: O = O^T / l, written row-major; padded rows and empty rows are 0
  if (!mine_valid) return;
  const float lt = l_run + partner(l_run);
  if (a.kv_chunk) {
    // the chunk's partial state of this block's rows, unnormalised; a block with nothing
    // in the chunk writes nothing (the combine skips the chunk from the same offsets)
    if (pr ? eB == sB : eA == sA) return;
    const int64_t slot = ((int64_t)row * a.nch + cidx) * 64 + wv * 32 + l32;
    if (hi == 0) a.part_ml[slot] = float2{m_run, lt};
    float* po = a.part_o + slot * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4_t*)(po + 32 * dt + 8 * g + 4 * hi) =
            f32x4_t{oacc[dt][4 * g], oacc[dt][4 * g + 1], oacc[dt][4 * g + 2], oacc[dt][4 * g + 3]};
    return;
  }
  const int q = i * 64 + wv * 32 + l32;
  const bool live = q < a.S_valid && lt > 0.f;
  const float inv = live ? 1.f / lt : 0.f;
  if (a.lse && hi == 0)
    a.lse[(int64_t)bh * a.S + q] = live ? (m_run + log2f(lt)) * 0.69314718055994530942f : -INFINITY;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * hi;
      if constexpr (MODE == ATTN_SPLIT_F32) {
        float* o = (float*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)q * a.o_ss + d;
        *(f32x4_t*)o = f32x4_t{oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv, oacc[dt][4 * g + 2] * inv,
                               oacc[dt][4 * g + 3] * inv};
      } else {
        u16* o = (u16*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)q * a.o_ss + d;
        uint2 w;
        w.x = pk_bf16(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv);
        w.y = pk_bf16(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        *(uint2*)o = w;
      }
    }
}

// f32 -> (hi, lo) bf16 split, written contiguous [B,H,S,D]
__global__ __launch_bounds__(256) void split_f32_kernel(const float* __restrict__ x, int64_t sb, int64_t sh,
                                                        int64_t ss, int H, int S, int D, u16* __restrict__ hi,
                                                        u16* __restrict__ lo, int64_t total) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int d = (int)(e % D);
    const int64_t s = (e / D) % S;
    const int64_t bh = e / ((int64_t)D * S);
    const float v = x[(bh / H) * sb + (bh % H) * sh + s * ss + d];
    const u16 hb = f32_to_bf16_bits(v);
    hi[e] = hb;
    lo[e] = f32_to_bf16_bits(v - bf16_bits_to_f32(hb));
  }
}

hipError_t launch_split_f32(const float* x, int64_t sb, int64_t sh, int64_t ss, int B, int H, int S, int D,
                            uint16_t* hi, uint16_t* lo, hipStream_t st) {
  const int64_t total = (int64_t)B * H * S * D;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(split_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, sb, sh, ss, H, S, D, hi, lo,
                     total);
  return hipGetLastError();
}

// ---- kv-chunked walk: chunk offsets and the combine
//
// Each chunk's partial state of a query is (m, l, u): m the running maximum of its scores
// (log2 units), l the sum of its probabilities 2^(s - m) and u the sum of those
// probabilities times the value rows. Online softmax is associative (FlashAttention,
// Daily Papers listing; the split reduction of LeanAttention, same listing): with
// M = max m_c, the whole row has l = sum_c l_c 2^(m_c - M), O = sum_c u_c 2^(m_c - M) / l
// and lse = (M + log2 l) ln 2, whatever the split.

// cofs[r][c] = position of row r's first list entry >= c W (c = 0 .. nch); lists ascending
__global__ __launch_bounds__(256) void chunk_offsets_kernel(const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col_idx,
                                                            const int32_t* __restrict__ row_len, int row_stride,
                                                            int64_t rows, int nch, int W, int32_t* __restrict__ cofs) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (nch + 1)) return;
  const int64_t r = t / (nch + 1);
  const int c = (int)(t - r * (nch + 1));
  int lo, hi;
  if (row_len) {
    lo = (int)(r * row_stride);
    hi = lo + row_len[r];
  } else {
    lo = row_ptr[r];
    hi = row_ptr[r + 1];
  }
  if (c < nch) {
    const int target = c * W;
    while (lo < hi) {   // first entry >= target
      const int mid = (lo + hi) >> 1;
      if (col_idx[mid] < target) lo = mid + 1;
      else hi = mid;
    }
  } else {
    lo = hi;
  }
  cofs[t] = lo;
}

// One workgroup per query block: thread t merges query t / 4, a quarter of its D columns,
// over the block's chunks in ascending order (a fixed order: the result does not depend
// on scheduling). Padded queries and queries with nothing kept get O = 0, lse = -inf.
template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int DQ = D / 4;   // columns per thread
  const int64_t row = blockIdx.x;
  const int bh = (int)(row / a.nb), blk = (int)(row - (int64_t)bh * a.nb);
  const int b = bh / a.H, h = bh % a.H;
  const int ql = threadIdx.x >> 2, d0 = (threadIdx.x & 3) * DQ;
  const int q = blk * 64 + ql;
  const int32_t* co = a.cofs + row * (a.nch + 1);
  f32x4_t acc[DQ / 4];
#pragma unroll
  for (int x = 0; x < DQ / 4; ++x) acc[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, L = 0.f;
  int prev = co[0];
  for (int c = 0; c < a.nch; ++c) {
    const int next = co[c + 1];
    if (next == prev) continue;   // nothing of this row in chunk c: no partial state written
    prev = next;
    const int64_t slot = (row * a.nch + c) * 64 + ql;
    const float2 ml = a.part_ml[slot];
    if (!(ml.y > 0.f)) continue;  // only padded keys in the chunk
    const f32x4_t* u = (const f32x4_t*)(a.part_o + slot * D + d0);
    float wc;
    if (ml.x > M) {
      const float r = __builtin_amdgcn_exp2f(M - ml.x);   // 0 on the first chunk (M = -inf)
#pragma unroll
      for (int x = 0; x < DQ / 4; ++x) acc[x] *= r;
      L *= r;
      M = ml.x;
      wc = 1.f;
    } else {
      wc = __builtin_amdgcn_exp2f(ml.x - M);
    }
    L += ml.y * wc;
#pragma unroll
    for (int x = 0; x < DQ / 4; ++x) acc[x] += u[x] * wc;
  }
  const bool live = q < a.S_valid && L > 0.f;
  const float inv = live ? 1.f / L : 0.f;
  if (a.lse && (threadIdx.x & 3) == 0)
    a.lse[(int64_t)bh * a.S + q] = live ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
  if constexpr (F32OUT) {
    float* o = (float*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)q * a.o_ss + d0;
#pragma unroll
    for (int x = 0; x < DQ / 4; ++x) *(f32x4_t*)(o + 4 * x) = acc[x] * inv;
  } else {
    u16* o = (u16*)a.o + b * a.o_sb + h * a.o_sh + (int64_t)q * a.o_ss + d0;
#pragma unroll
    for (int x = 0; x < DQ / 4; ++x) {
      uint2 w;
      w.x = pk_bf16(acc[x][0] * inv, acc[x][1] * inv);
      w.y = pk_bf16(acc[x][2] * inv, acc[x][3] * inv);
      *(uint2*)(o + 4 * x) = w;
    }
  }
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t chunk_ws_bytes(int64_t rows, int nb, int D, int kv_chunk) {
  if (kv_chunk <= 0) return 0;
  const size_t nch = (size_t)((nb + kv_chunk - 1) / kv_chunk);
  return al256((size_t)rows * (nch + 1) * 4) + al256((size_t)rows * nch * 64 * 8) +
         al256((size_t)rows * nch * 64 * D * 4);
}
void chunk_ws_carve(AttnArgs& a, void* ws) {
  const int64_t rows = (int64_t)a.B * a.H * a.nb;
  a.nch = (a.nb + a.kv_chunk - 1) / a.kv_chunk;
  char* w = (char*)ws;
  a.cofs = (int32_t*)w;
  w += al256((size_t)rows * (a.nch + 1) * 4);
  a.part_ml = (float2*)w;
  w += al256((size_t)rows * a.nch * 64 * 8);
  a.part_o = (float*)w;
}

template <int MODE, int D>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
  if (a.kv_chunk) {
    const int64_t rows = (int64_t)a.B * a.H * a.nb;
    const int64_t nofs = rows * (a.nch + 1);
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3((unsigned)((nofs + 255) / 256)), dim3(256), 0, st, a.row_ptr,
                       a.col_idx, a.row_len, a.row_stride, rows, a.nch, a.kv_chunk, a.cofs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = rows / a.nb * a.nch * ((a.nb + 1) / 2);
    const int64_t grid = (items + BSA_NXCD - 1) / BSA_NXCD * BSA_NXCD;
    hipLaunchKernelGGL((attn_fwd_kernel<MODE, D, false>), dim3((unsigned)grid), dim3(256), 0, st, a, a.row_ptr,
                       a.col_idx, a.q_scale, a.k_scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((attn_combine_kernel<D, MODE == ATTN_SPLIT_F32>), dim3((unsigned)rows), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int total = a.B * a.H * ((a.nb + 1) / 2);
  dim3 grid(a.pair_order || a.derive_order == 1 ? a.n_slots : ((total + BSA_NXCD - 1) / BSA_NXCD) * BSA_NXCD);
  {
    if (a.row_bits) {
      hipLaunchKernelGGL((attn_fwd_kernel<MODE, D, true>), grid, dim3(256), 0, st, a, a.row_ptr, a.col_idx, a.q_scale,
                         a.k_scale);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_fwd_kernel<MODE, D, false>), grid, dim3(256), 0, st, a, a.row_ptr, a.col_idx, a.q_scale,
                     a.k_scale);
  return hipGetLastError();
}

BSA_CHECK_ACCESSOR(check_flags_attn)

hipError_t launch_attn(const AttnArgs& a, AttnMode mode, hipStream_t st) {
  if (a.D == 64) {
    switch (mode) {
      case ATTN_BF16: return launch_attn_t<ATTN_BF16, 64>(a, st);
      case ATTN_SPLIT_F32: return launch_attn_t<ATTN_SPLIT_F32, 64>(a, st);
      case ATTN_FP8: return launch_attn_t<ATTN_FP8, 64>(a, st);
    }
  } else {
    switch (mode) {
      case ATTN_BF16: return launch_attn_t<ATTN_BF16, 128>(a, st);
      case ATTN_SPLIT_F32: return launch_attn_t<ATTN_SPLIT_F32, 128>(a, st);
      case ATTN_FP8: return launch_attn_t<ATTN_FP8, 128>(a, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace bsa
