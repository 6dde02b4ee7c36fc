// Host-side launchers of the library's kernels (internal interface between the
// C-ABI layer and the .hip translation units). All arguments are validated by the
// caller; every launcher returns the HIP launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// nabla.hip
// fp8 outputs of the pool kernel: codes [B,H,S,D] (byte strides) and one fp32 scale
// per (b, h, block), [B,H,nb] contiguous; index 0 for Q, 1 for K.
struct Fp8Out {
  uint8_t* codes[2];
  int64_t sb[2], sh[2], ss[2];
  float* scale[2];
  // incoherent processing: rot != 0 rotates every row to H (s . x) before the
  // quantisation (H the Sylvester Hadamard matrix, bit d of sbits set where s_d = -1)
  // and multiplies tensor x's stored scales by smul[x] (1, or 1/D on the key side)
  int rot;
  uint64_t sbits[2];
  float smul[2];
};
// Block means of q and k into qbar / kbarT; with f8, also their fp8 block quantisation
// from the same read. qbar == NULL: quantisation of q alone (f8 index 0).
hipError_t launch_pool(bool f32, int D, const void* q, const int64_t* q_strides, const void* k,
                       const int64_t* k_strides, int B, int H, int nb, double* qbar, double* kbarT,
                       const Fp8Out* f8, hipStream_t st);
// The sliding-tile rule of tile-major layouts made of whole tiles of whole blocks: block
// i lies in tile i / bpt of a row-major tile grid with GH x GW tiles per frame of tiles;
// blocks i and j are kept together when their tiles are within (rt, rh, rw) of each
// other on every axis. bpt == 0: no rule.
struct StaRule {
  int bpt, GH, GW, rt, rh, rw;
};
struct StaCoord {
  int t, h, w;   // tile coordinates of a block
};
__device__ __forceinline__ StaCoord sta_rule_coord(const StaRule& s, int i) {
  const int ti = i / s.bpt;
  return {ti / (s.GH * s.GW), (ti / s.GW) % s.GH, ti % s.GW};
}
__device__ __forceinline__ bool sta_rule_near(const StaRule& s, StaCoord a, StaCoord c) {
  return abs(a.t - c.t) <= s.rt && abs(a.h - c.h) <= s.rh && abs(a.w - c.w) <= s.rw;
}
__device__ __forceinline__ bool sta_rule_keep(const StaRule& s, int i, int j) {
  return sta_rule_near(s, sta_rule_coord(s, i), sta_rule_coord(s, j));
}
// kv lists written beside the mask rows (short rows, nb <= SELR_MAX_NB, only): row r's
// kept blocks, ascending, at kv_idx[r * nb ..], their number at kv_len[r].
struct SelLists {
  int32_t* kv_len;
  int32_t* kv_idx;
};
constexpr int SELR_MAX_NB = 256;
// near-threshold flags (flags == NULL: none): an entry's flag is 1 iff its exclusive
// fixed-point mass E satisfies t_lo <= E < t_hi; flags have mask_out's layout
struct SelNear {
  uint8_t* flags;
  uint64_t t_lo, t_hi;
};
// T_fixed = floor((1 - thr) 2^60) for the cumulative-mass rule; topk > 0 keeps the
// topk largest entries of each row instead (T_fixed unused). The result is OR'd with
// or_mask (if any) and with the sliding-tile rule sta (if sta.bpt > 0).
hipError_t launch_select(const double* qbar, const double* kbarT, int B, int H, int nb, int D, double scale,
                         uint64_t T_fixed, int topk, const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                         StaRule sta, uint8_t* mask_out, hipStream_t st, const SelLists& lists = SelLists{},
                         const SelNear& near = SelNear{});

// sta.hip
struct StaGeom {
  int T, H, W;           // latent grid
  int tt, th, tw;        // window tile
  int rt, rh, rw;        // window half-widths (window / 2)
  int order;             // 0 row-major, 1 tile-major
  int ot, oh, ow;        // tile of the tile-major order
  int S_valid, nb;
};
constexpr int STA_MAX_TILES = 64;   // distinct window tiles touched by one 64-token block
hipError_t launch_sta(const StaGeom& g, int32_t* tiles_ws, uint8_t* mask_out, hipStream_t st);
// the rule of g when its layout is aligned (tile-major, whole tiles, tiles of whole
// blocks, no padding), else {0}
StaRule sta_rule_of(const StaGeom& g);

// mask_ops.hip
hipError_t launch_mask_or(uint8_t* dst, const uint8_t* a, int64_t n, const uint8_t* b, int64_t b_n,
                          hipStream_t st);
// with pair_order: also the attention work order of these lists (pair_schedule_fits must
// hold); masks on the single-launch path get it from one extra workgroup of that launch
hipError_t launch_csr(const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int B, int H, int nb,
                      int32_t* row_ptr, int32_t* col_idx, int32_t* counts_ws, hipStream_t st,
                      int32_t* pair_order = nullptr);
// rows sorted by kept count (descending, ties by row index); workspace in int32s,
// 0 when nb is too large for the sort
size_t lpt_rows_ws_ints(int rows, int nk);
hipError_t launch_lpt_rows(const int32_t* row_ptr, int rows, int nb, int32_t* ws, int32_t* order, hipStream_t st);
// attention work order: per-XCD ranges of query-block pairs, longest first; fits for
// few items and small nb (one workgroup sorts them in shared memory)
constexpr int PAIR_SCHED_MAX_NB = 512;    // two [8][nb+1] int tables in 64 KB of shared memory
constexpr int PAIR_SCHED_MAX_ITEMS = 8192;
bool pair_schedule_fits(int BH, int nb);
int pair_schedule_slots(int BH, int nb);   // entries of the order = workgroups to launch
hipError_t launch_pair_schedule(const int32_t* row_ptr, int BH, int nb, int32_t* order, hipStream_t st);
// the same order for fixed-stride lists, from their lengths kv_len [BH * nb]
hipError_t launch_pair_schedule_len(const int32_t* kv_len, int BH, int nb, int32_t* order, hipStream_t st);

// pairing offsets of the attention's query-block pairs: for each head the d in
// [1, min(PAIR_D_MAX, nb / 2)] whose pairs (pair_blocks) have the fewest union steps, sum
// over pairs of |list(a) u list(b)|, ties to the smaller d; lists as in AttnArgs (row_len
// != NULL: fixed stride). bits: pair_bits_ws bytes of workspace, the lists' bit rows
// [rows][ceil(nb / 64)] first.
constexpr int PAIR_D_MAX = 64;
size_t pair_bits_ws(int64_t rows, int nb);
hipError_t launch_pair_offsets(const int32_t* row_ptr, const int32_t* col_idx, const int32_t* row_len,
                               int row_stride, int BH, int nb, uint64_t* bits, int32_t* pair_d, hipStream_t st);

// reorder.hip
constexpr int ORDER_ROW = 0, ORDER_TILE = 1, ORDER_SPATIAL = 2;
struct ReorderGeom {
  int T, H, W;       // latent grid
  int tt, th, tw;    // tile of ORDER_TILE
  int order;
};
// dst = src reordered (inverse: back to row-major); strides in bytes; row_bytes in {64, 128, 256, 512}
hipError_t launch_token_reorder(const void* src, const int64_t* s_strides_bytes, void* dst,
                                const int64_t* d_strides_bytes, int B, int H, int S, int row_bytes,
                                const ReorderGeom& g, bool inverse, hipStream_t st);

// checked build: each translation unit's flag word (CHK_* bits of common.h), read and
// optionally cleared; synchronous; 0 in the production build, ~0u on a HIP error
unsigned check_flags_attn(int clear);
unsigned check_flags_mask_ops(int clear);
unsigned check_flags_bwd(int clear);

// attn.hip
struct AttnArgs {
  const void* q; int64_t q_sb, q_sh, q_ss;
  const void* k; int64_t k_sb, k_sh, k_ss;
  const void* v; int64_t v_sb, v_sh, v_ss;
  // split copies (f32 inputs: hi parts in q/k/v above, lo parts here; contiguous)
  const void* q_lo; const void* k_lo; const void* v_lo;
  void* o; int64_t o_sb, o_sh, o_ss;
  float* lse;
  const int32_t* row_ptr; const int32_t* col_idx;
  // fixed-stride lists instead (row_len != NULL): row r's list is
  // col_idx[r * row_stride .. r * row_stride + row_len[r]); row_ptr unused
  const int32_t* row_len; int row_stride;
  const int32_t* pair_order;   // work order of the (head, query-block pair) items, or NULL;
  int n_slots;                 // its length (entries -1: no item)
  int derive_order;            // no pair_order: 1 = each of the n_slots workgroups derives its
                               // item of that order from the list lengths; 2 = natural XCD
                               // ranges, longest first inside each head; 0 = natural order
  const float* q_scale; const float* k_scale;
  int B, H, nb, S, S_valid, D;
  float scale_log2;      // softmax scale * log2(e)
  // pairing offset of each head [B*H] (NULL: adjacent pairs): pair p walks the query
  // blocks pair_blocks(p, pair_d[head], nb); pair_order, when given, assumes adjacent pairs
  const int32_t* pair_d;
  // the lists as bit rows [rows][nw] (launch_pair_offsets builds them), or NULL; the
  // whole-row walk then reads them instead of the entries
  const uint64_t* row_bits; int nw;
  // kv-chunked walk (kv_chunk > 0; pair_order and derive_order unused): the work items
  // are (head, chunk c, pair), chunk c = key blocks [c kv_chunk, (c+1) kv_chunk), walked
  // chunk-major inside each head; every item leaves its rows' partial state in part_o /
  // part_ml and a combine launch merges the chunks. Workspace: chunk_ws_bytes().
  int kv_chunk, nch;     // chunk width in key blocks; chunks per row = ceil(nb / kv_chunk)
  int32_t* cofs;         // [rows][nch + 1]: position in col_idx of row r's first entry >= c kv_chunk
  float* part_o;         // [rows][nch][64][D] fp32: sum of p V over the chunk's tiles (p relative to m)
  float2* part_ml;       // [rows][nch][64]: (m, l) = running maximum (log2 units) and sum of p
};
enum AttnMode { ATTN_BF16 = 0, ATTN_SPLIT_F32 = 1, ATTN_FP8 = 2 };
// workspace bytes of the kv-chunked walk (0 when kv_chunk == 0); rows = B H nb
size_t chunk_ws_bytes(int64_t rows, int nb, int D, int kv_chunk);
// points a.cofs, a.part_o, a.part_ml into ws (chunk_ws_bytes bytes, 256-aligned)
void chunk_ws_carve(AttnArgs& a, void* ws);
// the attention launch (with kv_chunk > 0: the offsets, the chunk walk and the combine)
hipError_t launch_attn(const AttnArgs& a, AttnMode mode, hipStream_t st);
hipError_t launch_split_f32(const float* x, int64_t sb, int64_t sh, int64_t ss, int B, int H, int S, int D,
                            uint16_t* hi, uint16_t* lo, hipStream_t st);

// attn_bwd.hip (bf16 q, k, v, o, dO; dq, dk, dv bf16 or f32; strides in elements)
struct BwdArgs {
  const void* q; int64_t q_sb, q_sh, q_ss;
  const void* k; int64_t k_sb, k_sh, k_ss;
  const void* v; int64_t v_sb, v_sh, v_ss;
  const void* o; int64_t o_sb, o_sh, o_ss;
  const void* d_o; int64_t do_sb, do_sh, do_ss;
  const float* lse;      // [B, H, S] natural log, as the forward writes it
  void* dq; int64_t dq_sb, dq_sh, dq_ss;
  void* dk; int64_t dk_sb, dk_sh, dk_ss;
  void* dv; int64_t dv_sb, dv_sh, dv_ss;
  int B, H, nb, S, S_valid, D;
  float scale;           // softmax scale
  float scale_log2;      // scale * log2(e)
  int derive_order;      // 1: longest first inside each head (kv-list lengths), else natural order
  // pairing offsets of the key-block pairs (dK/dV, from the transposed lists) and of the
  // query-block pairs (dQ, from the kv lists), [B*H] each, or NULL for adjacent pairs; with
  // them the bit rows of those lists ([rows][nw]), which the walks then read
  const int32_t* pair_dk; const int32_t* pair_dq;
  const uint64_t* bits_k; const uint64_t* bits_q; int nw;
};
// (lse2, delta) per query into ld [B*H*S (+64 entries of padding read by the tile copies)]
hipError_t launch_bwd_prep(const BwdArgs& a, float2* ld, hipStream_t st);
// mt [B*H, nb, nb] contiguous = the mask transposed per head
hipError_t launch_mask_transpose(const uint8_t* m, int64_t sb, int64_t sh, int B, int H, int nb, uint8_t* mt,
                               hipStream_t st);
// dK, dV from the per-key-block query lists (col_ptr, row_idx), then dQ from the kv lists
hipError_t launch_bwd(const BwdArgs& a, bool f32_out, const int32_t* row_ptr, const int32_t* col_idx,
                      const int32_t* col_ptr, const int32_t* row_idx, const float2* ld, hipStream_t st);

}  // namespace bsa
