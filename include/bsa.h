/*
 * bsa.h - block-sparse attention with adaptive (NABLA) and sliding-tile (STA)
 * block masks, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages:
 *   [NABLA]  Pith review of "NABLA: Neighborhood Adaptive Block-Level Attention"
 *            (arXiv 2507.13546), sections "What carries the argument", "Core claim"
 *            and the referee report (minor comment 2 on Algorithm 1);
 *   [STA]    blog review "Fast Video Generation with SLIDING TILE ATTENTION",
 *            section "Observation & Proposed Method", and the STA abstract in the
 *            Daily Papers listing;
 *   [FA]     FlashAttention / FlashAttention-2 / FlashAttention-3 abstracts in the
 *            Daily Papers listing (exact tiled attention, block-sparse extension,
 *            online softmax);
 *   [CalibAtt] the CalibAtt page (per-block skip lists handed to the kernel).
 *
 * Conventions shared by every call
 *   - Tensors Q, K, V, O are [B, H, S, D] with D contiguous; the strides sb, sh, ss
 *     of bsa_tensor are in ELEMENTS. S is a multiple of the block size N = 64;
 *     tokens at positions >= S_valid are padding.
 *   - Block masks are uint8 (0 = skip, nonzero = keep) [B, H, nb, nb] with
 *     nb = S / 64, rows contiguous (row stride nb bytes); the per-(b,h) plane
 *     strides are given in BYTES (0 broadcasts one plane to every head).
 *   - Every pointer is a device pointer unless stated otherwise. The caller owns
 *     all memory; the library never allocates, frees or synchronises.
 *   - Every call validates its arguments on the host first and returns a status
 *     without launching anything if they are invalid (bsa_last_error() then holds
 *     a message for the calling thread). Work is enqueued on `stream` and runs
 *     asynchronously; device faults surface at the caller's next synchronisation.
 *     On an error the contents of the outputs are undefined.
 *   - Calls are stateless and may be issued from several threads at once.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* bsa_stream_t;   /* same type as hipStream_t; NULL = default stream */

typedef enum {
  BSA_OK = 0,
  BSA_EINVAL = 1,         /* invalid argument (shape, stride, alignment, value)      */
  BSA_EUNSUPPORTED = 2,   /* valid but not implemented (e.g. head_dim not 64/128)    */
  BSA_EWORKSPACE = 3,     /* workspace missing or smaller than the *_workspace_size  */
  BSA_EHIP = 4            /* a HIP launch failed; the message names the HIP error    */
} bsa_status;

typedef enum {
  BSA_F32 = 0,
  BSA_BF16 = 1,
  BSA_FP8_E4M3FN = 2      /* OCP fp8 e4m3 (max 448), one scale per 64-token block    */
} bsa_dtype;

/* A [B, H, S, D] tensor: element (b,h,s,d) lives at ptr + b*sb + h*sh + s*ss + d. */
typedef struct {
  const void* ptr;
  bsa_dtype dtype;
  int64_t sb, sh, ss;
} bsa_tensor;

/* B batch, H heads, S padded sequence (multiple of N), S_valid real tokens
 * (1 <= S_valid <= S), D head dim, N block size (must be 64). */
typedef struct {
  int B, H, S, S_valid, D, N;
} bsa_shape;

/* ---------------------------------------------------------------------------
 * Adaptive block mask [NABLA, "What carries the argument"; "Core claim"].
 *
 * For every (b, h): Qbar, Kbar = means of Q, K over each block of N tokens
 * (padding rows included as zeros); L = scale * Qbar Kbar^T ((S/N) x (S/N));
 * P = softmax of each row of L; in each row, visit the entries by descending P
 * (ties: ascending key-block index) and keep an entry iff the mass of the entries
 * visited before it is < 1 - thr, i.e. keep the smallest prefix whose cumulative
 * mass reaches 1 - thr; write the result in the original column order
 * (referee report, minor comment 2: sort and cumsum along the key-block axis,
 * then reorder). The top entry of a row is always kept.
 *
 *   q, k       bf16 or f32 [B,H,S,D] (the same dtype), D in {64, 128}
 *   thr        0 <= thr < 1
 *   scale      softmax temperature of the reduced map; <= 0 selects 1/sqrt(D)
 *   or_mask    optional (NULL = none) uint8 mask OR'd into the result, e.g. a
 *              sliding-tile mask [NABLA: the adaptive mask may be OR'd with STA];
 *              plane strides or_sb, or_sh in bytes (0, 0 = one shared plane)
 *   mask_out   uint8 [B,H,nb,nb], contiguous; written with 0/1
 *   near_thr_out  optional (NULL = none) uint8 [B,H,nb,nb], contiguous, distinct
 *              from mask_out: 1 where the block's exclusive cumulative mass E (the
 *              mass of the entries visited before it) lies within 1e-6 of the
 *              threshold, |E - (1 - thr)| <= 1e-6, else 0 [NABLA, "Core claim": the
 *              prefix reaching 1 - thr; blocks this close to it are the ones an fp64
 *              evaluation in another summation order may decide either way]. The
 *              flag describes the adaptive rule only (an OR'd mask does not change
 *              it). Asking for the flags runs the selection for the two band edges
 *              as well, which costs time; the mask is the same either way.
 *   ws         device workspace of at least nabla_workspace_size(shape) bytes,
 *              256-byte aligned; its contents on entry do not matter
 * The reduced map, softmax and cumulative mass are evaluated in fp64 (the
 * cumulative mass in 2^-60 fixed point, E 2^60 compared with floor((1 - thr) 2^60)
 * and, for the flags, with floor((1 - thr -+ 1e-6) 2^60)), so a block whose
 * exclusive cumulative mass lies within ~1e-12 of 1 - thr (of a band edge) may be
 * decided (flagged) differently from an exact-arithmetic evaluation; all others
 * are decided exactly.
 * ------------------------------------------------------------------------- */
size_t nabla_workspace_size(const bsa_shape* shape);
bsa_status nabla_build_mask(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape,
                            double thr, double scale,
                            const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                            uint8_t* mask_out, uint8_t* near_thr_out,
                            void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * nabla_build_mask for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments, results and errors as nabla_build_mask, without ws / ws_bytes. The
 * workspace is a static device array of BSA_NOALLOC_SCRATCH_BYTES (128 MiB) inside the
 * library, one per GPU the library runs on, held until the process ends; the call
 * allocates and frees nothing. Shapes with nabla_workspace_size(shape) above that
 * (2 B H ceil(S/1024)*16 D 8 bytes: the 40-head 14B 720p shape needs 97 MB) return
 * BSA_EUNSUPPORTED before any launch. Every call on one GPU uses the same array, which
 * keeps the last call's contents (nothing in it needs to start at zero): calls that
 * overlap in time on one GPU race, so the caller must order them (one stream, or
 * events between streams). The array's device address is looked up on the first call
 * on each device.
 * ------------------------------------------------------------------------- */
#define BSA_NOALLOC_SCRATCH_BYTES (128u << 20)
bsa_status nabla_build_mask_noalloc(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape,
                                    double thr, double scale,
                                    const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                                    uint8_t* mask_out, uint8_t* near_thr_out, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Top-k block selection [NABLA review, Appendix C / Theorem 1: the fixed-count
 * alternative that CDF thresholding is compared with at equal retained blocks].
 * The same reduced map and row softmax as nabla_build_mask; each row keeps its topk
 * largest entries in the same descending order (equal probabilities by ascending
 * block index, entries closer than 2^-60 counting as equal), then the optional OR.
 * Rows with nb <= topk keep every block. topk >= 1 (else BSA_EINVAL); other
 * arguments, workspace and errors as for nabla_build_mask.
 * ------------------------------------------------------------------------- */
bsa_status nabla_build_mask_topk(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape,
                                 int topk, double scale,
                                 const uint8_t* or_mask, int64_t or_sb, int64_t or_sh,
                                 uint8_t* mask_out, void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * fp8 e4m3fn block quantisation of Q and K [FA3: block quantisation for FP8
 * attention; the combined-sweep workload: fp8 e4m3 Q/K with one scale per block].
 * Per (b, h, 64-token block): scale = amax / 448 over its 64 x D values, computed in
 * fp32 (1 for an all-zero block); code = e4m3fn(x / scale) with the quotient in fp32,
 * round to nearest even, saturating at +-448 (OCP e4m3fn: bias 7, 3 mantissa bits,
 * no infinities). The value of code c of block j is fp8(c) * scale[b,h,j], which is
 * what block_sparse_attn_fwd takes as q_scale / k_scale.
 *
 * quantize_fp8_blocks: x bf16 or f32 [B,H,S,D] -> codes (dtype BSA_FP8_E4M3FN,
 *   [B,H,S,D], own strides) and scales float [B,H,nb] contiguous. All S rows are
 *   quantised (zero padding gives code 0).
 * nabla_build_mask_fp8: nabla_build_mask (with its optional near_thr_out) plus the
 *   quantisation of q and k from the same read (q8, q_scale, k8, k_scale as codes,
 *   scales above); same workspace.
 * Errors as for nabla_build_mask; BSA_EINVAL for a codes tensor of another dtype or
 * misaligned scales.
 * ------------------------------------------------------------------------- */
bsa_status quantize_fp8_blocks(const bsa_tensor* x, const bsa_shape* shape, const bsa_tensor* codes,
                               float* scales, bsa_stream_t stream);
bsa_status nabla_build_mask_fp8(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape,
                                double thr, double scale,
                                const uint8_t* or_mask, int64_t or_sb, int64_t or_sh, uint8_t* mask_out,
                                uint8_t* near_thr_out,
                                const bsa_tensor* q8, float* q_scale, const bsa_tensor* k8, float* k_scale,
                                void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Incoherent processing before the fp8 block quantisation [FA3 abstract: named
 * beside block quantisation as the means of lowering the fp8 error; the pages give no
 * formula, so this is a reading]. Q and K are both multiplied by the orthogonal matrix
 * M = diag(s) H / sqrt(D), H the D x D Sylvester Hadamard matrix and s a vector of
 * random signs the caller draws: Q M (K M)^T = Q K^T, while a few large channels are
 * spread over all D of them, so the block amax (and the quantisation step) shrinks.
 * Each row x is rotated to y = H (s . x), computed in fp32 by the fast Walsh-Hadamard
 * transform, butterflies (a, b) -> (a + b, a - b) at strides 1, 2, ..., D/2 in that
 * order; y is then quantised exactly as by quantize_fp8_blocks (amax, scale, codes of
 * y). The 1/D of M M^T is carried by the KEY side's stored scales (scale / D, exact:
 * D is a power of two), so block_sparse_attn_fwd on the codes with q_scale, k_scale
 * computes the attention of the unrotated Q and K. V is not rotated.
 *
 * sign_bits: HOST array of D/64 words (one for D = 64, two for D = 128); bit (d % 64)
 *   of word d / 64 is set where s_d = -1. Read during the call; not retained.
 * quantize_fp8_blocks_rotated: one tensor; key_side = 0 (query side, scales as
 *   computed) or 1 (key side, scales / D). Otherwise as quantize_fp8_blocks.
 * nabla_build_mask_fp8_rotated: as nabla_build_mask_fp8 (the mask is that of the
 *   unrotated q, k), with q's codes rotated on the query side and k's on the key side.
 * Errors: BSA_EINVAL for sign_bits == NULL or key_side not 0/1; otherwise as the
 * unrotated calls.
 * ------------------------------------------------------------------------- */
bsa_status quantize_fp8_blocks_rotated(const bsa_tensor* x, const bsa_shape* shape, const uint64_t* sign_bits,
                                       int key_side, const bsa_tensor* codes, float* scales, bsa_stream_t stream);
bsa_status nabla_build_mask_fp8_rotated(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape,
                                        double thr, double scale,
                                        const uint8_t* or_mask, int64_t or_sb, int64_t or_sh, uint8_t* mask_out,
                                        uint8_t* near_thr_out, const uint64_t* sign_bits,
                                        const bsa_tensor* q8, float* q_scale, const bsa_tensor* k8,
                                        float* k_scale, void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Static sliding-tile block mask [STA, "Observation & Proposed Method"].
 *
 * The T x H x W latent grid (T*H*W == shape->S_valid) is cut into tiles of
 * tile_thw tokens (smaller tiles at the far borders if they do not divide).
 * A query tile a sees key tile c iff |a - c| <= win_thw / 2 on every axis
 * (odd window sizes, centred, cut off at the grid border, not shifted).
 * Sequence position p holds grid cell token_order(p): order 0 = row-major (t,h,w);
 * order 1 = tile-major with tiles of order_tile_thw tokens visited row-major and
 * tokens row-major inside each tile. Block pair (i, j) is kept iff some real
 * token of block i may see some real token of block j (whole blocks are computed).
 *
 *   grid_thw, tile_thw, win_thw, order_tile_thw   host arrays of 3 ints
 *                  (order_tile_thw may be NULL for order 0)
 *   mask_out       uint8 [nb, nb] (one plane shared by all heads), contiguous
 *   ws             workspace of at least sta_workspace_size(shape) bytes
 * ------------------------------------------------------------------------- */
size_t sta_workspace_size(const bsa_shape* shape);
bsa_status sta_build_mask(const bsa_shape* shape, const int grid_thw[3], const int tile_thw[3],
                          const int win_thw[3], int token_order, const int order_tile_thw[3],
                          uint8_t* mask_out, void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * NABLA mask OR'd with the sliding-tile mask in one call [NABLA: the adaptive mask
 * combined with STA]. The result equals nabla_build_mask with or_mask = the
 * sta_build_mask plane of (grid_thw, tile_thw, win_thw, token_order, order_tile_thw) for
 * every head. For tile-major layouts of whole tiles made of whole blocks (no padding)
 * the sliding-tile rule is evaluated inside the selection and no plane is built;
 * otherwise the plane is built in the workspace first.
 *   q, k, shape, thr, scale, mask_out, near_thr_out   as nabla_build_mask (the flags
 *              describe the adaptive rule, before the sliding tiles are OR'd in)
 *   grid_thw .. order_tile_thw          as sta_build_mask (T*H*W must equal S_valid)
 *   ws         at least nabla_sta_workspace_size(shape) bytes, 256-byte aligned
 * Errors as the two calls; every check precedes any launch.
 * ------------------------------------------------------------------------- */
size_t nabla_sta_workspace_size(const bsa_shape* shape);
bsa_status nabla_build_mask_sta(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                                double scale, const int grid_thw[3], const int tile_thw[3], const int win_thw[3],
                                int token_order, const int order_tile_thw[3], uint8_t* mask_out,
                                uint8_t* near_thr_out, void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * The mask of nabla_build_mask_sta (or of nabla_build_mask with no or_mask, when
 * grid_thw is NULL) together with its per-query-block kv lists and, optionally, the
 * attention work order [NABLA: the binary block mask tells the operator which blocks
 * to compute; CalibAtt skip lists]. The lists come out of the same launch that writes
 * the mask rows: there is no separate pass over the mask.
 *   q .. near_thr_out  as nabla_build_mask_sta; grid_thw NULL: no sliding tiles
 *                  (tile_thw, win_thw, token_order, order_tile_thw unused)
 *   kv_len     int32 [B*H*nb]: the number of kept kv blocks of row r = (b*H + h)*nb + i
 *   kv_idx     int32 [B*H*nb*nb]: row r's kept kv blocks, ascending, at
 *              kv_idx[r*nb .. r*nb + kv_len[r]); the rest of the row is not written
 *   work_order optional (NULL = none) int32 [attn_work_order_slots(shape)]: the
 *              attention work order of these lists, as attn_work_order writes it (one
 *              more small launch, from kv_len); when attn_work_order_slots(shape) is 0
 *              a non-NULL work_order is BSA_EUNSUPPORTED
 *   ws         at least nabla_lists_workspace_size(shape) bytes, 256-byte aligned;
 *              calls that share a workspace must not overlap in time
 * nb must be at most 256 (BSA_EUNSUPPORTED otherwise: build the mask, then call
 * bsa_mask_to_csr), and B*H*nb*nb below 2^31. Errors as nabla_build_mask_sta.
 * ------------------------------------------------------------------------- */
size_t nabla_lists_workspace_size(const bsa_shape* shape);
bsa_status nabla_build_mask_lists(const bsa_tensor* q, const bsa_tensor* k, const bsa_shape* shape, double thr,
                                  double scale, const int grid_thw[3], const int tile_thw[3], const int win_thw[3],
                                  int token_order, const int order_tile_thw[3], uint8_t* mask_out,
                                  uint8_t* near_thr_out, int32_t* kv_len, int32_t* kv_idx, int32_t* work_order,
                                  void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Union of block masks [NABLA: adaptive mask OR sliding-tile mask].
 *   dst[i] = (a[i] | b[i % b_n]) != 0 for 0 <= i < n; b_n divides n (b_n == n is a
 *   plain elementwise OR; b_n == nb*nb broadcasts one plane over every head).
 *   dst may alias a.
 * ------------------------------------------------------------------------- */
bsa_status mask_or(uint8_t* dst, const uint8_t* a, int64_t n, const uint8_t* b, int64_t b_n,
                   bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Mask compaction into per-query-block kv lists [CalibAtt skip lists].
 *   mask       uint8 [B,H,nb,nb] with plane strides mask_sb, mask_sh (bytes)
 *   row_ptr    int32 [B*H*nb + 1]; row r = (b*H + h)*nb + i
 *   col_idx    int32 [B*H*nb*nb] capacity; row r's kept kv blocks, ascending, are
 *              col_idx[row_ptr[r] .. row_ptr[r+1])
 *   order      optional (NULL = none) int32 [B*H*nb]: the rows sorted by kept count,
 *              largest first, equal counts by ascending row index (a longest-first
 *              work list); nb at most 16382, else BSA_EUNSUPPORTED
 *   ws         at least csr_workspace_size(B, H, nb) bytes
 * ------------------------------------------------------------------------- */
size_t csr_workspace_size(int B, int H, int nb);
bsa_status bsa_mask_to_csr(const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int B, int H,
                           int nb, int32_t* row_ptr, int32_t* col_idx, int32_t* order, void* ws,
                           size_t ws_bytes, bsa_stream_t stream);

/* The same kv lists plus the attention kernel's work order for them (the order
 * attn_work_order writes; see block_sparse_attn_fwd below) in one call. For small masks
 * (B*H*nb <= 4096 rows, nb a multiple of 16 and <= 512, contiguous or one plane) both come
 * from a single launch, the order built by one extra workgroup from the mask's row
 * counts beside the compaction; otherwise the order is a second launch.
 *   work_order int32 [attn_work_order_slots(shape)] for a shape with these B, H and
 *              S = 64 nb; BSA_EUNSUPPORTED when that is 0 (the shape runs in the
 *              default order)
 * Other arguments, workspace and errors as bsa_mask_to_csr. Equal keys may be ordered
 * differently from attn_work_order's; the attention results never depend on the order. */
bsa_status bsa_mask_to_csr_ordered(const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int B, int H,
                                   int nb, int32_t* row_ptr, int32_t* col_idx, int32_t* work_order,
                                   void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Block-sparse attention forward [FA: exact tiled attention with online softmax,
 * extended to block-sparse attention; NABLA: the mask tells the operator which
 * N x N blocks to compute].
 *
 * For query token p of head (b,h): key token q is allowed iff mask[p/64][q/64]
 * is nonzero and q < S_valid;  O_p = sum_q softmax_q(scale * <Q_p, K_q>) V_q over
 * allowed q. Only kept 64 x 64 tiles are computed. Query rows >= S_valid, and
 * query rows with no allowed key, get O = 0 and lse = -inf.
 *
 *   q, k       bf16 [B,H,S,D]; or both f32; or both fp8 e4m3fn (then q_scale,
 *              k_scale are float [B,H,nb] contiguous: the value of a code c in
 *              block j is fp8(c) * scale[b,h,j]); D in {64, 128}
 *   v          bf16 (f32 when q, k are f32) [B,H,S,D]
 *   scale      softmax scale; <= 0 selects 1/sqrt(D)
 *   o          output [B,H,S,D]: bf16, or f32 when q, k are f32; o->ptr is written
 *   lse        optional (NULL = none) float [B,H,S] natural-log sum of exp
 *   ws         at least attn_workspace_size(shape, q->dtype) bytes, 256-byte
 *              aligned (holds the kv lists, for f32 inputs hi/lo bf16 copies, and
 *              the partial states of the kv-chunked walk below)
 * All of q, k, v, o must have 16-byte aligned rows (ss*elem_size % 16 == 0 and the
 * base pointers 16-byte aligned).
 * block_sparse_attn_fwd_csr takes kv lists already built by bsa_mask_to_csr (for
 * masks reused across calls) and needs attn_csr_workspace_size(shape, q->dtype)
 * bytes, 256-byte aligned (for f32 inputs the hi/lo bf16 copies, and the partial
 * states of the kv-chunked walk; when the size is 0, ws may be NULL).
 *
 * Work order: one workgroup per pair of adjacent query blocks; the pairs are cut
 * into 8 contiguous ranges, one per XCD. When the pairs make at most four rounds over
 * the device's workgroup slots (3 per compute unit) and nb <= 512, each range is sorted by the longer of
 * the pair's two kv lists and started longest first, so that short pairs fill the
 * tail. attn_work_order_slots(shape) gives the length of that order (0: the shape
 * runs in the natural order; -1: invalid shape); attn_work_order writes it for the
 * kv lists row_ptr into order (int32 [slots]; entry x is the pair index
 * (b*H + h) * ceil(nb/2) + p started by workgroup x, or -1). Pass it as work_order to
 * block_sparse_attn_fwd_csr to reuse it; with work_order NULL each attention workgroup
 * derives its own item of that order from the kv-list lengths (no extra launch). Shapes
 * with more pairs (0 slots) run the ranges in natural order, or, from nb = 512 on, with
 * each head's pairs longest first, also derived in the kernel. The order never changes
 * the results.
 *
 * Pairing offsets: for shapes without a work order and from nb = 512 on, the two query
 * blocks of a workgroup are not always neighbours. The workgroup walks the union of their
 * kv lists, and a tile that only one block keeps idles the other block's waves for a step;
 * in row-major video layouts a block's list is often closer to that of the block one
 * frame later. So each call first picks, for every head, the offset d in [1, min(64,
 * nb/2)] whose pairing has the fewest union steps (sum over pairs of |list(a) u list(b)|,
 * ties to the smaller d): the blocks are taken in runs of 2d, block a of a run's first half
 * paired with a + d, and the blocks after the last whole run pair with their neighbour
 * (d = 1: pairs (2p, 2p + 1)). Three small launches; the workspace includes their
 * buffers. The pairing never changes the results beyond the order of the list walk, which
 * is ascending for every block either way: outputs are the same bit for bit.
 * attn_pair_offsets writes the offsets the attention would choose for the kv lists
 * (row_ptr/col_idx, or with row_ptr NULL the fixed-stride lists kv_len/col_idx of stride
 * nb) into pair_d (int32 [B*H]); its workspace is attn_pair_workspace_size(shape) bytes,
 * 256-byte aligned.
 *
 * kv-chunked walk [LeanAttention (Daily Papers listing): the online softmax of a row
 * split into parts that are merged afterwards], taken only when asked for:
 * bsa_set_attn_kv_chunk(w) with w > 0 makes every later attention call (and workspace
 * query) of the process cut the key blocks into chunks of w blocks and run every
 * (head, chunk, pair of query blocks) as a work item; the 8 XCD ranges take the items
 * chunk-major inside each head, so that the workgroups running together on an XCD read
 * the same K/V tiles from its L2 (w = 64 at D = 128 keeps 2 MB of K and V per chunk).
 * Each item leaves the unnormalised partial output and (max, sum) of its rows in the
 * workspace (B*H*nb rows x ceil(nb/w) chunks x 64 x (4 D + 8) bytes: 27.9 GB at B=1,
 * H=40, S=75648, D=128, w=64), and a combine launch merges a row's chunks in ascending
 * order. The results are deterministic and equal to the whole-row walk's up to rounding
 * (each chunk rounds its probabilities to bf16 against its own running maximum). The
 * work order is not used. w <= 0 returns to whole rows (the default); the call returns
 * the previous width. Workspace sizes follow the setting, so query them after changing
 * it. At the 14B shape the chunked walk cuts the attention kernel's L2 misses twelvefold
 * but not its time, and the combine adds about 12%.
 * ------------------------------------------------------------------------- */
int bsa_set_attn_kv_chunk(int kv_chunk);
size_t attn_pair_workspace_size(const bsa_shape* shape);
bsa_status attn_pair_offsets(const bsa_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                             const int32_t* kv_len, int32_t* pair_d, void* ws, size_t ws_bytes,
                             bsa_stream_t stream);
size_t attn_workspace_size(const bsa_shape* shape, bsa_dtype qk_dtype);
bsa_status block_sparse_attn_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                 const bsa_shape* shape,
                                 const uint8_t* mask, int64_t mask_sb, int64_t mask_sh,
                                 const float* q_scale, const float* k_scale, double scale,
                                 const bsa_tensor* o, float* lse,
                                 void* ws, size_t ws_bytes, bsa_stream_t stream);

size_t attn_csr_workspace_size(const bsa_shape* shape, bsa_dtype qk_dtype);
bsa_status block_sparse_attn_fwd_csr(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                     const bsa_shape* shape,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     const int32_t* work_order,
                                     const float* q_scale, const float* k_scale, double scale,
                                     const bsa_tensor* o, float* lse,
                                     void* ws, size_t ws_bytes, bsa_stream_t stream);

/* block_sparse_attn_fwd_lists takes the fixed-stride kv lists of nabla_build_mask_lists
 * (row r's kv blocks at kv_idx[r*nb .. r*nb + kv_len[r]), ascending, B*H*nb*nb below
 * 2^31) in place of row_ptr / col_idx; everything else as block_sparse_attn_fwd_csr
 * (workspace attn_csr_workspace_size; work_order NULL: each attention workgroup derives
 * its item of that order from kv_len, with no extra launch). */
bsa_status block_sparse_attn_fwd_lists(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                       const bsa_shape* shape,
                                       const int32_t* kv_len, const int32_t* kv_idx,
                                       const int32_t* work_order,
                                       const float* q_scale, const float* k_scale, double scale,
                                       const bsa_tensor* o, float* lse,
                                       void* ws, size_t ws_bytes, bsa_stream_t stream);

int attn_work_order_slots(const bsa_shape* shape);
bsa_status attn_work_order(const bsa_shape* shape, const int32_t* row_ptr, int32_t* order,
                           bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Block-sparse attention backward [FA: exact tiled attention trains Transformers
 * and extends to block-sparse attention; NABLA review, "Editorial extensions": a DiT
 * trains with the NABLA block mask]. The gradients of the forward above, for the
 * same mask, from the upstream gradient dO:
 *   P = softmax over allowed keys,  dV = P^T dO,  dP = dO V^T,
 *   delta_p = <dO_p, O_p>,  dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q.
 * Query rows >= S_valid and query rows with no allowed key (lse = -inf) carry no
 * gradient: their dQ rows are 0 and they add nothing to dK, dV; key rows >= S_valid
 * get dK = dV = 0. The probabilities are recomputed from lse; no atomics are used, so
 * the results are the same on every run.
 *
 *   q, k, v    bf16 [B,H,S,D], D in {64, 128} (the forward's inputs)
 *   o          bf16 [B,H,S,D], the forward's output for these inputs and this mask
 *   d_o        bf16 [B,H,S,D], the gradient of the loss with respect to o
 *   lse        float [B,H,S] contiguous, the forward's lse output
 *   mask       the forward's block mask (same layout and strides as there)
 *   scale      softmax scale; <= 0 selects 1/sqrt(D) (must match the forward)
 *   dq, dk, dv outputs [B,H,S,D], all three bf16 or all three f32; every row written
 *   ws         at least attn_bwd_workspace_size(shape) bytes, 256-byte aligned (holds
 *              delta, the transposed mask and both index lists)
 * Row alignment as for the forward. Errors: BSA_EINVAL for bad pointers, strides or
 * dtypes, BSA_EUNSUPPORTED for other dtypes or D, BSA_EWORKSPACE for a short ws.
 * ------------------------------------------------------------------------- */
size_t attn_bwd_workspace_size(const bsa_shape* shape);
bsa_status block_sparse_attn_bwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                 const bsa_tensor* o, const bsa_tensor* d_o, const float* lse,
                                 const bsa_shape* shape,
                                 const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, double scale,
                                 const bsa_tensor* dq, const bsa_tensor* dk, const bsa_tensor* dv,
                                 void* ws, size_t ws_bytes, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Token reordering [NABLA review, Figure 4 and "Assumptions & free parameters":
 * fractal flattening into P x P spatial patches; STA: tokens grouped into 3D tiles;
 * SVG: layout transformation grouping one spatial position across frames]. The
 * T*H*W token rows of x [B,H,S,D] are permuted between the row-major (t, h, w) order
 * and one of:
 *   BSA_ORDER_TILE     tiles of tile_thw in row-major tile order, tokens row-major
 *                      inside a tile, smaller tiles at the grid border (fractal
 *                      flattening with patch P is tile_thw = {1, P, P});
 *   BSA_ORDER_SPATIAL  (h, w, t): the frames of one spatial position together;
 *   BSA_ORDER_ROW      the identity (a copy).
 * inverse = 0: out = x (row-major) in the chosen order; inverse = 1: x is in the
 * chosen order and out is row-major (the scatter back of the attention output).
 * Rows >= S_valid of out are written as zeros. x and out: same dtype (bf16, f32 or
 * fp8 codes), own strides, distinct buffers; S_valid = T*H*W. Errors: BSA_EINVAL.
 * ------------------------------------------------------------------------- */
#define BSA_ORDER_ROW 0
#define BSA_ORDER_TILE 1
#define BSA_ORDER_SPATIAL 2
bsa_status token_reorder(const bsa_tensor* x, const bsa_shape* shape, const int grid_thw[3], int order,
                         const int tile_thw[3], int inverse, const bsa_tensor* out, bsa_stream_t stream);

/* Message describing the last failed call on this thread ("" if none). */
const char* bsa_last_error(void);

/* Version of this interface (incremented on incompatible changes). */
int bsa_abi_version(void);

/* ---------------------------------------------------------------------------
 * Checked build (libbsa_checked.so, compiled with -DBSA_CHECKED; for tests and
 * debugging, not for timing). Its kernels test the indices they read from list data
 * before using them: kv-list entries in [0, nb) and list lengths in [0, nb] in the
 * attention forward and its in-kernel work order, list entries inside the bit rows of
 * the pairing pass, list entries of the backward walks. A failed test sets a bit of a
 * device flag word and skips the access (the bad list is cut short), so a run with bad
 * lists from a caller completes and reports instead of reading or writing out of bounds.
 * bsa_checked_build: 1 in the checked library, 0 in the production one.
 * bsa_check_flags: the OR of the flag words since the last clear (bit 0: attention list
 * entry, bit 1: list length, bit 2: bit-row entry, bit 3: backward list entry); clear != 0
 * also resets them. Synchronous (waits for the device); 0 in the production library;
 * 0xFFFFFFFF if reading the device words failed.
 * ------------------------------------------------------------------------- */
int bsa_checked_build(void);
unsigned bsa_check_flags(int clear);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
