/*
 * libidx -- dense prefill indexer for AMD Instinct MI355X (gfx950).
 *
 * The indexer scores a prefill chunk of T query rows against a compressed key
 * prefix of L rows and keeps, per query row, the top-K keys:
 *
 *     I[t, s] = sum_h w[t, h] * max(0, scale * <qd[t, h, :], kd[s, :]>),
 *     s in the row's key window [ks[t], ke[t])
 *
 * qd / kd are the dequantised fp8 E4M3 queries and fp8 E4M3 or MXFP4 keys.
 * The pages this library follows describe the call but do not print the
 * formula; it is the DeepSeek sparse-attention indexer score.  Sources, cited
 * by page title and section:
 *
 *   P1  "Running CHUNKED_PREFILL_SIZE above 1024 without the long-prompt
 *       memory problem" -- section 1 (the dense indexer call: T rows against
 *       the whole compressed prefix, output [T, max_seqlen_k] fp32, ragged
 *       top-k, the layer-20 candidate source pooling 8-key blocks into a
 *       top-2048 block mask consumed by later layers through masked_fill_),
 *       section 2.3 (key blocks of B_k with per-block top-k and a merge:
 *       topk(union) == topk(union of per-block topk); memory c*T*B_k).
 *   P2  "[DeepSeek-V4.1] Bound the dense prefill indexer transient: row-chunk
 *       logits, tail-only candidate masks" -- Motivation (fp8 q x fp4 k
 *       logits [T, lc] fp32 are the transient), Modifications (row chunks
 *       under a 2 GiB logits budget, top-k of each chunk into one shared
 *       selected buffer, masks written into one preallocated [rows, lc]
 *       tensor), Accuracy/equivalence (index sets and masks compared
 *       bitwise; row-count invariance; determinism).
 *   P3  commit messages of an SGLang fork -- the NSA-indexer chunk-budget
 *       microbenchmark (fp8_mqa_logits + fast_topk_transform_fused at H=32,
 *       D=128, topk=2048) and the per-batch ragged plan / no per-request
 *       host syncs in forward_indexer.
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers owned by the caller.  libidx never
 *     allocates or frees memory and never synchronises the stream (the
 *     IDX_DEBUG checks and idx_launch_timing_read, which waits for its
 *     events, excepted).  Scratch space is the caller's `ws` buffer, sized by
 *     idx_workspace_size().
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *   - A status other than IDX_OK from argument checking means nothing was
 *     enqueued.  IDX_E_LAUNCH reports a failed launch (hipGetLastError); the
 *     outputs are then undefined.
 *   - Arrays are row-major with a contiguous last dimension; leading
 *     dimensions (ld*) count elements.  q, k and logits need 16-byte
 *     alignment, everything else its element alignment.
 *   - Key indices in outputs are absolute rows of k.  Selected indices of a
 *     row are ascending; unused slots hold -1 (values -inf).
 *   - Order of selection: fp32 score descending, then key index ascending.
 *     The selected set is unique under this total order, so results are
 *     bitwise deterministic and independent of row chunking and key blocking.
 *   - Scores come from the fp8 MFMA, whose accumulation truncates (groups of 8
 *     products, each cut toward zero 13 bits below the group's largest
 *     exponent sum e_q + e_k; group sums added in fp32 with two guard bits,
 *     ties to even): about 2e-5 relative on Gaussian data.  Where every head
 *     weight of the rows a workgroup scores is >= 0, each ReLU'd head term is
 *     rounded to f16 (2^-11 relative, plus at most 2^-25 absolute once every
 *     possible term is scaled into [0, 1)) and the weighted head sum runs on
 *     an f16 MFMA that accumulates exactly in fp32: at most about 5e-4
 *     relative, 2.6e-4 measured, inside the 1e-3 logit tolerance.  Other rows
 *     take an fp32 head sum.  The error scales with the head terms, so with
 *     head weights of both signs it is relative to sum_h |w'[t, h]| *
 *     ReLU(...), not to a score that those terms cancel down to.  Paths that
 *     select from q/k (idx_logits_topk_fused, idx_block_candidates without
 *     logits, idx_refine_topk) keep K + 512 candidates and re-score exactly
 *     (fp64 over the exact fp8 products) every candidate within +-2D of the
 *     K-th score, D a per-row error scale: twice the truncation unit 2^-13
 *     Kmax Mq_h of each head (4.5 to 36 standard deviations of the error
 *     measured on N(0,1) data), plus the f16 rounding bound.  Their selection
 *     is that of the exact scores rounded to fp32 whenever no key's scoring
 *     error exceeds D.  D is not a worst-case bound: keys can be built whose
 *     products cancel but for small terms the MFMA drops, so that their error
 *     exceeds it; such keys can be misplaced.  idx_topk selects exactly on the
 *     values it is given.  The first 4 bytes of the workspace receive the
 *     number of rows whose candidate list was too short to settle the boundary
 *     (0 on every workload this library was measured on).
 *   - Exact mode.  With the environment variable IDX_EXACT set (to anything
 *     but "0", read on every call) every score is computed exactly from the
 *     stored codes instead: fp8 x fp8 and fp8 x e2m1 products are exact, their
 *     128-term sums are exact in fp64, scales, ReLU, weights and the head sum
 *     follow in fp64, and each score rounds to fp32 once.  Logits are then
 *     within one fp32 ulp of the exact values, for head weights of any sign,
 *     and the selection is that of the exact scores for any keys.  The fused
 *     path then scores key blocks into its scratch only (no candidate slabs).
 *     This runs on the fp64 VALU, some 50 times slower than the default mode;
 *     workspace sizes and every other contract are unchanged.
 *   - Preconditions the host cannot check without reading device memory
 *     (0 <= ks[t] <= ke[t] <= L, finite inputs, q_scale/k_scale >= 0, window
 *     length <= W where a W is given) are the caller's; violating them gives
 *     undefined results but no out-of-bounds access of q/k (key rows are
 *     clamped to [0, L)).  With the environment variable IDX_DEBUG set (to
 *     anything but "0"), every entry point that reads windows first checks
 *     them, and the scales and weights of its problem, on the device,
 *     synchronises the stream, and returns IDX_E_DEVICE_CHECK without
 *     enqueueing its own kernels if one fails.
 *   - Supported: D = 128; H in {32, 64}; 1 <= K <= 2048; block_k a multiple of
 *     256 in [256, 32768]; pool = 8; 1 <= n_blocks <= 2048.
 */
#ifndef LIBIDX_IDX_H
#define LIBIDX_IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t idx_status;
enum {
  IDX_OK = 0,
  IDX_E_NULL = 1,        /* a required pointer is NULL                          */
  IDX_E_SHAPE = 2,       /* inconsistent sizes (T, L, W, leading dimensions)    */
  IDX_E_PARAM = 3,       /* parameter out of range (K, block_k, row_chunk, ...) */
  IDX_E_FORMAT = 4,      /* unknown key format                                  */
  IDX_E_WORKSPACE = 5,   /* ws_bytes below idx_workspace_size()                 */
  IDX_E_UNSUPPORTED = 6, /* valid but not provided (D != 128, H, ...)           */
  IDX_E_LAUNCH = 7,      /* a kernel launch failed                              */
  IDX_E_ALIGN = 8,       /* a pointer lacks the required alignment              */
  IDX_E_DEVICE_CHECK = 9 /* IDX_DEBUG: a precondition in device memory failed   */
};

enum { IDX_K_FP8_E4M3 = 0, IDX_K_MXFP4 = 1 };

/* Operations for idx_workspace_size(). */
enum {
  IDX_OP_MQA_LOGITS = 0,       /* idx_mqa_logits: no workspace                          */
  IDX_OP_TOPK = 1,             /* idx_topk: no workspace                                */
  IDX_OP_LOGITS_TOPK_FUSED = 2,
  IDX_OP_BLOCK_CANDIDATES = 3, /* idx_block_candidates with logits == NULL (fused)      */
  IDX_OP_BLOCK_CANDIDATES_DENSE = 4, /* idx_block_candidates from given logits          */
  IDX_OP_GATHER_ROWS = 5       /* idx_gather_rows of K rows                             */
};

/* One indexer call's inputs (all device pointers). */
typedef struct idx_problem {
  const uint8_t *q;       /* [T, H, D] fp8 E4M3 (OCP "FN": max 448, no inf)                 */
  const float *q_scale;   /* [T, H] dequantisation scale of each (t, h) row of D, >= 0       */
  const void *k;          /* fp8: uint8 [L, D] E4M3;  MXFP4: uint8 [L, D/2] E2M1 pairs,
                             element d in the low nibble of byte d/2 when d is even          */
  const void *k_scale;    /* fp8: float [L] per key row, >= 0;  MXFP4: uint8 E8M0 [L, D/32],
                             one power-of-two scale per 32 consecutive d                    */
  int32_t k_fmt;          /* IDX_K_FP8_E4M3 or IDX_K_MXFP4                                  */
  const float *w;         /* [T, H] head weights, any sign                                   */
  const int32_t *ks;      /* [T] first key of row t's window                                 */
  const int32_t *ke;      /* [T] one past the last key of row t's window                     */
  int32_t T, H, D, L;     /* query rows, heads, head dim (128), key rows                     */
  float scale;            /* extra positive factor inside the ReLU (1.0 if unused)           */
} idx_problem;

/* Dense MQA logits (P1 section 1: output [T, max_seqlen_k] fp32; P2 Motivation).
 * logits: [T, ld] fp32, ld >= W.  Column j of row t holds I[t, ks[t] + j] for
 * j < ke[t] - ks[t] and -inf for ke[t] - ks[t] <= j < W.  Columns >= W are not
 * touched.  W is normally the longest window (max_seqlen_k). */
idx_status idx_mqa_logits(const idx_problem *p, float *logits, int64_t ld, int32_t W, void *stream);

/* Logits of one rectangle in key-block layout: rows [row0, row0 + nrows) and
 * absolute keys [key0, key0 + nkeys), key0 a multiple of 256.  out: [nrows, ld]
 * fp32, ld >= nkeys; column c of row r holds I[row0 + r, key0 + c] where that key
 * is inside the row's window; other columns are not written.  This is the
 * scoring stage of the key-blocked indexer (P1 section 2.3), exposed so callers
 * can drive their own block loop. */
idx_status idx_mqa_logits_block(const idx_problem *p, int32_t row0, int32_t nrows, int32_t key0,
                                int32_t nkeys, float *out, int64_t ld, void *stream);

/* Top-K of dense row-relative logits (P2 Modifications: ragged top-k into the
 * shared selected buffer; P1 section 2.3).
 * logits: [T, ld] fp32 as written by idx_mqa_logits; row t's candidates are
 * columns j < ke[t] - ks[t] (key ks[t] + j).  mask (nullable): [T, ld_mask]
 * bytes over the same columns; keys whose mask byte is 0 are never selected.
 * block_k: columns scored per pass (the selection is exact for any value).
 * out_idx: [T, K] int32 absolute key indices, ascending, -1 padded.
 * out_val (nullable): [T, K] fp32 logits of the selected keys, -inf padded.
 * ws may be NULL (no workspace).  K may go up to 2560 here, so that the list
 * can feed idx_refine_topk. */
idx_status idx_topk(const float *logits, int64_t ld, int32_t W, const int32_t *ks, const int32_t *ke,
                    const uint8_t *mask, int64_t ld_mask, int32_t T, int32_t K, int32_t block_k,
                    int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes, void *stream);

/* Fused key-blocked indexer (P1 section 2.3): for each chunk of row_chunk rows,
 * score its first key block of block_k keys into a [row_chunk, block_k] fp32
 * scratch and take each row's top-(K + 512) from it; every later launch (up to
 * four blocks of keys) writes only the scores above each row's running
 * (K + 512)-th to per-row candidate slabs in the scratch rows, which are merged
 * into the running lists (the rows of a row block where a slab overflowed are
 * scored again into the scratch, one block at a time); then settle the boundary
 * exactly (idx_refine_topk).  [T, L] logits
 * are never materialised: the workspace is O(row_chunk * (block_k + K)), with
 * a bound that holds whatever L.  The result
 * equals idx_mqa_logits + idx_topk (K + 512 columns) + idx_refine_topk
 * bitwise.  mask (nullable):
 * [T, ld_mask] bytes, column j <-> key ks[t] + j (the candidate mask of
 * idx_block_candidates); keys with mask 0 are excluded.  Outputs as idx_topk. */
idx_status idx_logits_topk_fused(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                                 const uint8_t *mask, int64_t ld_mask, int32_t *out_idx,
                                 float *out_val, void *ws, size_t ws_bytes, void *stream);

/* Size of the library's own workspace for idx_logits_topk_fused_static: 128 MiB of device
 * memory per GPU the library is loaded on, held until the process ends. */
#define IDX_STATIC_WS_BYTES (128u << 20)

/* For callers that cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc): idx_logits_topk_fused with the library's static
 * workspace instead of a caller buffer.  Arguments, outputs and results are those of
 * idx_logits_topk_fused.  Returns IDX_E_WORKSPACE (nothing enqueued) when the call needs more
 * than IDX_STATIC_WS_BYTES, i.e. idx_workspace_size(IDX_OP_LOGITS_TOPK_FUSED, ...) is larger:
 * a smaller row_chunk fits (256 rows do for block_k 32768 at any K).  No memory is
 * allocated or freed.  The workspace keeps the last
 * call's contents, and the overflow word that idx_logits_topk_fused leaves in its first 4
 * bytes is not visible to the caller.  Every call on one GPU shares the workspace: calls
 * that overlap in time on the same GPU (two streams, two host threads) race. */
idx_status idx_logits_topk_fused_static(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                                        const uint8_t *mask, int64_t ld_mask, int32_t *out_idx, float *out_val,
                                        void *stream);

/* The fused indexer with the index -> KV-slot transform in its final write (P3:
 * the top-k kernel with the transform fused in; P2 Accuracy/equivalence:
 * page_indices published next to raw_indices).  As idx_logits_topk_fused, plus
 * slot_of_key: device int32 [L], the KV-cache slot of every key row (the caller's
 * token -> slot table over the rows of k); out_slot: [T, K] int32,
 * out_slot[t, j] = slot_of_key[out_idx[t, j]], -1 where out_idx[t, j] is -1.
 * Both NULL: exactly idx_logits_topk_fused; one of them NULL: IDX_E_NULL. */
idx_status idx_logits_topk_fused_paged(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                                       const uint8_t *mask, int64_t ld_mask, const int32_t *slot_of_key,
                                       int32_t *out_idx, float *out_val, int32_t *out_slot, void *ws,
                                       size_t ws_bytes, void *stream);

/* The fused indexer as a block-aware consumer of the candidate source (P1 section
 * 2.3: the consumers' masking applies per block; P2 Motivation: a byte mask over
 * [rows, lc] is the memory problem).  As idx_logits_topk_fused with a mask, but the
 * mask is given as block ids: row t may select key s only if block
 * (s - ks[t]) / pool is among blocks[t * ld_blocks + i], i < n_blocks (the
 * out_blocks layout of idx_block_candidates; ids -1 are ignored).  The result equals
 * idx_logits_topk_fused with the byte mask those blocks expand to.  No [T, L] byte
 * mask is read or written.  pool: a power of two with block_k / pool + 2 <= 9216
 * (pool >= 4 at block_k = 32768; IDX_E_UNSUPPORTED otherwise): each launch takes
 * one key block. */
idx_status idx_logits_topk_fused_blocks(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                                        const int32_t *blocks, int64_t ld_blocks, int32_t n_blocks, int32_t pool,
                                        int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes, void *stream);

/* Exact boundary of a top-K from K + R approximate candidates per row.
 * cand_idx / cand_val: device [T, ld_cand], the output of idx_topk with Kc
 * columns (ids ascending, -1 padded; values are the scores the ids were
 * selected by).  Candidates whose score lies within a per-row error bound of
 * the K-th score are re-scored exactly from p (pool = 1: ids are keys;
 * pool = 8: ids are 8-key blocks from ks[t], scored by their max) and the
 * K best under (exact fp32 score desc, id asc) are kept.  out_idx: [T, K]
 * ascending, -1 padded; out_val (nullable) the scores (exact where
 * re-scored).  ws: at least 2304 bytes (256-byte aligned) of scratch.
 * K <= Kc <= 2560, K <= 2048. */
idx_status idx_refine_topk(const idx_problem *p, const int32_t *cand_idx, const float *cand_val, int64_t ld_cand,
                           int32_t Kc, int32_t K, int32_t pool, int32_t *out_idx, float *out_val, void *ws,
                           size_t ws_bytes, void *stream);

/* Candidate source (P1 section 1, select_candidate_blocks; P2 Modifications:
 * masks written in place into one preallocated [rows, lc] tensor).
 * Pool the logits of each row over blocks of `pool` keys starting at ks[t]
 * (max; a partial last block takes the max of its in-window keys), keep the
 * n_blocks blocks with the highest pooled fp32 value (ties: lower block), and
 * write mask: [T, ld_mask] bytes, mask[t, j] = 1 iff j < ke[t] - ks[t] and block
 * j / pool is kept, else 0, for 0 <= j < W.
 * logits != NULL: read dense row-relative logits [T, ld] (idx_mqa_logits layout;
 * q/k/w of p are not read) and select exactly on them.  logits == NULL: score
 * from p block by block (block_k keys, row_chunk rows) and settle the block
 * boundary exactly as idx_refine_topk does; blocks start at each row's ks[t] whatever its
 * alignment.
 * out_blocks (nullable): [T, n_blocks] int32 kept block ids, ascending, -1 padded. */
idx_status idx_block_candidates(const idx_problem *p, const float *logits, int64_t ld, int32_t pool,
                                int32_t n_blocks, int32_t block_k, int32_t row_chunk, uint8_t *mask,
                                int64_t ld_mask, int32_t W, int32_t *out_blocks, void *ws,
                                size_t ws_bytes, void *stream);

/* Workspace bytes an operation needs (host only; touches no device). */
idx_status idx_workspace_size(int32_t op, const idx_problem *p, int32_t K, int32_t block_k,
                              int32_t row_chunk, int32_t pool, int32_t n_blocks, int32_t W,
                              size_t *bytes);

/* Per-row windows of a varlen batch (P3: one ragged plan per batch instead of
 * per-layer descriptor rebuilds; P1 section 2.1: a request landing on a cached
 * prefix).  Request i owns query rows [cu_q[i], cu_q[i+1]) and key rows
 * [cu_k[i], cu_k[i+1]); its new rows are the last of its keys, so row j of
 * request i gets ks = cu_k[i], ke = cu_k[i] + (len_k - len_q) + j + 1.
 * cu_q, cu_k: device int32 [B + 1]; ks, ke: device int32 [T]; rows at or past
 * cu_q[B] get the empty window ks = ke = 0. */
idx_status idx_ragged_windows(const int32_t *cu_q, const int32_t *cu_k, int32_t B, int32_t T,
                              int32_t *ks, int32_t *ke, void *stream);

/* Per-row windows over compressed keys (P1 section 1: the ratio-1/2 source layers
 * score a chunk against the compressed prefix; P1 section 1 also puts the row's
 * own position into its window).  Request i owns query rows [cu_q[i], cu_q[i+1]),
 * token rows [cu_k[i], cu_k[i+1]) (its new tokens are the last len_q of them) and
 * key rows [cu_c[i], cu_c[i+1]), one key per `ratio` consecutive tokens.  New row j
 * of request i is token prefix + j, prefix = len_k - len_q, and sees the keys of
 * the complete groups up to it: ks = cu_c[i],
 * ke = cu_c[i] + min(floor((prefix + j + 1) / ratio), cu_c[i+1] - cu_c[i]).
 * ratio = 1 with cu_c = cu_k is idx_ragged_windows.  Rows at or past cu_q[B] get
 * ks = ke = 0.  cu_q, cu_k, cu_c: device int32 [B + 1]; ratio >= 1. */
idx_status idx_ragged_windows_ratio(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_c, int32_t ratio,
                                    int32_t B, int32_t T, int32_t *ks, int32_t *ke, void *stream);

/* Row subset of a problem (P2 Modifications: publish only each request's tail
 * rows, which the consumer would slice the masks down to anyway).  Copies row
 * rows[r] of p (q, q_scale, w, ks, ke) for r < R into ws, and fills *out with a
 * problem of R rows over p's keys whose row arrays point into ws.  Any entry point
 * run on *out then scores only those rows; its output row r belongs to p's row
 * rows[r].  rows[r] = -1 (or outside [0, p->T)) gives a padding row: zero q and the
 * empty window.  rows: device int32 [R]; ws: idx_workspace_size(IDX_OP_GATHER_ROWS,
 * p, K = R, ...) bytes, 256-byte aligned, and it must outlive the use of *out. */
idx_status idx_gather_rows(const idx_problem *p, const int32_t *rows, int32_t R, idx_problem *out, void *ws,
                           size_t ws_bytes, void *stream);

/* The last n query rows of every request of a varlen batch (the rows a tail-only
 * output keeps): rows[i * n + m] = cu_q[i+1] - n + m, or -1 where request i has
 * fewer than n rows.  cu_q: device int32 [B + 1]; rows: device int32 [B * n]. */
idx_status idx_tail_rows(const int32_t *cu_q, int32_t B, int32_t n, int32_t *rows, void *stream);

/* Launch timing, for benchmarks and profilers (P3: the chunk-budget and CPU-gap
 * commits attribute the indexer's time to its kernels).  idx_launch_timing(1) clears
 * the record and starts recording on the current device: from then on each scoring
 * launch of idx_mqa_logits, idx_mqa_logits_block, the fused entries and
 * idx_block_candidates (both dispatches of a launch pair, or the exact kernel under
 * IDX_EXACT) is bracketed by two HIP events on its call's stream.  At most
 * IDX_TIMING_MAX launches are recorded; launches on another device or on a stream under
 * capture are not.  idx_launch_timing(0) stops recording and keeps the record.
 * idx_launch_timing_read waits for the recorded events, writes the first min(cap, *n)
 * entries to out (host memory) in launch order, sets *n to the number recorded, and
 * clears the record.  An entry whose launch failed has ms < 0.  Events are created at
 * the first idx_launch_timing(1) on a device (IDX_E_LAUNCH if that fails) and kept until
 * the process ends or another device starts a record.  One record per process, guarded
 * by a lock: launches of calls that overlap on several host threads interleave in it. */
#define IDX_TIMING_MAX 1024
enum {
  IDX_LAUNCH_DENSE = 0, /* dense row-relative logits (idx_mqa_logits)                  */
  IDX_LAUNCH_BLOCK = 1, /* scores of a key rectangle (block launches of the fused path) */
  IDX_LAUNCH_POOL8 = 2, /* pooled 8-key blocks (the fused candidate source)             */
  IDX_LAUNCH_SLAB = 4   /* only the scores above each row's running threshold, to its
                           candidate slabs (the fused path's later launches)           */
};
typedef struct idx_launch_time {
  float ms;        /* first event to second event; < 0: the launch failed             */
  int32_t mode;    /* IDX_LAUNCH_*                                                    */
  int32_t flagged; /* 1: a pass over the row blocks whose slabs overflowed only       */
  int32_t row0, nrows; /* the launch's rows                                           */
  int32_t key0, nkeys; /* its keys; in the fused entries before the row chunk's shift
                          to its first window key                                     */
} idx_launch_time;
idx_status idx_launch_timing(int32_t enable);
idx_status idx_launch_timing_read(idx_launch_time *out, int32_t cap, int32_t *n);

/* Static description of a status code. */
const char *idx_status_str(idx_status s);

#ifdef __cplusplus
}
#endif
#endif /* LIBIDX_IDX_H */
