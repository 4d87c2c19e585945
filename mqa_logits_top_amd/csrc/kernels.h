// Internal interface between the C ABI layer (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

// STORE_SLAB: no scores, only the candidate output (LogitsArgs::cand).
enum LogitsMode { STORE_DENSE = 0, STORE_BLOCK = 1, STORE_POOL8 = 2, STORE_SLAB = 4 };

// Largest number of parts a scoring work item (row block x key split) is cut into.
constexpr int CAND_PARTS = 4;
// Candidate count word: the part's candidates (CAND_OVER if they exceeded its share of
// the slab) in the low 16 bits, the pair offset of its share in the slab above them.
constexpr uint32_t CAND_OVER = 0xFFFFu;

// One launch of the scoring kernel: rows [row0, row0 + nrows) against absolute
// keys [key_lo, key_hi), split into nsplit ranges of `split` keys.  A work item is
// one row block x one key split; the launch layout (set by launch_logits) gives the
// first nfull workgroups one whole item each, and cuts each later item into `parts`
// consecutive tile ranges, one workgroup each, so that the last wave of workgroups
// is as wide as the machine instead of a remainder.
struct LogitsArgs {
  const uint8_t *q;
  const float *q_scale;
  const uint8_t *k;
  const uint8_t *k_scale;  // fp8: float[L] bytes; MXFP4: uint8 [L, 4]
  const float *w;
  const int32_t *ks;
  const int32_t *ke;
  int32_t L;
  float scale;
  int32_t row0, nrows;
  int32_t key_lo, key_hi;
  int32_t split, nsplit;
  float *out;     // row r of the launch is out + r * ld
  int64_t ld;
  int32_t wcols;  // columns available in an output row (dense W, block nkeys, pool ceil(nkeys/8))
  int32_t nfull, parts;  // launch layout (filled by launch_logits)
  // Candidate output (STORE_SLAB): launch row r's in-window values above thr[r] (NaN: none)
  // go, as (value bits, key id) word pairs in key order, to its slab for the split: caps pairs
  // at pair r * cand_ld + split * caps of cand, part p of an item to its p-th share; the count
  // word ccnt[(r * nsplit + split) * CAND_PARTS + p] describes that share (parts that do not
  // exist: count 0).
  const float *thr;
  uint32_t *cand;
  int64_t cand_ld;   // pairs from one row's slabs to the next row's (>= nsplit * caps)
  uint32_t *ccnt;
  // STORE_BLOCK: score only the row blocks (RPW rows of the launch) whose word here is
  // nonzero (nullable: all)
  const uint32_t *only_flagged;
  int32_t caps;
  // The launch's window flag word (nullable; see WindowFlags).  Bit 1 set: no row of the launch
  // has a window key in its key range, and the launch does nothing.  Bit 0 picks the workgroup
  // -> XCD layout.  By key split (bit clear), each split's workgroups share an XCD, so its keys
  // stay in one L2 (rows whose windows span the keys).  By row block (bit set), each row block's
  // workgroups share an XCD; a launch whose rows each see only a small part of the keys (a
  // ragged batch of short requests) then spreads its active workgroups over every XCD instead
  // of the few that own the splits those windows touch.
  const uint32_t *by_row;
  // Launch pair marker (filled by launch_logits): a scoring launch is an f16 form and an fp32
  // form over the same grid.  An f16-form workgroup whose rows hold a head weight below zero
  // raises *neg_seq to seq (atomic max, a device word); fp32-form workgroups find nothing to
  // do unless *neg_seq >= seq.  seq grows with every launch pair in the process.
  unsigned long long *neg_seq;
  unsigned long long seq;
  // nullable: a device word added to key_lo and key_hi (the row chunk's first window key,
  // see WindowFlags)
  const int32_t *kshift;
};

hipError_t launch_logits(const LogitsArgs &a, int k_fmt, int H, int mode, hipStream_t s);
// The same scores computed exactly from the codes in fp64 (STORE_DENSE, STORE_BLOCK and
// STORE_POOL8 layouts; split and nsplit unused); rounded to fp32 once.
hipError_t launch_logits_exact(const LogitsArgs &a, int k_fmt, int H, int mode, hipStream_t s);
int logits_rows_per_workgroup(int H);   // RPW of the scoring launches
// Row blocks of a candidate-slab launch whose rows the top-K cannot serve from the slabs
// alone (a share overflowed, the shares together exceed the merge capacity, or the row's
// list is not full yet: thr NaN): flags[b] = 1 for them, 0 for the others (all 0 when
// launch_flag, nullable, marks the launch as holding no window key).
hipError_t launch_slab_check(const uint32_t *ccnt, int32_t nshares, const float *thr, int32_t nrows, int32_t rpw,
                             uint32_t *flags, const uint32_t *launch_flag, hipStream_t s);

// Top-K over row-major fp32 values (one workgroup per row, running top-K kept
// across passes).  Row r of the launch is problem row t = row0 + r.  Column c
// of that row is candidate id
//   TOPK_DENSE:        ks[t] + c              (absolute key; row-relative logits)
//   TOPK_BLOCK:        key0 + c               (absolute key; key-block scratch)
//   TOPK_POOL_DENSE:   c                      (pooled block id; row-relative)
//   TOPK_POOL_BLOCK:   key0 / pool - ks[t] / pool + c   (pooled block id; key-block scratch whose
//                      column c holds the block that starts in key group key0 / pool + c)
// Valid ids are [ks, ke) for keys and [0, ceil((ke - ks) / pool)) for blocks.
enum TopkMode { TOPK_DENSE = 0, TOPK_BLOCK = 1, TOPK_POOL_DENSE = 2, TOPK_POOL_BLOCK = 3 };
struct TopkArgs {
  const float *vals;
  int64_t ld;
  int32_t ncols;          // columns in one row of vals
  int32_t block;          // columns scored per pass (<= 32768)
  const int32_t *ks, *ke;
  int32_t row0, nrows;
  int32_t mode;
  int32_t key0;
  int32_t pool;
  const uint8_t *mask;    // nullable (key modes only); byte (id - ks) of row t
  int64_t ld_mask;
  int64_t mask_w;         // mask columns per row; bytes at or past it count as 0
  // Block-list consumer (nullable, TOPK_BLOCK only; exclusive with mask): row t may only
  // select keys whose block (id - ks) >> bpool_sh is among blocks[t * ld_blocks + i],
  // i < n_blocks (ids -1 ignored).  The launch's columns span at most BMAP_BITS blocks.
  const int32_t *blocks;
  int64_t ld_blocks;
  int32_t n_blocks, bpool_sh;
  int32_t K;
  int32_t *out_idx;       // row r at out_idx + r * K
  float *out_val;         // row r at out_val + r * K
  int32_t first;          // 1: no running state yet (out_* contents are ignored)
  // launch_merge only: the scoring launch's candidate slabs (layout as in LogitsArgs), and the
  // slab check's flags of its row blocks (slab_rpw rows each), whose rows were scored again into
  // vals and are left to topk_kernel
  const uint32_t *cand;
  int64_t cand_ld;
  const uint32_t *ccnt;
  int32_t nslab, caps;
  const uint32_t *slab_flags;
  int32_t slab_rpw;
  float *thr_out;         // nullable: per launch row, the full list's smallest value, else NaN
  // A launch's columns in several calls: vcols > 0 limits the columns read from vals to
  // [0, vcols); col_rows (nullable) receives 1 for a row that reads columns (launch_merge: 0 for a
  // row it merged); a call with only_rows set serves only the rows whose word there is nonzero.
  int32_t vcols;
  uint32_t *col_rows;
  const uint32_t *only_rows;
  const int32_t *kshift;  // nullable: a device word added to key0 (as LogitsArgs::kshift)
  // nullable: the scoring launch's window flag word (LogitsArgs::by_row); with its bit 1 set a
  // call other than the first has nothing new for any row and returns at once
  const uint32_t *launch_flag;
};
constexpr int BMAP_BITS = 9216;   // block bitmap of a top-K launch (65536 keys in 8-key blocks, and slack)
hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
// Slab merge of the rows outside flagged row blocks (TOPK_BLOCK args with cand, ccnt, nslab,
// caps, slab_flags, slab_rpw, col_rows and thr_out set; no mask or block list): each row's new
// running list from its list and its slabs.  col_rows receives 0 for a row merged (or with
// nothing to merge) and 1 for a row left to topk_kernel's column pass.
hipError_t launch_merge(const TopkArgs &a, hipStream_t s);

// Exact boundary refinement of per-row candidate lists (see refine.hip).
struct RefineArgs {
  const uint8_t *q;
  const float *q_scale;
  const uint8_t *k;
  const uint8_t *k_scale;
  int32_t k_fmt;
  const float *w;
  const int32_t *ks, *ke;
  int32_t H, L;
  float scale;
  int32_t row0, nrows;
  const int32_t *cand_idx;  // row r at cand_idx + r * ld_cand: ids ascending, -1 padded
  const float *cand_val;
  int64_t ld_cand;
  int32_t Kc, K;
  int32_t pool;             // 1: ids are keys; > 1: ids are pooled blocks of `pool` keys from ks
  const float *kmax_part;   // partial maxima of |k| (launch_key_bound), then at +256 those of the per-key
                            // factor the scoring kernel's F16 form applies after its head sum
  int32_t npart;
  uint32_t *overflow;       // rows whose band may extend below the list
  int32_t *out_idx;         // row r at out_idx + r * K
  float *out_val;
  // Index -> KV-slot transform of the written list (pool 1 only; nullable pair):
  // out_slot[r * K + j] = slot_of_key[out_idx[r * K + j]], -1 where the id is -1.
  const int32_t *slot_of_key;
  int32_t *out_slot;
};
int key_bound_parts(int L);
// Window coverage of the scoring launches of a row-chunked, key-blocked call: for row chunk c
// (rows [c Tc, c Tc + Tc)) and key launch l (keys [l LB, l LB + LB)), flags[c * nlaunch + l] = 1
// when the rows' windows cover less than half of that rectangle (the launch then lays its
// workgroups out by row block), else 0.
struct WindowFlags {
  const int32_t *ks, *ke;
  int32_t T, Tc;
  // launch l < nb takes keys [l B0, (l + 1) B0), launch l >= nb [nb B0 + (l - nb) LB, + LB)
  int32_t B0, nb, LB, nlaunch;
  // one word per (row chunk, launch): bit 0 when the rows' windows cover less than half of the
  // rectangle, bit 1 when they cover none of it
  uint32_t *flags;
  // nullable: per row chunk, the smallest ks of its rows with a non-empty window, rounded
  // down to 256 (0 when there is none); the chunk's launches are shifted by it, so that its
  // first launch holds the first keys its rows see
  int32_t *kshift;
};
constexpr int32_t KEY_SHIFT_ALIGN = 256;
constexpr int32_t MAX_WINDOW_FLAGS = 16384;
hipError_t launch_key_bound(const uint8_t *k, const uint8_t *k_scale, int k_fmt, int L, float *part,
                            uint32_t *overflow, const WindowFlags *wf, hipStream_t s);
hipError_t launch_refine(const RefineArgs &a, hipStream_t s);

// Dense-logits helpers
hipError_t launch_fill_tail(float *logits, int64_t ld, int32_t W, const int32_t *ks, const int32_t *ke,
                            int32_t row0, int32_t nrows, hipStream_t s);
hipError_t launch_pool_dense(const float *logits, int64_t ld, int32_t W, const int32_t *ks, const int32_t *ke,
                             int32_t row0, int32_t nrows, int32_t pool, float *out, int64_t ld_out,
                             int32_t ncols_out, hipStream_t s);
hipError_t launch_expand_mask(const int32_t *blocks, int32_t n_blocks, const int32_t *ks, const int32_t *ke,
                              int32_t row0, int32_t nrows, int32_t pool, int32_t W, uint8_t *mask,
                              int64_t ld_mask, hipStream_t s);
hipError_t launch_ragged(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_c, int32_t ratio, int32_t B,
                         int32_t T, int32_t *ks, int32_t *ke, hipStream_t s);
hipError_t launch_tail_rows(const int32_t *cu_q, int32_t B, int32_t n, int32_t *rows, hipStream_t s);
hipError_t launch_gather_rows(const int32_t *rows, int32_t R, int32_t T, const uint8_t *q, const float *q_scale,
                              const float *w, const int32_t *ks, const int32_t *ke, int32_t H, int32_t D, uint8_t *oq,
                              float *oqs, float *ow, int32_t *oks, int32_t *oke, hipStream_t s);

}  // namespace idx
