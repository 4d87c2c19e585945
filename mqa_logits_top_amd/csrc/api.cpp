// libidx C ABI: argument checking, workspace arithmetic, row-chunk / key-block
// planning and the launch sequence on the caller's stream.  Nothing here
// allocates device memory or synchronises; every check runs on the host
// before the first HIP call, so an error status means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/idx.h"
#include "api_internal.h"
#include "kernels.h"

namespace {

constexpr int32_t MAX_K = 2048;
constexpr int32_t RESERVE = 512;   // extra candidates kept for the exact boundary refinement
constexpr int32_t MAX_KC = 2560;
constexpr int32_t MAX_BLOCK = 32768;
constexpr int32_t MAX_W = 1 << 22;
constexpr int32_t KEY_ALIGN = 256;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

idx_status check_problem(const idx_problem *p, bool need_scores) {
  if (!p) return IDX_E_NULL;
  if (!p->ks || !p->ke) return IDX_E_NULL;
  if (p->T < 0 || p->L < 0 || p->H <= 0 || p->D <= 0) return IDX_E_SHAPE;
  if (!aligned(p->ks, 4) || !aligned(p->ke, 4)) return IDX_E_ALIGN;
  if (!need_scores) return IDX_OK;
  if (!p->q || !p->q_scale || !p->k || !p->k_scale || !p->w) return IDX_E_NULL;
  if (p->k_fmt != IDX_K_FP8_E4M3 && p->k_fmt != IDX_K_MXFP4) return IDX_E_FORMAT;
  if (p->D != 128) return IDX_E_UNSUPPORTED;
  if (p->H != 32 && p->H != 64) return IDX_E_UNSUPPORTED;
  if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return IDX_E_PARAM;
  if (!aligned(p->q, 16) || !aligned(p->k, 16)) return IDX_E_ALIGN;
  if (!aligned(p->q_scale, 4) || !aligned(p->w, 4)) return IDX_E_ALIGN;
  if (!aligned(p->k_scale, 4)) return IDX_E_ALIGN;  // fp32 per key, or 4 E8M0 bytes per key
  return IDX_OK;
}

int32_t round_up(int32_t x, int32_t a) { return (x + a - 1) / a * a; }
size_t round_up_sz(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Default / clamp the key block and row chunk.
int32_t eff_block(const idx_problem *p, int32_t block_k) {
  if (block_k > 0) return block_k;
  const int32_t b = round_up(p->L > 0 ? p->L : 1, KEY_ALIGN);
  return b < MAX_BLOCK ? b : MAX_BLOCK;
}
int32_t eff_chunk(const idx_problem *p, int32_t row_chunk) {
  if (row_chunk > 0) return row_chunk < p->T ? row_chunk : (p->T > 0 ? p->T : 1);
  return p->T > 0 ? p->T : 1;
}
idx_status check_block(int32_t block_k) {
  if (block_k < KEY_ALIGN || block_k > MAX_BLOCK || block_k % KEY_ALIGN) return IDX_E_PARAM;
  return IDX_OK;
}

// Workgroup key splits for one scoring launch over n keys: a multiple of 8 splits
// when possible (one XCD per split residue), each a multiple of 256 keys (whole
// scoring stages), about 8192 keys each.  Every split's workgroups load their rows' q
// (64 KiB per workgroup) once, so q is fetched once per split: longer splits fetch it
// less often and pay fewer workgroup prologues (same-box A/B against 4096-key splits:
// long_ctx fused step -2%, dsv4_mxfp4 -2.5%, glm_chunk unchanged).  The slabs hold
// 512 candidates per split, which the first slab launch of long_ctx fills to ~45%.
void plan_splits(int32_t n, int32_t &split, int32_t &nsplit) {
  if (n <= 0) { split = 128; nsplit = 0; return; }
  const int32_t target = 8192;
  int32_t ns = 8 * ((n + 8 * target - 1) / (8 * target));
  split = round_up((n + ns - 1) / ns, 256);
  if (split < 512) split = 512;
  nsplit = (n + split - 1) / split;
}

idx::LogitsArgs logits_args(const idx_problem *p, int32_t row0, int32_t nrows, int32_t key_lo, int32_t key_hi,
                            float *out, int64_t ld, int32_t wcols) {
  idx::LogitsArgs a{};
  a.q = p->q;
  a.q_scale = p->q_scale;
  a.k = (const uint8_t *)p->k;
  a.k_scale = (const uint8_t *)p->k_scale;
  a.w = p->w;
  a.ks = p->ks;
  a.ke = p->ke;
  a.L = p->L;
  a.scale = p->scale;
  a.row0 = row0;
  a.nrows = nrows;
  a.key_lo = key_lo;
  a.key_hi = key_hi;
  plan_splits(key_hi - key_lo, a.split, a.nsplit);
  a.out = out;
  a.ld = ld;
  a.wcols = wcols;
  return a;
}

// A scoring launch on the fp8 MFMA, or the exact fp64 kernel when `exact` (IDX_EXACT).
// One scoring launch (exact: the fp64 kernel), timed when a launch-timing record is on.
// flagged: a pass over the row blocks the slab check flagged.
hipError_t score(const idx::LogitsArgs &a, const idx_problem *p, int mode, bool exact, hipStream_t s,
                 bool flagged = false) {
  static_assert(IDX_LAUNCH_DENSE == idx::STORE_DENSE && IDX_LAUNCH_BLOCK == idx::STORE_BLOCK &&
                    IDX_LAUNCH_POOL8 == idx::STORE_POOL8 && IDX_LAUNCH_SLAB == idx::STORE_SLAB,
                "launch-timing modes name the scoring modes");
  const int token = idx::timing_begin(s);
  const hipError_t e =
      exact ? idx::launch_logits_exact(a, p->k_fmt, p->H, mode, s) : idx::launch_logits(a, p->k_fmt, p->H, mode, s);
  idx::timing_end(token, s, e == hipSuccess, mode, flagged ? 1 : 0, a.row0, a.nrows, a.key_lo, a.key_hi - a.key_lo);
  return e;
}

idx_status launched(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_E_LAUNCH; }

struct Carve {
  uint8_t *base;
  size_t off = 0;
  template <class T>
  T *take(size_t n) {
    T *r = (T *)(base + off);
    off = round_up_sz(off + n * sizeof(T), 256);
    return r;
  }
};

int32_t cand_cap(int32_t K) { return K + RESERVE < MAX_KC ? K + RESERVE : MAX_KC; }

// Workspace layout (every region 256-byte aligned):
//   [0, 256)            uint32 overflow counter of the last call, then free
//   key-bound partials  256 floats of max |k|, then 256 floats of the largest per-key factor
//   candidate ids/vals  [Tc, Kc] each
//   scratch             [Tc, pitch(Bk)] fp32 scores (or [Tc, pitch(Bk / pool)] pooled maxima)
constexpr size_t HEAD = 256 + 2048;
// Row pitch of scratch rows: 256 bytes beyond the row, so that the rows that
// the selection kernel streams at the same time start on different HBM channels
// instead of all sitting a power of two apart.
int32_t pitch(int32_t cols) { return cols + 64; }
size_t refine_ws(int32_t Tc, int32_t Kc) { return HEAD + 2 * round_up_sz((size_t)Tc * Kc * 4, 256); }
// Candidate slabs of the fused path: in a slab launch the scoring kernel appends each row's
// values above its running list's smallest entry to one slab of CAPS entries per key split;
// the top-K merges them instead of the keys.  A row's slabs lie in its row of the score
// scratch, which slab launches leave unused: a row block that the slab check flags is scored
// again into the scratch, over its slabs, and its rows then read columns instead.
constexpr int32_t CAPS = 512;
int32_t block_slabs(int32_t Bk) {
  int32_t split, nsplit;
  plan_splits(Bk, split, nsplit);
  return nsplit;
}
// Thresholds, slab-check flags and count words of ns slabs per row; then the per-row words of
// the two-call top-K of a launch wider than B_k.
size_t slab_ws(int32_t Tc, int32_t ns) {
  return round_up_sz((size_t)Tc * 4, 256) + round_up_sz((size_t)(Tc / 8 + 1) * 4, 256) +
         round_up_sz((size_t)Tc * ns * idx::CAND_PARTS * 4, 256) + round_up_sz((size_t)Tc * 4, 256);
}
// Floats per score scratch row: B_k scores (plus pitch), or the row's ns slabs of CAPS
// (value, id) pairs if they take more.
int32_t scratch_pitch(int32_t Bk, int32_t ns) { return std::max(pitch(Bk), ns * CAPS * 2); }
// Key launches of the fused path (P1 section 2.3: key blocks scored one after another, each
// row's running top-K merged across them; memory c * T * B_k).  The first launches of a row
// chunk score one block of B_k keys each into the [Tc, B_k] score scratch, from which the
// top-K builds and updates each row's running list of Kc = K + 512 entries and its threshold
// (the list's smallest entry).  Once the keys seen reach SLAB_DENSITY x Kc, so that at most one
// in SLAB_DENSITY of the next scores can still enter a list, every later launch writes only
// the scores above the threshold, to candidate slabs, and takes up to SLAB_BLOCKS blocks'
// keys (spread evenly over the keys left): fewer launches, each with more work items, so
// fewer merges per row and fewer last waves of workgroups that drain with the CU partly
// empty.  Row blocks with a slab that overflowed are scored again into the scratch, one block
// at a time.  At higher candidate densities a slab launch costs more than a block launch with
// its top-K (glm_chunk's second block, 8% of its scores above the threshold: 298 + 93 us
// against 243 + 108 us).  Without slabs (a consumer mask or block list, or exact scores) every
// launch takes one block.
struct KeySchedule {
  int32_t bk, nb, step, n;   // block keys, block launches, keys of each slab launch, launches
  int32_t start(int32_t l) const { return l < nb ? l * bk : nb * bk + (l - nb) * step; }
  int32_t keys(int32_t l) const { return l < nb ? bk : step; }
  bool slab(int32_t l) const { return l >= nb; }
};
constexpr int32_t SLAB_BLOCKS = 4;
constexpr int32_t SLAB_DENSITY = 20;
KeySchedule key_schedule(const idx_problem *p, int32_t Bk, int32_t Kc, bool slabs) {
  KeySchedule k{Bk, 1, Bk, 1};
  const int64_t L = p->L > 0 ? p->L : 0;
  if (L <= Bk) return k;
  int64_t nb = 1;
  if (!slabs) nb = (L + Bk - 1) / Bk;
  else
    while (nb * Bk < L && (int64_t)Kc * SLAB_DENSITY > nb * Bk) ++nb;
  k.nb = (int32_t)nb;
  k.n = k.nb;
  const int64_t rest = L - nb * Bk;
  if (rest <= 0) return k;
  const int64_t n2 = (rest + SLAB_BLOCKS * (int64_t)Bk - 1) / (SLAB_BLOCKS * (int64_t)Bk);
  k.step = (int32_t)(((rest + n2 - 1) / n2 + KEY_ALIGN - 1) / KEY_ALIGN * KEY_ALIGN);   // <= SLAB_BLOCKS B_k
  k.n = (int32_t)(nb + (rest + k.step - 1) / k.step);
  return k;
}
// Slabs per row of the widest slab launch.
int32_t schedule_slabs(const KeySchedule &k, int32_t L) {
  if (k.n <= k.nb) return 0;
  return std::max(block_slabs(std::min(k.step, L - k.start(k.nb))), block_slabs(L - k.start(k.n - 1)));
}
// Row gather: q [R, H, D] bytes, q_scale and w [R, H] floats, ks and ke [R].
size_t gather_ws(int32_t R, int32_t H, int32_t D) {
  return round_up_sz((size_t)R * H * D, 256) + 2 * round_up_sz((size_t)R * H * 4, 256) +
         2 * round_up_sz((size_t)R * 4, 256);
}
// Window flags of the scoring launches (idx::WindowFlags), a fixed region.
constexpr size_t FLAGS_WS = (size_t)idx::MAX_WINDOW_FLAGS * 4;
// The row chunks' first window keys (WindowFlags::kshift).
size_t shift_ws(const idx_problem *p, int32_t Tc) { return round_up_sz((size_t)((p->T + Tc - 1) / Tc + 1) * 4, 256); }
// The fused path's workspace: refinement, the score scratch (which also holds the slabs of the
// slab schedule, the widest the call can take), the slabs' bookkeeping, the window flags and
// the key shifts.
size_t fused_ws(const idx_problem *p, int32_t Tc, int32_t Bk, int32_t K) {
  const int32_t ns = schedule_slabs(key_schedule(p, Bk, cand_cap(K), true), p->L);
  return refine_ws(Tc, cand_cap(K)) + round_up_sz((size_t)Tc * scratch_pitch(Bk, ns) * 4, 256) + slab_ws(Tc, ns) +
         FLAGS_WS + shift_ws(p, Tc);
}
size_t cand_ws(int32_t Tc, int32_t pooled_cols, int32_t n_blocks, bool fused) {
  return refine_ws(Tc, cand_cap(n_blocks)) + round_up_sz((size_t)Tc * pitch(pooled_cols) * 4, 256) +
         round_up_sz((size_t)Tc * n_blocks * 4, 256) + (fused ? FLAGS_WS : 0);
}
// The flags of a call whose row chunks of Tc rows meet the key launches of `k` (nullptr in
// `flags` when there would be more than the region holds: the launches then stay by key split).
idx::WindowFlags window_flags(const idx_problem *p, int32_t Tc, const KeySchedule &k, uint32_t *region) {
  idx::WindowFlags f{};
  f.ks = p->ks;
  f.ke = p->ke;
  f.T = p->T;
  f.Tc = Tc;
  f.B0 = k.bk;
  f.nb = k.nb;
  f.LB = k.step;
  f.nlaunch = p->L > 0 ? k.n : 0;
  const int64_t n = (int64_t)((p->T + Tc - 1) / Tc) * f.nlaunch;
  f.flags = n > 0 && n <= idx::MAX_WINDOW_FLAGS ? region : nullptr;
  return f;
}
const uint32_t *launch_flag(const idx::WindowFlags &f, int32_t r0, int32_t kb) {
  const int32_t l = kb < f.nb * f.B0 ? kb / f.B0 : f.nb + (kb - f.nb * f.B0) / f.LB;
  return f.flags ? f.flags + (int64_t)(r0 / f.Tc) * f.nlaunch + l : nullptr;
}

struct RefineWs {
  uint32_t *overflow;
  float *kpart;
  int32_t *cidx;
  float *cval;
};
RefineWs carve_refine(Carve &cv, int32_t Tc, int32_t Kc) {
  RefineWs w;
  w.overflow = cv.take<uint32_t>(64);
  w.kpart = cv.take<float>(512);
  w.cidx = cv.take<int32_t>((size_t)Tc * Kc);
  w.cval = cv.take<float>((size_t)Tc * Kc);
  return w;
}

idx::RefineArgs refine_args(const idx_problem *p, const RefineWs &w, int32_t row0, int32_t nrows, int32_t Kc,
                            int32_t K, int32_t pool, int32_t *out_idx, float *out_val) {
  idx::RefineArgs r{};
  r.q = p->q;
  r.q_scale = p->q_scale;
  r.k = (const uint8_t *)p->k;
  r.k_scale = (const uint8_t *)p->k_scale;
  r.k_fmt = p->k_fmt;
  r.w = p->w;
  r.ks = p->ks;
  r.ke = p->ke;
  r.H = p->H;
  r.L = p->L;
  r.scale = p->scale;
  r.row0 = row0;
  r.nrows = nrows;
  r.cand_idx = w.cidx;
  r.cand_val = w.cval;
  r.ld_cand = Kc;
  r.Kc = Kc;
  r.K = K;
  r.pool = pool;
  r.kmax_part = w.kpart;
  r.npart = idx::key_bound_parts(p->L);
  r.overflow = w.overflow;
  r.out_idx = out_idx;
  r.out_val = out_val;
  return r;
}

}  // namespace

extern "C" {

const char *idx_status_str(idx_status s) {
  switch (s) {
    case IDX_OK: return "ok";
    case IDX_E_NULL: return "a required pointer is NULL";
    case IDX_E_SHAPE: return "inconsistent sizes";
    case IDX_E_PARAM: return "parameter out of range";
    case IDX_E_FORMAT: return "unknown key format";
    case IDX_E_WORKSPACE: return "workspace too small";
    case IDX_E_UNSUPPORTED: return "unsupported configuration";
    case IDX_E_LAUNCH: return "kernel launch failed";
    case IDX_E_ALIGN: return "pointer not aligned";
    case IDX_E_DEVICE_CHECK: return "a device-side precondition failed (IDX_DEBUG)";
    default: return "unknown status";
  }
}

idx_status idx_workspace_size(int32_t op, const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                              int32_t pool, int32_t n_blocks, int32_t W, size_t *bytes) {
  if (!bytes || !p) return IDX_E_NULL;
  *bytes = 0;
  if (p->T < 0 || p->L < 0) return IDX_E_SHAPE;
  const int32_t Tc = eff_chunk(p, row_chunk);
  switch (op) {
    case IDX_OP_MQA_LOGITS:
    case IDX_OP_TOPK: return IDX_OK;
    case IDX_OP_GATHER_ROWS:
      if (K < 0 || p->H <= 0 || p->D <= 0) return IDX_E_PARAM;
      *bytes = gather_ws(K, p->H, p->D);
      return IDX_OK;
    case IDX_OP_LOGITS_TOPK_FUSED: {
      if (K < 1 || K > MAX_K) return IDX_E_PARAM;
      const int32_t Bk = eff_block(p, block_k);
      if (check_block(Bk) != IDX_OK) return IDX_E_PARAM;
      *bytes = fused_ws(p, Tc, Bk, K);
      return IDX_OK;
    }
    case IDX_OP_BLOCK_CANDIDATES: {
      if (pool != 8) return IDX_E_UNSUPPORTED;
      if (n_blocks < 1 || n_blocks > MAX_K) return IDX_E_PARAM;
      const int32_t Bk = eff_block(p, block_k);
      if (check_block(Bk) != IDX_OK) return IDX_E_PARAM;
      *bytes = cand_ws(Tc, Bk / pool, n_blocks, true);
      return IDX_OK;
    }
    case IDX_OP_BLOCK_CANDIDATES_DENSE: {
      if (pool != 8) return IDX_E_UNSUPPORTED;
      if (n_blocks < 1 || n_blocks > MAX_K) return IDX_E_PARAM;
      if (W < 0 || W > MAX_W) return IDX_E_SHAPE;
      *bytes = cand_ws(Tc, (W + pool - 1) / pool, n_blocks, false);
      return IDX_OK;
    }
    default: return IDX_E_PARAM;
  }
}

idx_status idx_mqa_logits(const idx_problem *p, float *logits, int64_t ld, int32_t W, void *stream) {
  idx_status st = check_problem(p, true);
  if (st) return st;
  if (!logits) return IDX_E_NULL;
  if (W < 0 || ld < W || W > MAX_W) return IDX_E_SHAPE;
  if (!aligned(logits, 16)) return IDX_E_ALIGN;
  if (p->T == 0 || W == 0) return IDX_OK;
  if ((st = idx::debug_check(p->ks, p->ke, p->T, p->L, W, p, stream))) return st;
  hipStream_t s = (hipStream_t)stream;
  if (p->L > 0) {
    idx::LogitsArgs a = logits_args(p, 0, p->T, 0, p->L, logits, ld, W);
    st = launched(score(a, p, idx::STORE_DENSE, idx::exact_enabled(), s));
    if (st) return st;
  }
  return launched(idx::launch_fill_tail(logits, ld, W, p->ks, p->ke, 0, p->T, s));
}

idx_status idx_mqa_logits_block(const idx_problem *p, int32_t row0, int32_t nrows, int32_t key0, int32_t nkeys,
                                float *out, int64_t ld, void *stream) {
  idx_status st = check_problem(p, true);
  if (st) return st;
  if (!out) return IDX_E_NULL;
  if (row0 < 0 || nrows < 0 || (int64_t)row0 + nrows > p->T) return IDX_E_SHAPE;
  if (key0 < 0 || nkeys < 0 || key0 % KEY_ALIGN) return IDX_E_PARAM;
  if (ld < nkeys) return IDX_E_SHAPE;
  if (!aligned(out, 16)) return IDX_E_ALIGN;
  const int32_t key_hi = (int32_t)std::min<int64_t>((int64_t)key0 + nkeys, p->L);
  if (nrows == 0 || key_hi <= key0) return IDX_OK;
  if ((st = idx::debug_check(p->ks, p->ke, p->T, p->L, -1, p, stream))) return st;
  idx::LogitsArgs a = logits_args(p, row0, nrows, key0, key_hi, out, ld, nkeys);
  return launched(score(a, p, idx::STORE_BLOCK, idx::exact_enabled(), (hipStream_t)stream));
}

idx_status idx_topk(const float *logits, int64_t ld, int32_t W, const int32_t *ks, const int32_t *ke,
                    const uint8_t *mask, int64_t ld_mask, int32_t T, int32_t K, int32_t block_k, int32_t *out_idx,
                    float *out_val, void *ws, size_t ws_bytes, void *stream) {
  (void)ws;
  (void)ws_bytes;
  if (!logits || !ks || !ke || !out_idx) return IDX_E_NULL;
  if (T < 0 || W < 0 || ld < W) return IDX_E_SHAPE;
  if (mask && ld_mask < W) return IDX_E_SHAPE;
  if (K < 1 || K > MAX_KC) return IDX_E_PARAM;  // up to the refinement's candidate capacity
  if (block_k <= 0) block_k = MAX_BLOCK;
  if (block_k > MAX_BLOCK) return IDX_E_PARAM;
  if (!aligned(logits, 4) || !aligned(out_idx, 4) || (out_val && !aligned(out_val, 4))) return IDX_E_ALIGN;
  if (T == 0) return IDX_OK;
  idx_status st = idx::debug_check(ks, ke, T, INT32_MAX, W, nullptr, stream);
  if (st) return st;
  idx::TopkArgs a{};
  a.vals = logits;
  a.ld = ld;
  a.ncols = W;
  a.block = block_k;
  a.ks = ks;
  a.ke = ke;
  a.row0 = 0;
  a.nrows = T;
  a.mode = idx::TOPK_DENSE;
  a.key0 = 0;
  a.pool = 1;
  a.mask = mask;
  a.ld_mask = ld_mask;
  a.mask_w = ld_mask < W ? ld_mask : W;
  a.K = K;
  a.out_idx = out_idx;
  a.out_val = out_val;
  a.first = 1;
  return launched(idx::launch_topk(a, (hipStream_t)stream));
}

idx_status idx_logits_topk_fused(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                                 const uint8_t *mask, int64_t ld_mask, int32_t *out_idx, float *out_val, void *ws,
                                 size_t ws_bytes, void *stream) {
  return idx_logits_topk_fused_paged(p, K, block_k, row_chunk, mask, ld_mask, nullptr, out_idx, out_val, nullptr, ws,
                                     ws_bytes, stream);
}

}  // extern "C"

namespace idx {
// The fused indexer with its optional consumers: a byte mask or a block list restricting
// the selectable keys, and the index -> KV-slot transform of the final write.
idx_status fused_impl(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk, const uint8_t *mask,
                      int64_t ld_mask, const int32_t *blocks, int64_t ld_blocks, int32_t n_blocks, int32_t pool,
                      const int32_t *slot_of_key, int32_t *out_idx, float *out_val, int32_t *out_slot, void *ws,
                      size_t ws_bytes, void *stream, WorkspaceSource ws_source) {
  idx_status st = check_problem(p, true);
  if (st) return st;
  if (!out_idx) return IDX_E_NULL;
  if (!slot_of_key != !out_slot) return IDX_E_NULL;   // the transform needs both
  if (K < 1 || K > MAX_K) return IDX_E_PARAM;
  const int32_t Bk = eff_block(p, block_k);
  if ((st = check_block(Bk))) return st;
  if (row_chunk < 0) return IDX_E_PARAM;
  const int32_t Tc = eff_chunk(p, row_chunk);
  if (mask && ld_mask < 0) return IDX_E_SHAPE;
  if (!aligned(out_idx, 4) || (out_val && !aligned(out_val, 4)) || (out_slot && !aligned(out_slot, 4)) ||
      (slot_of_key && !aligned(slot_of_key, 4)))
    return IDX_E_ALIGN;
  int32_t bsh = 0;
  if (blocks) {
    if (mask) return IDX_E_PARAM;                        // one consumer at a time
    if (n_blocks < 0 || ld_blocks < n_blocks) return IDX_E_SHAPE;
    if (pool < 1 || (pool & (pool - 1))) return IDX_E_UNSUPPORTED;
    while ((1 << bsh) < pool) ++bsh;
    if (((Bk - 1) >> bsh) + 2 > idx::BMAP_BITS) return IDX_E_UNSUPPORTED;   // blocks of one launch
    if (!aligned(blocks, 4)) return IDX_E_ALIGN;
  }
  const size_t need = fused_ws(p, Tc, Bk, K);
  if (p->T == 0) return IDX_OK;
  if (ws_bytes < need) return IDX_E_WORKSPACE;
  // a workspace the library provides is looked up only once every host check has passed
  if (ws_source && ws_source(&ws) != hipSuccess) return IDX_E_LAUNCH;
  if (!ws) return IDX_E_NULL;
  if (!aligned(ws, 256)) return IDX_E_ALIGN;
  if ((st = debug_check(p->ks, p->ke, p->T, p->L, -1, p, stream))) return st;
  hipStream_t s = (hipStream_t)stream;
  const int32_t Kc = cand_cap(K);
  Carve cv{(uint8_t *)ws};
  RefineWs rw = carve_refine(cv, Tc, Kc);
  const int32_t nslab_max = schedule_slabs(key_schedule(p, Bk, cand_cap(K), true), p->L);
  const int32_t sld = scratch_pitch(Bk, nslab_max);
  float *scratch = cv.take<float>((size_t)Tc * sld);
  uint32_t *slab = (uint32_t *)scratch;                     // row r's slabs in its scratch row
  float *thr = cv.take<float>((size_t)Tc);
  uint32_t *ovf = cv.take<uint32_t>((size_t)Tc / 8 + 1);   // per scoring row block (>= 8 rows)
  uint32_t *ccnt = cv.take<uint32_t>((size_t)Tc * nslab_max * idx::CAND_PARTS);
  uint32_t *col_rows = cv.take<uint32_t>((size_t)Tc);
  // Slab launches after the first block launches, unless a consumer mask or block list
  // restricts the keys (the scoring kernel cannot drop the keys they exclude, which would
  // fill the slabs), or exact scores (IDX_EXACT) come from the fp64 kernel, which writes no
  // slabs: then every launch takes one block.
  const bool exact = exact_enabled();
  const KeySchedule ksch = key_schedule(p, Bk, Kc, !mask && !blocks && !exact);
  idx::WindowFlags wf = window_flags(p, Tc, ksch, cv.take<uint32_t>(idx::MAX_WINDOW_FLAGS));
  wf.kshift = cv.take<int32_t>(shift_ws(p, Tc) / 4);
  if ((st = launched(idx::launch_key_bound((const uint8_t *)p->k, (const uint8_t *)p->k_scale, p->k_fmt, p->L,
                                           rw.kpart, rw.overflow, &wf, s))))
    return st;
  for (int32_t r0 = 0; r0 < p->T; r0 += Tc) {
    const int32_t nr = std::min(Tc, p->T - r0);
    const int32_t *kshift = wf.kshift + r0 / Tc;
    for (int32_t l = 0; l < ksch.n; ++l) {
      const int32_t kb = ksch.start(l);
      const int32_t nk = std::max(0, std::min(ksch.keys(l), p->L - kb));
      idx::TopkArgs b{};
      b.thr_out = thr;
      b.vals = scratch;
      b.ld = sld;
      b.ncols = nk;
      b.block = Bk;
      b.ks = p->ks;
      b.ke = p->ke;
      b.row0 = r0;
      b.nrows = nr;
      b.mode = idx::TOPK_BLOCK;
      b.key0 = kb;
      b.pool = 1;
      b.mask = mask;
      b.ld_mask = ld_mask;
      b.mask_w = ld_mask;
      b.blocks = blocks;
      b.ld_blocks = ld_blocks;
      b.n_blocks = n_blocks;
      b.bpool_sh = bsh;
      b.K = Kc;
      b.out_idx = rw.cidx;
      b.out_val = rw.cval;
      b.first = l == 0;
      b.kshift = kshift;
      idx::LogitsArgs a = logits_args(p, r0, nr, kb, kb + nk, scratch, sld, nk);
      a.by_row = launch_flag(wf, r0, kb);
      a.kshift = kshift;
      b.launch_flag = a.by_row;
      if (ksch.slab(l) && nk > 0) {
        if (a.nsplit > nslab_max) return IDX_E_LAUNCH;   // (not reached: the schedule sized the slabs)
        // the launch writes the scores above each row's running threshold to its slabs; the
        // row blocks where a slab overflowed are scored again into the scratch, one block of
        // keys per pass, and the top-K reads those rows' columns there
        idx::LogitsArgs c = a;
        c.thr = thr;
        c.cand = slab;
        c.cand_ld = sld / 2;
        c.ccnt = ccnt;
        c.caps = CAPS;
        if ((st = launched(score(c, p, idx::STORE_SLAB, false, s)))) return st;
        const int32_t rpw = idx::logits_rows_per_workgroup(p->H);
        if ((st = launched(
                 idx::launch_slab_check(ccnt, a.nsplit * idx::CAND_PARTS, thr, nr, rpw, ovf, a.by_row, s))))
          return st;
        for (int32_t h0 = 0; h0 < nk; h0 += Bk) {
          const int32_t hn = std::min(Bk, nk - h0);
          idx::LogitsArgs f = logits_args(p, r0, nr, kb + h0, kb + h0 + hn, scratch, sld, hn);
          f.by_row = a.by_row;
          f.kshift = kshift;
          f.only_flagged = ovf;
          if ((st = launched(score(f, p, idx::STORE_BLOCK, false, s, true)))) return st;
          idx::TopkArgs bh = b;
          if (h0 == 0) {
            // slab merges of the rows outside flagged row blocks, which mark the rest in col_rows
            idx::TopkArgs bm = b;
            bm.cand = slab;
            bm.cand_ld = sld / 2;
            bm.ccnt = ccnt;
            bm.nslab = a.nsplit;
            bm.caps = CAPS;
            bm.slab_flags = ovf;
            bm.slab_rpw = rpw;
            bm.col_rows = col_rows;
            if ((st = launched(idx::launch_merge(bm, s)))) return st;
            bh.vcols = hn;   // then the first block's columns for the marked rows
          } else {           // the next block's columns, for the same rows
            bh.key0 = kb + h0;
            bh.ncols = hn;
          }
          bh.col_rows = col_rows;
          bh.only_rows = col_rows;
          if ((st = launched(idx::launch_topk(bh, s)))) return st;
        }
        continue;
      }
      if (nk > Bk) return IDX_E_UNSUPPORTED;   // the scratch holds one block (not reached: see key_schedule)
      if (nk > 0 && (st = launched(score(a, p, idx::STORE_BLOCK, exact, s)))) return st;
      if ((st = launched(idx::launch_topk(b, s)))) return st;
    }
    idx::RefineArgs r = refine_args(p, rw, r0, nr, Kc, K, 1, out_idx + (int64_t)r0 * K,
                                    out_val ? out_val + (int64_t)r0 * K : nullptr);
    r.slot_of_key = slot_of_key;
    r.out_slot = out_slot ? out_slot + (int64_t)r0 * K : nullptr;
    if ((st = launched(idx::launch_refine(r, s)))) return st;
  }
  return IDX_OK;
}
}  // namespace idx

extern "C" {

idx_status idx_logits_topk_fused_paged(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                                       const uint8_t *mask, int64_t ld_mask, const int32_t *slot_of_key,
                                       int32_t *out_idx, float *out_val, int32_t *out_slot, void *ws,
                                       size_t ws_bytes, void *stream) {
  return idx::fused_impl(p, K, block_k, row_chunk, mask, ld_mask, nullptr, 0, 0, 1, slot_of_key, out_idx, out_val,
                         out_slot, ws, ws_bytes, stream, nullptr);
}

idx_status idx_logits_topk_fused_blocks(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk,
                                        const int32_t *blocks, int64_t ld_blocks, int32_t n_blocks, int32_t pool,
                                        int32_t *out_idx, float *out_val, void *ws, size_t ws_bytes, void *stream) {
  if (!blocks) return IDX_E_NULL;
  return idx::fused_impl(p, K, block_k, row_chunk, nullptr, 0, blocks, ld_blocks, n_blocks, pool, nullptr, out_idx,
                         out_val, nullptr, ws, ws_bytes, stream, nullptr);
}

idx_status idx_refine_topk(const idx_problem *p, const int32_t *cand_idx, const float *cand_val, int64_t ld_cand,
                           int32_t Kc, int32_t K, int32_t pool, int32_t *out_idx, float *out_val, void *ws,
                           size_t ws_bytes, void *stream) {
  idx_status st = check_problem(p, true);
  if (st) return st;
  if (!cand_idx || !cand_val || !out_idx) return IDX_E_NULL;
  if (K < 1 || K > MAX_K || Kc < K || Kc > MAX_KC) return IDX_E_PARAM;
  if (pool != 1 && pool != 8) return IDX_E_UNSUPPORTED;
  if (ld_cand < Kc) return IDX_E_SHAPE;
  if (!aligned(cand_idx, 4) || !aligned(cand_val, 4) || !aligned(out_idx, 4) || (out_val && !aligned(out_val, 4)))
    return IDX_E_ALIGN;
  if (p->T == 0) return IDX_OK;
  if (!ws) return IDX_E_NULL;
  if (ws_bytes < HEAD) return IDX_E_WORKSPACE;
  if (!aligned(ws, 256)) return IDX_E_ALIGN;
  if ((st = idx::debug_check(p->ks, p->ke, p->T, p->L, -1, p, stream))) return st;
  hipStream_t s = (hipStream_t)stream;
  Carve cv{(uint8_t *)ws};
  RefineWs rw;
  rw.overflow = cv.take<uint32_t>(64);
  rw.kpart = cv.take<float>(512);
  rw.cidx = const_cast<int32_t *>(cand_idx);
  rw.cval = const_cast<float *>(cand_val);
  if ((st = launched(idx::launch_key_bound((const uint8_t *)p->k, (const uint8_t *)p->k_scale, p->k_fmt, p->L,
                                           rw.kpart, rw.overflow, nullptr, s))))
    return st;
  idx::RefineArgs r = refine_args(p, rw, 0, p->T, Kc, K, pool, out_idx, out_val);
  r.ld_cand = ld_cand;
  return launched(idx::launch_refine(r, s));
}

idx_status idx_block_candidates(const idx_problem *p, const float *logits, int64_t ld, int32_t pool,
                                int32_t n_blocks, int32_t block_k, int32_t row_chunk, uint8_t *mask, int64_t ld_mask,
                                int32_t W, int32_t *out_blocks, void *ws, size_t ws_bytes, void *stream) {
  idx_status st = check_problem(p, logits == nullptr);
  if (st) return st;
  if (!mask) return IDX_E_NULL;
  if (pool != 8) return IDX_E_UNSUPPORTED;
  if (n_blocks < 1 || n_blocks > MAX_K) return IDX_E_PARAM;
  if (W < 0 || W > MAX_W || ld_mask < W) return IDX_E_SHAPE;
  if (logits && ld < W) return IDX_E_SHAPE;
  if (row_chunk < 0) return IDX_E_PARAM;
  if (out_blocks && !aligned(out_blocks, 4)) return IDX_E_ALIGN;
  if (logits && !aligned(logits, 4)) return IDX_E_ALIGN;
  const int32_t Tc = eff_chunk(p, row_chunk);
  const int32_t Bk = eff_block(p, block_k);
  if (!logits && (st = check_block(Bk))) return st;
  const int32_t pooled_cols = logits ? (W + pool - 1) / pool : Bk / pool;
  const size_t need = cand_ws(Tc, pooled_cols, n_blocks, !logits);
  if (p->T == 0) return IDX_OK;
  if (!ws) return IDX_E_NULL;
  if (ws_bytes < need) return IDX_E_WORKSPACE;
  if (!aligned(ws, 256)) return IDX_E_ALIGN;
  if ((st = idx::debug_check(p->ks, p->ke, p->T, logits ? INT32_MAX : p->L, W, logits ? nullptr : p, stream)))
    return st;
  hipStream_t s = (hipStream_t)stream;
  const bool exact = idx::exact_enabled();
  Carve cv{(uint8_t *)ws};
  const int32_t Kc = logits ? n_blocks : cand_cap(n_blocks);
  RefineWs rw = carve_refine(cv, Tc, cand_cap(n_blocks));
  const int32_t pld = pitch(pooled_cols);
  float *pooled = cv.take<float>((size_t)Tc * pld);
  int32_t *kept = cv.take<int32_t>((size_t)Tc * n_blocks);
  idx::WindowFlags wf{};
  if (!logits) {
    wf = window_flags(p, Tc, key_schedule(p, Bk, 0, false), cv.take<uint32_t>(idx::MAX_WINDOW_FLAGS));
    if ((st = launched(idx::launch_key_bound((const uint8_t *)p->k, (const uint8_t *)p->k_scale, p->k_fmt, p->L,
                                             rw.kpart, rw.overflow, &wf, s))))
      return st;
  }
  for (int32_t r0 = 0; r0 < p->T; r0 += Tc) {
    const int32_t nr = std::min(Tc, p->T - r0);
    int32_t *blocks = out_blocks ? out_blocks + (int64_t)r0 * n_blocks : kept;
    idx::TopkArgs b{};
    b.ks = p->ks;
    b.ke = p->ke;
    b.row0 = r0;
    b.nrows = nr;
    b.pool = pool;
    b.mask = nullptr;
    b.K = Kc;
    if (logits) {
      // selection is exact on the given logits
      b.out_idx = blocks;
      b.out_val = rw.cval;
      if ((st = launched(idx::launch_pool_dense(logits + (int64_t)r0 * ld, ld, W, p->ks, p->ke, r0, nr, pool, pooled,
                                                pld, pooled_cols, s))))
        return st;
      b.vals = pooled;
      b.ld = pld;
      b.ncols = pooled_cols;
      b.block = MAX_BLOCK;
      b.mode = idx::TOPK_POOL_DENSE;
      b.key0 = 0;
      b.first = 1;
      if ((st = launched(idx::launch_topk(b, s)))) return st;
    } else {
      b.out_idx = rw.cidx;
      b.out_val = rw.cval;
      int32_t kb = 0;
      do {
        const int32_t nk = std::min(Bk, p->L - kb);
        if (nk > 0) {
          idx::LogitsArgs a = logits_args(p, r0, nr, kb, kb + nk, pooled, pld, (nk + pool - 1) / pool);
          a.by_row = launch_flag(wf, r0, kb);
          b.launch_flag = a.by_row;
          if ((st = launched(score(a, p, idx::STORE_POOL8, exact, s)))) return st;
        }
        b.vals = pooled;
        b.ld = pld;
        b.ncols = nk > 0 ? (nk + pool - 1) / pool : 0;
        b.block = MAX_BLOCK;
        b.mode = idx::TOPK_POOL_BLOCK;
        b.key0 = kb;
        b.first = kb == 0;
        if ((st = launched(idx::launch_topk(b, s)))) return st;
        kb += Bk;
      } while (kb < p->L);
      // exact boundary: blocks scored by the max of their keys' exact scores
      idx::RefineArgs r = refine_args(p, rw, r0, nr, Kc, n_blocks, pool, blocks, nullptr);
      if ((st = launched(idx::launch_refine(r, s)))) return st;
    }
    if ((st = launched(idx::launch_expand_mask(blocks, n_blocks, p->ks, p->ke, r0, nr, pool, W, mask, ld_mask, s))))
      return st;
  }
  return IDX_OK;
}

idx_status idx_ragged_windows(const int32_t *cu_q, const int32_t *cu_k, int32_t B, int32_t T, int32_t *ks,
                              int32_t *ke, void *stream) {
  return idx_ragged_windows_ratio(cu_q, cu_k, cu_k, 1, B, T, ks, ke, stream);
}

idx_status idx_gather_rows(const idx_problem *p, const int32_t *rows, int32_t R, idx_problem *out, void *ws,
                           size_t ws_bytes, void *stream) {
  idx_status st = check_problem(p, true);
  if (st) return st;
  if (!out || (R > 0 && (!rows || !ws))) return IDX_E_NULL;
  if (R < 0) return IDX_E_SHAPE;
  if (R > 0 && ws_bytes < gather_ws(R, p->H, p->D)) return IDX_E_WORKSPACE;
  if ((rows && !aligned(rows, 4)) || (ws && !aligned(ws, 256))) return IDX_E_ALIGN;
  Carve cv{(uint8_t *)ws};
  uint8_t *oq = cv.take<uint8_t>((size_t)R * p->H * p->D);
  float *oqs = cv.take<float>((size_t)R * p->H);
  float *ow = cv.take<float>((size_t)R * p->H);
  int32_t *oks = cv.take<int32_t>((size_t)R);
  int32_t *oke = cv.take<int32_t>((size_t)R);
  *out = *p;
  out->T = R;
  out->q = oq;
  out->q_scale = oqs;
  out->w = ow;
  out->ks = oks;
  out->ke = oke;
  return launched(idx::launch_gather_rows(rows, R, p->T, p->q, p->q_scale, p->w, p->ks, p->ke, p->H, p->D, oq, oqs, ow,
                                          oks, oke, (hipStream_t)stream));
}

idx_status idx_tail_rows(const int32_t *cu_q, int32_t B, int32_t n, int32_t *rows, void *stream) {
  if (!cu_q || !rows) return IDX_E_NULL;
  if (B < 0 || n < 0) return IDX_E_SHAPE;
  if (!aligned(cu_q, 4) || !aligned(rows, 4)) return IDX_E_ALIGN;
  return launched(idx::launch_tail_rows(cu_q, B, n, rows, (hipStream_t)stream));
}

idx_status idx_ragged_windows_ratio(const int32_t *cu_q, const int32_t *cu_k, const int32_t *cu_c, int32_t ratio,
                                    int32_t B, int32_t T, int32_t *ks, int32_t *ke, void *stream) {
  if (!cu_q || !cu_k || !cu_c || !ks || !ke) return IDX_E_NULL;
  if (B < 0 || T < 0) return IDX_E_SHAPE;
  if (ratio < 1) return IDX_E_PARAM;
  if (!aligned(cu_q, 4) || !aligned(cu_k, 4) || !aligned(cu_c, 4) || !aligned(ks, 4) || !aligned(ke, 4))
    return IDX_E_ALIGN;
  return launched(idx::launch_ragged(cu_q, cu_k, cu_c, ratio, B, T, ks, ke, (hipStream_t)stream));
}

}  // extern "C"
