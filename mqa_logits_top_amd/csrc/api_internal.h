// Declarations shared by the C ABI's source files (not part of the public interface).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/idx.h"

namespace idx {

// Supplies a workspace the library owns, once every host check of a call has passed.
typedef hipError_t (*WorkspaceSource)(void **ws);

// The fused indexer (idx_logits_topk_fused and its variants): optional byte mask or block
// list consumer, optional index -> slot transform.  ws_source (nullable) replaces `ws` by the
// workspace it returns; ws_bytes is then that workspace's size.
idx_status fused_impl(const idx_problem *p, int32_t K, int32_t block_k, int32_t row_chunk, const uint8_t *mask,
                      int64_t ld_mask, const int32_t *blocks, int64_t ld_blocks, int32_t n_blocks, int32_t pool,
                      const int32_t *slot_of_key, int32_t *out_idx, float *out_val, int32_t *out_slot, void *ws,
                      size_t ws_bytes, void *stream, WorkspaceSource ws_source);

// IDX_DEBUG set (and not "0") in the environment, read on every call.
bool debug_enabled();
// IDX_EXACT set (and not "0") in the environment, read on every call: scores are computed
// exactly (fp64 over the codes) instead of on the fp8 MFMA, and no candidate slabs are used.
bool exact_enabled();
// In debug mode: check on the device that 0 <= ks[t] <= ke[t] <= L and ke[t] - ks[t] <= W (W >= 0)
// for t < T, and, with a problem p, that its q_scale are >= 0, its w finite and its key scales
// valid; synchronises `stream` and returns IDX_E_DEVICE_CHECK on a failure.  IDX_OK otherwise,
// and always when debug mode is off (nothing is enqueued then).
idx_status debug_check(const int32_t *ks, const int32_t *ke, int32_t T, int32_t L, int64_t W, const idx_problem *p,
                       void *stream);

// Launch timing (idx_launch_timing): timing_begin records a launch's first event on s when a
// record is on, and returns a token for its slot (-1: not recorded); timing_end records the
// second event (ok: the launch was enqueued) and the launch's description.
int timing_begin(hipStream_t s);
void timing_end(int token, hipStream_t s, bool ok, int mode, int flagged, int row0, int nrows, int key0, int nkeys);

}  // namespace idx
