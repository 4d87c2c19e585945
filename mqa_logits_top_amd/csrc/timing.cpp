// Launch timing (idx_launch_timing): two HIP events around each scoring launch while a
// record is on.  The events are created once per record device; recording takes a lock.
#include <atomic>
#include <cmath>
#include <mutex>

#include "api_internal.h"

namespace idx {
namespace {

struct Record {
  std::mutex mu;
  std::atomic<bool> on{false};
  int dev = -1;                          // device whose events exist (-1: none yet)
  hipEvent_t ev[2 * IDX_TIMING_MAX] = {};
  idx_launch_time entry[IDX_TIMING_MAX];
  bool closed[IDX_TIMING_MAX];           // both events recorded
  int n = 0;
  int gen = 0;                           // bumped whenever the record is cleared
};

Record &record() {
  static Record r;
  return r;
}

}  // namespace

// A slot token: the entry index and (modulo 2^16) the record generation it belongs to, so that
// a launch whose record was cleared meanwhile on another thread writes nothing.
int timing_begin(hipStream_t s) {
  Record &r = record();
  if (!r.on.load(std::memory_order_acquire)) return -1;
  int dev = -1;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipGetDevice(&dev) != hipSuccess || hipStreamIsCapturing(s, &cs) != hipSuccess ||
      cs != hipStreamCaptureStatusNone)
    return -1;
  std::lock_guard<std::mutex> g(r.mu);
  if (!r.on.load(std::memory_order_relaxed) || dev != r.dev || r.n >= IDX_TIMING_MAX) return -1;
  const int i = r.n;
  if (hipEventRecord(r.ev[2 * i], s) != hipSuccess) return -1;
  r.closed[i] = false;
  r.entry[i] = idx_launch_time{-1.f, 0, 0, 0, 0, 0, 0};
  ++r.n;
  return i + IDX_TIMING_MAX * (r.gen & 0xFFFF);
}

void timing_end(int token, hipStream_t s, bool ok, int mode, int flagged, int row0, int nrows, int key0, int nkeys) {
  if (token < 0) return;
  Record &r = record();
  std::lock_guard<std::mutex> g(r.mu);
  const int slot = token % IDX_TIMING_MAX;
  if (token / IDX_TIMING_MAX != (r.gen & 0xFFFF) || slot >= r.n) return;   // the record was cleared meanwhile
  r.entry[slot] = idx_launch_time{-1.f, mode, flagged, row0, nrows, key0, nkeys};
  r.closed[slot] = ok && hipEventRecord(r.ev[2 * slot + 1], s) == hipSuccess;
}

}  // namespace idx

extern "C" {

idx_status idx_launch_timing(int32_t enable) {
  idx::Record &r = idx::record();
  std::lock_guard<std::mutex> g(r.mu);
  if (!enable) {
    r.on.store(false, std::memory_order_release);
    return IDX_OK;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return IDX_E_LAUNCH;
  if (dev != r.dev) {
    // events of another device: recreate them for this one
    if (r.dev >= 0)
      for (hipEvent_t &e : r.ev) {
        if (e) (void)hipEventDestroy(e);
        e = nullptr;
      }
    r.dev = -1;
    for (hipEvent_t &e : r.ev)
      if (hipEventCreate(&e) != hipSuccess) {
        for (hipEvent_t &f : r.ev) {
          if (f) (void)hipEventDestroy(f);
          f = nullptr;
        }
        return IDX_E_LAUNCH;
      }
    r.dev = dev;
  }
  r.n = 0;
  ++r.gen;
  r.on.store(true, std::memory_order_release);
  return IDX_OK;
}

idx_status idx_launch_timing_read(idx_launch_time *out, int32_t cap, int32_t *n) {
  if (!n || (cap > 0 && !out)) return IDX_E_NULL;
  if (cap < 0) return IDX_E_PARAM;
  idx::Record &r = idx::record();
  std::lock_guard<std::mutex> g(r.mu);
  *n = r.n;
  for (int i = 0; i < r.n && i < cap; ++i) {
    idx_launch_time e = r.entry[i];
    float ms = -1.f;
    if (r.closed[i] && hipEventSynchronize(r.ev[2 * i + 1]) == hipSuccess &&
        hipEventElapsedTime(&ms, r.ev[2 * i], r.ev[2 * i + 1]) != hipSuccess)
      ms = -1.f;
    e.ms = r.closed[i] && std::isfinite(ms) ? ms : -1.f;
    out[i] = e;
  }
  r.n = 0;
  ++r.gen;
  return IDX_OK;
}

}  // extern "C"
