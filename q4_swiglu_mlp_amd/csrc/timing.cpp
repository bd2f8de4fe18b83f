// Optional kernel timing: HIP event pairs recorded around the main kernels of
// each call, for benchmarks and profiles.  Off unless zinc_timing_enable()
// was called; then every launcher brackets its main kernel(s) with
// timing_begin()/timing_end() on the call's stream.
#include "../../include/zinc_mlp.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "launch.hpp"

namespace {

struct Timing {
  std::mutex mu;
  bool enabled = false;
  int count = 0;
  std::vector<hipEvent_t> start, stop;
};

Timing& timing() {
  static Timing t;
  return t;
}

void destroy_events(Timing& t) {
  for (hipEvent_t e : t.start) (void)hipEventDestroy(e);
  for (hipEvent_t e : t.stop) (void)hipEventDestroy(e);
  t.start.clear();
  t.stop.clear();
}

}  // namespace

namespace zinc {

void timing_begin(hipStream_t stream) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  if (t.enabled && t.count < (int)t.start.size()) (void)hipEventRecord(t.start[t.count], stream);
}

void timing_end(hipStream_t stream) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  if (t.enabled && t.count < (int)t.start.size()) {
    (void)hipEventRecord(t.stop[t.count], stream);
    ++t.count;
  }
}

}  // namespace zinc

extern "C" {

int zinc_timing_enable(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return ZINC_ERR_ARG;
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  destroy_events(t);
  t.start.resize(capacity);
  t.stop.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    // timing only: no system-scope fence on record (a fence would write back
    // and invalidate the caches between the timed kernel and its neighbours,
    // adding its own cost to the call being measured)
    if (hipEventCreateWithFlags(&t.start[i], hipEventDisableSystemFence) != hipSuccess ||
        hipEventCreateWithFlags(&t.stop[i], hipEventDisableSystemFence) != hipSuccess) {
      t.start.resize(i);
      t.stop.resize(i);
      destroy_events(t);
      return ZINC_ERR_HIP;
    }
  }
  t.count = 0;
  t.enabled = true;
  return ZINC_OK;
}

int zinc_timing_collect(float* ms, int32_t capacity, int32_t* n_out) {
  if (!ms || !n_out) return ZINC_ERR_NULL;
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  const int n = t.count < capacity ? t.count : capacity;
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(t.stop[i]) != hipSuccess) return ZINC_ERR_HIP;
    if (hipEventElapsedTime(&ms[i], t.start[i], t.stop[i]) != hipSuccess) return ZINC_ERR_HIP;
  }
  *n_out = n;
  t.count = 0;
  return ZINC_OK;
}

void zinc_timing_disable(void) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.enabled = false;
  t.count = 0;
  destroy_events(t);
}

}  // extern "C"
