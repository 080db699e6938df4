// Opt-in per-kernel timing: when enabled, each kernel launch of the library
// is bracketed by two hipEvents recorded on the launch stream, so a caller
// can read the device time of every kernel without a profiler.  Events come
// from a pool created when timing is enabled; launches beyond the pool's
// capacity between two reads are not recorded (and counted as dropped).
#include <vector>

#include "jfa.h"
#include "jfa_timing.hpp"

namespace jfa {

namespace {

struct Pending {
  int kernel;
  int ev;  // index of the start event; end event is ev + 1
};

struct Timer {
  bool on = false;
  std::vector<hipEvent_t> events;  // 2 per slot
  std::vector<int> free_slots;
  std::vector<Pending> pending;
  int64_t launches[K_COUNT] = {};
  double total_ms[K_COUNT] = {};
  int64_t dropped = 0;
};

Timer g_timer;

const char* const kNames[K_COUNT] = {"sched_sort_scan", "sched_expand", "sched_dump", "fwd_kernel",
                                     "delta_kernel",    "dkdv_kernel",  "dq_reduce",  "dq_kernel",
                                     "delta_exact_kernel", "group_sum_kernel", "fwd_mx_kernel",
                                     "delta_mx_kernel", "dkdv_mx_kernel", "dq_mx_kernel"};

void release_all() {
  for (hipEvent_t e : g_timer.events) (void)hipEventDestroy(e);
  g_timer.events.clear();
  g_timer.free_slots.clear();
  g_timer.pending.clear();
}

int drain() {
  int rc = JFA_OK;
  for (const Pending& p : g_timer.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timer.events[p.ev + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.events[p.ev], g_timer.events[p.ev + 1]) != hipSuccess) {
      rc = JFA_ERR_HIP;
    } else {
      g_timer.launches[p.kernel] += 1;
      g_timer.total_ms[p.kernel] += ms;
    }
    g_timer.free_slots.push_back(p.ev);
  }
  g_timer.pending.clear();
  return rc;
}

}  // namespace

int timing_begin(hipStream_t stream, int kernel) {
  if (!g_timer.on) return -1;
  if (g_timer.free_slots.empty()) {
    ++g_timer.dropped;
    return -1;
  }
  const int ev = g_timer.free_slots.back();
  g_timer.free_slots.pop_back();
  if (hipEventRecord(g_timer.events[ev], stream) != hipSuccess) {
    g_timer.free_slots.push_back(ev);
    return -1;
  }
  g_timer.pending.push_back(Pending{kernel, ev});
  return ev;
}

void timing_end(hipStream_t stream, int token) {
  if (token < 0) return;
  (void)hipEventRecord(g_timer.events[token + 1], stream);
}

}  // namespace jfa

using namespace jfa;

extern "C" {

int jfa_timing_enable(int capacity) {
  if (capacity < 0) return JFA_ERR_INVALID_ARG;
  drain();
  release_all();
  g_timer.on = capacity > 0;
  for (int i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      release_all();
      g_timer.on = false;
      return JFA_ERR_HIP;
    }
    g_timer.events.push_back(e);
  }
  for (int i = 2 * capacity - 2; i >= 0; i -= 2) g_timer.free_slots.push_back(i);
  return JFA_OK;
}

int jfa_timing_reset(void) {
  const int rc = drain();
  for (int k = 0; k < K_COUNT; ++k) {
    g_timer.launches[k] = 0;
    g_timer.total_ms[k] = 0.0;
  }
  g_timer.dropped = 0;
  return rc;
}

int jfa_timing_read(int kernel, int64_t* launches, double* total_ms) {
  if (kernel < 0 || kernel >= K_COUNT || !launches || !total_ms) return JFA_ERR_INVALID_ARG;
  const int rc = drain();
  *launches = g_timer.launches[kernel];
  *total_ms = g_timer.total_ms[kernel];
  return rc;
}

const char* jfa_kernel_name(int kernel) {
  if (kernel < 0 || kernel >= K_COUNT) return nullptr;
  return kNames[kernel];
}

}  // extern "C"
