// Library-internal interface of the opt-in per-kernel event timer.
#pragma once
#include <hip/hip_runtime.h>

namespace jfa {

enum KernelId {
  K_SCHED_SORT = 0,
  K_SCHED_EXPAND,
  K_SCHED_DUMP,
  K_FWD,
  K_DELTA,
  K_DKDV,
  K_DQ_REDUCE,
  K_DQ,
  K_DELTA_EXACT,
  K_GROUP_SUM,
  K_FWD_MX,
  K_DELTA_MX,
  K_DKDV_MX,
  K_DQ_MX,
  K_COUNT
};

// Records a start event for `kernel` on `stream` when timing is enabled;
// returns a token for timing_end (negative when nothing was recorded).
int timing_begin(hipStream_t stream, int kernel);
void timing_end(hipStream_t stream, int token);

// Launch `...` bracketed by timing events.
#define JFA_TIMED_LAUNCH(kernel_id, stream, ...)              \
  do {                                                         \
    const int jfa_tok_ = ::jfa::timing_begin(stream, kernel_id); \
    hipLaunchKernelGGL(__VA_ARGS__);                           \
    ::jfa::timing_end(stream, jfa_tok_);                       \
  } while (0)

}  // namespace jfa
