// timing.hpp -- opt-in per-kernel HIP-event timing (diagnostics only).
//
// Off by default.  Between grpo_timing_begin() and grpo_timing_end() every
// launch made by this thread's library calls is bracketed by a pair of HIP
// events recorded on the launch's own stream; grpo_timing_end() waits for the
// last event and reports the summed elapsed time and launch count per kernel.
#pragma once

#include <hip/hip_runtime.h>

namespace grpo {

enum KernelKind {
  KK_ADVANTAGES = 0,
  KK_LSE_PARTIALS,
  KK_LSE_MERGE,
  KK_LOSS_FINAL,
  KK_ACTIVE_SCAN,
  KK_TRANSPOSE,
  KK_BWD_PREP,
  KK_DZ,
  KK_DH_GEMM,
  KK_DW_GEMM,
  KK_DH_SCATTER,
  KK_ZERO,
  KK_GEMM_NT,
  KK_SEQ_COUNTS,
  KK_FP8_QUANT,
  KK_FP8_DEQUANT,
  KK_COUNT
};

const char* kernel_kind_name(int k);

// Records a start event on construction and a stop event on destruction
// when timing is enabled on this thread.
class ScopedKernelTimer {
 public:
  ScopedKernelTimer(int kind, hipStream_t s);
  ~ScopedKernelTimer();

 private:
  int kind_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr;
};

bool timing_begin();
// Fills up to `max` entries; returns the number of kernel kinds with launches.
int timing_end(const char** names, int* launches, double* total_ms, int max);

}  // namespace grpo
