// timing.hip -- opt-in per-kernel HIP-event timing (diagnostics only).
#include "timing.hpp"

#include <vector>

namespace grpo {
namespace {

struct Record {
  int kind;
  hipEvent_t start, stop;
};

struct State {
  bool on = false;
  std::vector<Record> recs;
};

thread_local State g_state;

const char* const kNames[KK_COUNT] = {
    "advantages", "lse_partials", "lse_merge", "loss_final", "active_scan", "transpose",
    "bwd_prep",   "dz",           "dh_gemm",   "dw_gemm",    "dh_scatter",  "zero",
    "gemm_nt",    "seq_counts", "fp8_quantize", "fp8_dequantize"};

}  // namespace

const char* kernel_kind_name(int k) { return (k >= 0 && k < KK_COUNT) ? kNames[k] : "?"; }

ScopedKernelTimer::ScopedKernelTimer(int kind, hipStream_t s) : kind_(kind), s_(s) {
  if (!g_state.on) return;
  if (hipEventCreate(&start_) != hipSuccess) {
    start_ = nullptr;
    return;
  }
  if (hipEventRecord(start_, s_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    start_ = nullptr;
  }
}

ScopedKernelTimer::~ScopedKernelTimer() {
  if (start_ == nullptr) return;
  hipEvent_t stop = nullptr;
  if (hipEventCreate(&stop) != hipSuccess) {
    (void)hipEventDestroy(start_);
    return;
  }
  if (hipEventRecord(stop, s_) != hipSuccess) {   // an unrecorded pair is dropped
    (void)hipEventDestroy(start_);
    (void)hipEventDestroy(stop);
    return;
  }
  g_state.recs.push_back({kind_, start_, stop});
}

bool timing_begin() {
  for (auto& r : g_state.recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_state.recs.clear();
  g_state.on = true;
  return true;
}

int timing_end(const char** names, int* launches, double* total_ms, int max) {
  g_state.on = false;
  int cnt[KK_COUNT] = {0};
  double ms[KK_COUNT] = {0.0};
  for (auto& r : g_state.recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess &&
        hipEventElapsedTime(&t, r.start, r.stop) == hipSuccess) {
      ms[r.kind] += t;
      cnt[r.kind] += 1;
    }
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_state.recs.clear();
  int n = 0;
  for (int k = 0; k < KK_COUNT; ++k) {
    if (cnt[k] == 0) continue;
    if (n < max) {
      names[n] = kNames[k];
      launches[n] = cnt[k];
      total_ms[n] = ms[k];
    }
    ++n;
  }
  return n;
}

}  // namespace grpo
