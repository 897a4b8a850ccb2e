// Kernel timing: HIP events attached to each library launch while timing is on.
//
// The two events of a launch travel with its dispatch (hipExtLaunchKernel), so
// they record when the kernel itself starts and ends on its stream -- the
// interval a kernel-trace profiler reports -- without marker packets of their
// own between kernels.  Single-threaded use, like the rest of the library.
#include <utility>
#include <vector>

#include "pa_common.h"

namespace {

struct Record {
  int kind;
  hipEvent_t start, stop;
};

struct Timing {
  bool active = false;
  int used = 0;
  std::vector<Record> recs;
  std::vector<std::pair<int, double>> last;  // (kind, ms) of the last pa_timing_end
};

Timing& state() {
  static Timing t;
  return t;
}

}  // namespace

namespace pa {

TimedLaunch timing_events(int kind) {
  Timing& t = state();
  if (!t.active || t.used >= static_cast<int>(t.recs.size())) return TimedLaunch{nullptr, nullptr};
  Record& r = t.recs[t.used++];
  r.kind = kind;
  return TimedLaunch{r.start, r.stop};
}

}  // namespace pa

extern "C" {

pa_status pa_timing_begin(int32_t capacity) {
  if (capacity < 0) return PA_ERR_INVALID_ARG;
  Timing& t = state();
  while (static_cast<int>(t.recs.size()) < capacity) {
    Record r{-1, nullptr, nullptr};
    if (hipEventCreate(&r.start) != hipSuccess) return PA_ERR_DEVICE;
    if (hipEventCreate(&r.stop) != hipSuccess) {
      (void)hipEventDestroy(r.start);
      return PA_ERR_DEVICE;
    }
    t.recs.push_back(r);
  }
  t.used = 0;
  t.active = true;
  return PA_OK;
}

pa_status pa_timing_end(double* ms_out, int32_t* launches_out) {
  Timing& t = state();
  if (!ms_out || !launches_out) return PA_ERR_INVALID_ARG;
  for (int k = 0; k < PA_NUM_KERNEL_KINDS; ++k) {
    ms_out[k] = 0.0;
    launches_out[k] = 0;
  }
  pa_status st = PA_OK;
  t.last.clear();
  for (int i = 0; i < t.used; ++i) {
    Record& r = t.recs[i];
    if (r.kind < 0 || r.kind >= PA_NUM_KERNEL_KINDS) continue;
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = PA_ERR_DEVICE;
      continue;
    }
    ms_out[r.kind] += ms;
    launches_out[r.kind] += 1;
    t.last.emplace_back(r.kind, static_cast<double>(ms));
  }
  t.active = false;
  t.used = 0;
  return st;
}

pa_status pa_timing_launches(int32_t kind, double* ms_out, int32_t capacity,
                             int32_t* count_out) {
  if (kind < 0 || kind >= PA_NUM_KERNEL_KINDS || capacity < 0 || !count_out ||
      (capacity > 0 && !ms_out))
    return PA_ERR_INVALID_ARG;
  int32_t n = 0;
  for (const auto& e : state().last) {
    if (e.first != kind) continue;
    if (n < capacity) ms_out[n] = e.second;
    ++n;
  }
  *count_out = n;
  return PA_OK;
}

}  // extern "C"
