// Per-kernel-class launch timing with HIP events recorded on the launch stream.
#include <mutex>
#include <utility>
#include <vector>

#include "api_internal.h"

namespace {

struct TimingState {
  std::mutex mu;
  uint32_t mask = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[MTFM_K_COUNT];
  std::vector<hipEvent_t> pool;
};

TimingState& state() {
  static TimingState s;
  return s;
}

hipEvent_t take_event(TimingState& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

thread_local int g_timing_off = 0;

}  // namespace

TimingOff::TimingOff() { ++g_timing_off; }
TimingOff::~TimingOff() { --g_timing_off; }

TimedLaunch::TimedLaunch(int kclass, hipStream_t s) : cls_(kclass), stream_(s) {
  TimingState& st = state();
  if (g_timing_off || !(st.mask & (1u << kclass))) return;
  std::lock_guard<std::mutex> lk(st.mu);
  start_ = take_event(st);
  stop_ = take_event(st);
  if (start_ && stop_) (void)hipEventRecord(start_, s);
}

TimedLaunch::~TimedLaunch() {
  if (!start_ || !stop_) return;
  TimingState& st = state();
  (void)hipEventRecord(stop_, stream_);
  std::lock_guard<std::mutex> lk(st.mu);
  st.pending[cls_].push_back({start_, stop_});
}

extern "C" mtfm_status mtfm_timing_enable(uint32_t class_mask) {
  TimingState& st = state();
  std::lock_guard<std::mutex> lk(st.mu);
  st.mask = class_mask & ((1u << MTFM_K_COUNT) - 1);
  return MTFM_OK;
}

extern "C" mtfm_status mtfm_timing_read(int32_t kernel_class, int64_t* launches, double* total_ms) {
  if (!launches || !total_ms) return MTFM_E_NULL;
  if (kernel_class < 0 || kernel_class >= MTFM_K_COUNT) return MTFM_E_DIMS;
  TimingState& st = state();
  std::vector<std::pair<hipEvent_t, hipEvent_t>> items;
  {
    std::lock_guard<std::mutex> lk(st.mu);
    items.swap(st.pending[kernel_class]);
  }
  double sum = 0.0;
  mtfm_status status = MTFM_OK;
  for (auto& pr : items) {
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess && status == MTFM_OK) status = hip_fail(e, "mtfm_timing_read");
    sum += ms;
  }
  {
    std::lock_guard<std::mutex> lk(st.mu);
    for (auto& pr : items) {
      st.pool.push_back(pr.first);
      st.pool.push_back(pr.second);
    }
  }
  *launches = (int64_t)items.size();
  *total_ms = sum;
  return status;
}
