// Opt-in kernel timing: HIP event pairs recorded around the library's compute-kernel
// launches on the caller's stream, summed per kernel id when read back.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "ridgefill.h"
#include "rf_profile.h"

namespace rf {

namespace {
struct Pair {
  int id;
  hipEvent_t start, stop;
};
std::mutex g_mu;
bool g_enabled = false;
std::vector<Pair> g_pending;
std::vector<hipEvent_t> g_pool;
double g_total_ms[RF_KERNEL_COUNT] = {};
int64_t g_launches[RF_KERNEL_COUNT] = {};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Folds every recorded pair into the totals; caller holds the lock.
hipError_t drain() {
  hipError_t err = hipSuccess;
  for (Pair& p : g_pending) {
    hipError_t e = hipEventSynchronize(p.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e == hipSuccess) {
      g_total_ms[p.id] += ms;
      g_launches[p.id] += 1;
    } else {
      err = e;
    }
    g_pool.push_back(p.start);
    g_pool.push_back(p.stop);
  }
  g_pending.clear();
  return err;
}
}  // namespace

ProfileScope::ProfileScope(int id, hipStream_t s) : id_(id), stream_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled) return;
  start_ = take_event();
  stop_ = take_event();
  if (!start_ || !stop_ || hipEventRecord(start_, stream_) != hipSuccess) {
    if (start_) g_pool.push_back(start_);
    if (stop_) g_pool.push_back(stop_);
    start_ = stop_ = nullptr;
  }
}

ProfileScope::~ProfileScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(stop_, stream_) == hipSuccess) {
    g_pending.push_back({id_, start_, stop_});
  } else {
    g_pool.push_back(start_);
    g_pool.push_back(stop_);
  }
}

}  // namespace rf

extern "C" {

rf_status ridgefill_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(rf::g_mu);
  rf::g_enabled = enable != 0;
  return RF_OK;
}

rf_status ridgefill_profile_read(int32_t kernel, int64_t* launches, double* total_ms) {
  if (kernel < 0 || kernel >= RF_KERNEL_COUNT || !launches || !total_ms) return RF_E_INVALID;
  std::lock_guard<std::mutex> lk(rf::g_mu);
  if (rf::drain() != hipSuccess) return RF_E_HIP;
  *launches = rf::g_launches[kernel];
  *total_ms = rf::g_total_ms[kernel];
  return RF_OK;
}

rf_status ridgefill_profile_reset(void) {
  std::lock_guard<std::mutex> lk(rf::g_mu);
  hipError_t e = rf::drain();
  for (int i = 0; i < RF_KERNEL_COUNT; ++i) {
    rf::g_total_ms[i] = 0.0;
    rf::g_launches[i] = 0;
  }
  return e == hipSuccess ? RF_OK : RF_E_HIP;
}

}  // extern "C"
