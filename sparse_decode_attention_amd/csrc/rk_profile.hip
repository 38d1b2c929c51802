// rk_profile.hip -- optional per-kernel timing with HIP events (measurement
// support).  While enabled, every RK_LAUNCH records an event before and after
// its kernel on the launch stream; rk_profile_end() resolves and aggregates
// them per kernel name.  Events are pooled and reused across sessions.
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/rocketkv.h"
#include "rk_internal.hpp"

namespace rk {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;
hipError_t g_err = hipSuccess;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
  if (err != hipSuccess && g_err == hipSuccess) g_err = err;
  return err == hipSuccess ? e : nullptr;
}

}  // namespace

bool prof_enabled() { return g_on.load(std::memory_order_relaxed); }

void prof_before(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  Record r{name, take_event(), take_event()};
  if (r.start) {
    const hipError_t err = hipEventRecord(r.start, s);
    if (err != hipSuccess && g_err == hipSuccess) g_err = err;
  }
  g_records.push_back(r);
}

void prof_after(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_records.empty()) return;
  Record& r = g_records.back();
  if (r.stop) {
    const hipError_t err = hipEventRecord(r.stop, s);
    if (err != hipSuccess && g_err == hipSuccess) g_err = err;
  }
}

}  // namespace rk

extern "C" rk_status rk_profile_begin(void) {
  std::lock_guard<std::mutex> lk(rk::g_mu);
  for (auto& r : rk::g_records) {
    if (r.start) rk::g_pool.push_back(r.start);
    if (r.stop) rk::g_pool.push_back(r.stop);
  }
  rk::g_records.clear();
  rk::g_err = hipSuccess;
  rk::g_on.store(true);
  return RK_OK;
}

extern "C" rk_status rk_profile_end(rk_kernel_time* out, int32_t cap, int32_t* n_out) {
  rk::g_on.store(false);
  if (!out || !n_out || cap < 0) return RK_EINVAL;
  std::lock_guard<std::mutex> lk(rk::g_mu);
  int32_t n = 0;
  hipError_t err = rk::g_err;
  for (auto& r : rk::g_records) {
    float ms = 0.f;
    if (r.start && r.stop) {
      hipError_t e = hipEventSynchronize(r.stop);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
      if (e != hipSuccess && err == hipSuccess) err = e;
    }
    int32_t i = 0;
    while (i < n && strcmp(out[i].name, r.name) != 0) ++i;
    if (i == n) {
      if (n == cap) continue;
      memset(&out[n], 0, sizeof(out[n]));
      strncpy(out[n].name, r.name, sizeof(out[n].name) - 1);
      ++n;
    }
    out[i].launches += 1;
    out[i].total_ms += double(ms);
  }
  for (auto& r : rk::g_records) {
    if (r.start) rk::g_pool.push_back(r.start);
    if (r.stop) rk::g_pool.push_back(r.stop);
  }
  rk::g_records.clear();
  *n_out = n;
  return err == hipSuccess ? RK_OK : RK_EDEVICE;
}
