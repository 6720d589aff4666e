// Optional per-kernel timing with HIP events (a profiling aid, off by default).
// While enabled, each bracketed kernel launch records one event before and one after the
// kernel on the launch's own stream; hla_timing_read() waits for the recorded events and
// sums their elapsed times per kernel kind.
#include "timing.hpp"

#include <mutex>
#include <vector>

namespace hla {
namespace {

struct Record {
  int32_t which;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Record> g_records;

void clear_locked() {
  for (auto& r : g_records) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_records.clear();
}

}  // namespace

TimedLaunch::TimedLaunch(int32_t which, hipStream_t s) : which_(which), stream_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  if (hipEventCreate(&start_) != hipSuccess) return;
  if (hipEventCreate(&stop_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    return;
  }
  if (hipEventRecord(start_, stream_) != hipSuccess) {
    (void)hipEventDestroy(start_);
    (void)hipEventDestroy(stop_);
    return;
  }
  active_ = true;
}

TimedLaunch::~TimedLaunch() {
  if (!active_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(stop_, stream_) != hipSuccess || !g_on) {
    (void)hipEventDestroy(start_);
    (void)hipEventDestroy(stop_);
    return;
  }
  g_records.push_back({which_, start_, stop_});
}

}  // namespace hla

extern "C" {

hla_status_t hla_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(hla::g_mu);
  hla::clear_locked();
  hla::g_on = on != 0;
  return HLA_OK;
}

hla_status_t hla_timing_read(int32_t which, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return HLA_ERR_NULL_ARG;
  if (which < 0 || which >= HLA_KERNEL_COUNT) return HLA_ERR_BAD_SHAPE;
  std::lock_guard<std::mutex> lk(hla::g_mu);
  double sum = 0.0;
  int64_t n = 0;
  for (auto& r : hla::g_records) {
    if (r.which != which) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return HLA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return HLA_ERR_HIP;
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return HLA_OK;
}

}  // extern "C"
