// skv_timing.hip -- optional per-kernel timing: while recording is on, every
// main launch of the library is bracketed by a pair of HIP events recorded on
// the launch's own stream, so the elapsed time of one kernel can be read
// without a profiler and without synchronising between calls.
#include <mutex>
#include <vector>

#include "skv_internal.hpp"

namespace skv {
namespace {

std::mutex g_mu;
bool g_on = false;
int g_cap = 0;
int g_n = 0;
int g_open = -1;
std::vector<hipEvent_t> g_ev;  // 2 per record: begin, end
std::vector<int32_t> g_id;

void release_events() {
  for (hipEvent_t e : g_ev)
    if (e) (void)hipEventDestroy(e);
  g_ev.clear();
  g_id.clear();
}

}  // namespace

void timing_mark(int kernel, bool end, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  if (!end) {
    g_open = -1;
    if (g_n >= g_cap) return;  // full: later launches go unrecorded
    if (hipEventRecord(g_ev[2 * g_n], st) != hipSuccess) return;
    g_id[g_n] = kernel;
    g_open = g_n;
  } else {
    if (g_open < 0) return;
    if (hipEventRecord(g_ev[2 * g_open + 1], st) == hipSuccess) g_n = g_open + 1;
    g_open = -1;
  }
}

}  // namespace skv

using namespace skv;

extern "C" int skv_timing_start(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return SKV_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_on) return SKV_ERR_ARG;
  g_ev.assign(2 * (size_t)capacity, nullptr);
  g_id.assign((size_t)capacity, -1);
  for (auto &e : g_ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      release_events();
      return SKV_ERR_HIP;
    }
  }
  g_cap = capacity;
  g_n = 0;
  g_open = -1;
  g_on = true;
  return SKV_OK;
}

extern "C" int skv_timing_stop(int32_t *kernel, float *ms, int32_t capacity, int32_t *count) {
  if (capacity < 0 || (capacity > 0 && (!kernel || !ms)) || !count) return SKV_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return SKV_ERR_ARG;
  g_on = false;
  int rc = SKV_OK;
  for (int i = 0; i < g_n; ++i) {
    float t = 0.f;
    if (hipEventSynchronize(g_ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&t, g_ev[2 * i], g_ev[2 * i + 1]) != hipSuccess)
      rc = SKV_ERR_HIP;
    if (i < capacity) {
      kernel[i] = g_id[i];
      ms[i] = t;
    }
  }
  *count = g_n;
  release_events();
  g_cap = g_n = 0;
  g_open = -1;
  return rc;
}

extern "C" const char *skv_timed_kernel_name(int32_t kernel) {
  switch (kernel) {
    case kTimeModel: return "model";
    case kTimeEncode: return "k_encode";
    case kTimeDecode: return "k_decode";
    default: return "unknown";
  }
}
