// Launch timing for diagnostics: while a kernel's bit is set in the active
// mask, every eager launch of it is made with hipExtLaunchKernelGGL and a pair
// of HIP events that take the kernel's own start and end times on the stream
// it is launched on.  Launches under graph capture are not timed.
#include <vector>

#include "../../include/csahca.h"
#include "common.h"
#include "kernels.h"

namespace {

struct KernelTimes {
  std::vector<hipEvent_t> ev;   // 2 per launch: before, after
  int64_t n = 0;                // launches recorded
};

uint32_t g_mask = 0;
int64_t g_cap = 0;
KernelTimes g_times[CA_TIMED_KERNELS];

bool capturing(hipStream_t st) {
  hipStreamCaptureStatus s = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &s) != hipSuccess || s != hipStreamCaptureStatusNone;
}

void release() {
  for (auto& t : g_times) {
    for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
    t.ev.clear();
    t.n = 0;
  }
  g_mask = 0;
  g_cap = 0;
}

}  // namespace

namespace ca {

bool timer_events(int kernel, hipStream_t st, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!(g_mask >> kernel & 1u)) return false;
  KernelTimes& t = g_times[kernel];
  if (t.n >= g_cap || capturing(st)) return false;
  *start = t.ev[2 * t.n];
  *stop = t.ev[2 * t.n + 1];
  ++t.n;
  return true;
}

}  // namespace ca

extern "C" {

int ca_timer_start(uint32_t kernel_mask, int64_t max_launches) {
  release();
  if (kernel_mask >= (1u << CA_TIMED_KERNELS) || max_launches <= 0 || max_launches > (1 << 20))
    return CA_ERR_ARG;
  for (int k = 0; k < CA_TIMED_KERNELS; ++k) {
    if (!(kernel_mask >> k & 1u)) continue;
    g_times[k].ev.resize(2 * max_launches);
    for (auto& e : g_times[k].ev)
      if (hipEventCreate(&e) != hipSuccess) {
        e = nullptr;
        release();
        return CA_ERR_HIP;
      }
  }
  g_cap = max_launches;
  g_mask = kernel_mask;
  return CA_OK;
}

int ca_timer_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= CA_TIMED_KERNELS || total_ms == nullptr || launches == nullptr) return CA_ERR_ARG;
  const KernelTimes& t = g_times[kernel];
  double sum = 0.0;
  if (t.n > 0 && hipEventSynchronize(t.ev[2 * t.n - 1]) != hipSuccess) return CA_ERR_HIP;
  for (int64_t i = 0; i < t.n; ++i) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) return CA_ERR_HIP;
    sum += ms;
  }
  *total_ms = sum;
  *launches = t.n;
  return CA_OK;
}

int ca_timer_stop(void) {
  for (const auto& t : g_times)
    if (t.n > 0) (void)hipEventSynchronize(t.ev[2 * t.n - 1]);
  release();
  return CA_OK;
}

}  // extern "C"
