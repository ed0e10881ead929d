// A second stream per device for work that may overlap the caller's stream
// (the bulk of a trailing update while the critical path of the pass goes on),
// ordered through events. Non-blocking, default priority; created on first
// use and kept until the process ends. Launches on it should be bounded
// (GemmArgs::max_wgs) so that the caller's stream keeps room on every CU.
#include <mutex>
#include <utility>

#include "common.h"

namespace quip {
namespace {

struct Side {
  hipStream_t s = nullptr;
  hipEvent_t fwd = nullptr, back = nullptr;
  std::mutex use;  // held by the caller that enqueues on this side stream
};

constexpr int kMaxDevices = 64;
Side g_side[kMaxDevices];
std::mutex g_mu;  // creation

}  // namespace

quip_status side_stream(SideStream* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(QUIP_ERR_HIP, "side stream: no current device");
  Side& sd = g_side[dev];
  std::unique_lock<std::mutex> use(sd.use);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!sd.s) {
      hipStream_t st = nullptr;
      hipEvent_t a = nullptr, b = nullptr;
      if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess)
        return fail(QUIP_ERR_HIP, "side stream: hipStreamCreateWithFlags failed");
      if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess)
        return fail(QUIP_ERR_HIP, "side stream: hipEventCreateWithFlags failed");
      sd.s = st;
      sd.fwd = a;
      sd.back = b;
    }
  }
  out->s = sd.s;
  out->fwd = sd.fwd;
  out->back = sd.back;
  out->lock = std::move(use);
  return QUIP_OK;
}

quip_status stream_after(hipStream_t waiter, hipStream_t signaler, hipEvent_t ev) {
  if (hipEventRecord(ev, signaler) != hipSuccess)
    return fail(QUIP_ERR_HIP, "hipEventRecord failed");
  if (hipStreamWaitEvent(waiter, ev, 0) != hipSuccess)
    return fail(QUIP_ERR_HIP, "hipStreamWaitEvent failed");
  return QUIP_OK;
}

}  // namespace quip
