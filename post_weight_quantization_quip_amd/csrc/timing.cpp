// Per-kernel launch timing with HIP events, off by default. While on, every
// launch made through timed_launch gets an event pair that its dispatch
// stamps with the kernel's start and end; a report waits for the pairs and
// sums their durations per name.
#include <atomic>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace quip {
namespace {

struct Pending {
  std::string name;
  hipEvent_t a = nullptr, b = nullptr;
  double flops = 0.0, bytes = 0.0;
};

struct Total {
  long long launches = 0;
  double ms = 0.0, flops = 0.0, bytes = 0.0;
};

struct Registry {
  std::mutex mu;
  std::vector<Pending> pending;     // recorded, not yet read
  std::vector<hipEvent_t> pool;     // events free for reuse
  std::map<std::string, Total> totals;
};

Registry& reg() {
  static Registry r;
  return r;
}

std::atomic<bool> g_on{false};

hipEvent_t take_event(Registry& r) {
  if (!r.pool.empty()) {
    hipEvent_t e = r.pool.back();
    r.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Waits for every recorded pair and adds it to the totals (lock held).
quip_status drain(Registry& r) {
  quip_status st = QUIP_OK;
  for (Pending& p : r.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
      st = fail(QUIP_ERR_HIP, "quip_timing: event wait failed for " + p.name);
    } else {
      Total& t = r.totals[p.name];
      t.launches += 1;
      t.ms += ms;
      t.flops += p.flops;
      t.bytes += p.bytes;
    }
    r.pool.push_back(p.a);
    r.pool.push_back(p.b);
  }
  r.pending.clear();
  return st;
}

}  // namespace

bool timing_on() { return g_on.load(std::memory_order_relaxed); }

bool timing_begin(const char* name, double flops, double bytes, hipEvent_t* start,
                  hipEvent_t* stop) {
  Registry& r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  Pending p;
  p.name = name;
  p.flops = flops;
  p.bytes = bytes;
  p.a = take_event(r);
  p.b = take_event(r);
  if (!p.a || !p.b) {
    if (p.a) r.pool.push_back(p.a);
    if (p.b) r.pool.push_back(p.b);
    return false;
  }
  r.pending.push_back(p);
  *start = p.a;
  *stop = p.b;
  return true;
}

void timing_enable(bool on) { g_on.store(on); }

quip_status timing_reset() {
  Registry& r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  quip_status st = drain(r);
  r.totals.clear();
  return st;
}

quip_status timing_report(std::string& out) {
  Registry& r = reg();
  std::lock_guard<std::mutex> lk(r.mu);
  quip_status st = drain(r);
  out.clear();
  char line[320];
  for (const auto& kv : r.totals) {
    std::snprintf(line, sizeof(line), "%s %lld %.6f %.6e %.6e\n", kv.first.c_str(),
                  kv.second.launches, kv.second.ms, kv.second.flops, kv.second.bytes);
    out += line;
  }
  return st;
}

}  // namespace quip
