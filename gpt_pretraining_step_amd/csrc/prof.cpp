// Launch recording: per-launch HIP events kept while gpt_prof_start is on.
// C ABI declared in include/gpt_step.h (section "launch recording").
#include <cxxabi.h>
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "gpt_step.h"
#include "launch.h"

namespace gk {

volatile int g_prof_on = 0;

namespace {

struct Rec {
  const void* kernel;
  hipStream_t stream;
  Work work;
};

struct Recorder {
  std::mutex mu;
  std::vector<hipEvent_t> ev;  // 2 per record slot
  std::vector<Rec> recs;
  int capacity = 0;
  bool overflow = false;
};

Recorder& rec() {
  static Recorder r;
  return r;
}

void free_events(Recorder& r) {
  for (hipEvent_t e : r.ev) hipEventDestroy(e);
  r.ev.clear();
  r.recs.clear();
  r.capacity = 0;
  r.overflow = false;
}

}  // namespace

bool prof_slot(hipStream_t s, const void* kernel, Work w, hipEvent_t* start, hipEvent_t* stop) {
  Recorder& r = rec();
  std::lock_guard<std::mutex> lk(r.mu);
  if ((int)r.recs.size() >= r.capacity) {
    r.overflow = true;
    return false;
  }
  const size_t i = r.recs.size();
  *start = r.ev[2 * i];
  *stop = r.ev[2 * i + 1];
  r.recs.push_back(Rec{kernel, s, w});
  return true;
}

}  // namespace gk

extern "C" {

int gpt_prof_start(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return GPT_ERR_INVALID_ARG;
  gk::Recorder& r = gk::rec();
  std::lock_guard<std::mutex> lk(r.mu);
  gk::free_events(r);
  r.ev.resize(2 * (size_t)capacity, nullptr);
  for (auto& e : r.ev)
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      for (hipEvent_t x : r.ev)
        if (x) hipEventDestroy(x);
      r.ev.clear();
      return GPT_ERR_HIP;
    }
  r.capacity = capacity;
  r.recs.reserve(capacity);
  gk::g_prof_on = 1;
  return GPT_OK;
}

int gpt_prof_stop(void) {
  gk::g_prof_on = 0;
  gk::Recorder& r = gk::rec();
  std::lock_guard<std::mutex> lk(r.mu);
  return r.overflow ? 1 : 0;
}

int32_t gpt_prof_count(void) {
  gk::Recorder& r = gk::rec();
  std::lock_guard<std::mutex> lk(r.mu);
  return (int32_t)r.recs.size();
}

int gpt_prof_record(int32_t i, char* name, size_t name_len, float* ms, double* flops,
                    double* bytes) {
  gk::Recorder& r = gk::rec();
  std::lock_guard<std::mutex> lk(r.mu);
  if (i < 0 || i >= (int32_t)r.recs.size() || !name || name_len < 2 || !ms || !flops || !bytes)
    return GPT_ERR_INVALID_ARG;
  if (gk::g_prof_on) return GPT_ERR_INVALID_ARG;  // still recording
  const gk::Rec& x = r.recs[i];
  hipEvent_t a = r.ev[2 * i], b = r.ev[2 * i + 1];
  if (hipEventSynchronize(b) != hipSuccess) return GPT_ERR_HIP;
  float t = 0.f;
  if (hipEventElapsedTime(&t, a, b) != hipSuccess) return GPT_ERR_HIP;
  *ms = t;
  *flops = x.work.flops;
  *bytes = x.work.bytes;
  const char* raw = hipKernelNameRefByPtr(x.kernel, x.stream);
  std::string nm = raw ? raw : "?";
  int dst = 0;
  char* dem = abi::__cxa_demangle(nm.c_str(), nullptr, nullptr, &dst);
  if (dem && dst == 0) nm = dem;
  free(dem);
  snprintf(name, name_len, "%s", nm.c_str());
  return GPT_OK;
}

void gpt_prof_clear(void) {
  gk::g_prof_on = 0;
  gk::Recorder& r = gk::rec();
  std::lock_guard<std::mutex> lk(r.mu);
  gk::free_events(r);
}

}  // extern "C"
