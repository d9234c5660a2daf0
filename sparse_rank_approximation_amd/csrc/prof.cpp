// prof.cpp -- optional per-kernel timing (diagnostics, declared in elsaa.h).
// With profiling on, every kernel launch of the library is bracketed by two HIP
// events recorded on the launch stream; the report waits for them and sums the
// elapsed times per kernel name.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "elsaa.h"
#include "launch.hpp"

namespace elsaa {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;

void clear_locked() {
  for (Rec& r : g_recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
}

}  // namespace

// This thread's launches are not recorded while suspended; the record a
// prof_begin opened on this thread (-1: none) is the one its prof_end closes.
thread_local bool t_suspended = false;
thread_local long t_open = -1;

void prof_suspend(bool on) { t_suspended = on; }

void prof_begin(hipStream_t st, const char* name) {
  t_open = -1;
  if (t_suspended) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  Rec r{name, nullptr, nullptr};
  if (hipEventCreate(&r.a) != hipSuccess) return;
  if (hipEventCreate(&r.b) != hipSuccess) {
    (void)hipEventDestroy(r.a);
    return;
  }
  (void)hipEventRecord(r.a, st);
  g_recs.push_back(r);
  t_open = (long)g_recs.size() - 1;
}

void prof_end(hipStream_t st) {
  if (t_open < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_on && t_open < (long)g_recs.size()) (void)hipEventRecord(g_recs[t_open].b, st);
  t_open = -1;
}

}  // namespace elsaa

extern "C" {

elsaa_status elsaa_profile(int32_t enable) {
  std::lock_guard<std::mutex> lk(elsaa::g_mu);
  if (enable) elsaa::clear_locked();
  elsaa::g_on = enable != 0;
  return ELSAA_OK;
}

elsaa_status elsaa_profile_report(char* buf, size_t len, size_t* needed) {
  std::lock_guard<std::mutex> lk(elsaa::g_mu);
  struct Agg { long n = 0; double ms = 0.0; };
  std::map<std::string, Agg> agg;
  for (elsaa::Rec& r : elsaa::g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return ELSAA_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return ELSAA_ERR_HIP;
    Agg& g = agg[r.name];
    g.n += 1;
    g.ms += ms;
  }
  std::string out;
  char line[256];
  for (auto& kv : agg) {
    snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.n, kv.second.ms);
    out += line;
  }
  if (needed) *needed = out.size() + 1;
  if (buf && len > 0) {
    const size_t n = out.size() < len - 1 ? out.size() : len - 1;
    memcpy(buf, out.data(), n);
    buf[n] = '\0';
  }
  return ELSAA_OK;
}

}  // extern "C"
