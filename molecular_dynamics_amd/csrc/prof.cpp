// Per-kernel hipEvent timing (mp_profile_*).  Off by default; never active
// while a stream is being captured into a graph.
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "prof.hpp"

namespace mdmp {
namespace {
struct Rec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
std::vector<size_t> g_open;
thread_local int t_off = 0;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  hipEventCreate(&e);
  return e;
}

bool capturing(hipStream_t st) {
  hipStreamCaptureStatus s = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &s) != hipSuccess) return false;
  return s != hipStreamCaptureStatusNone;
}
}  // namespace

bool prof_on() { return g_on && t_off == 0; }

ProfOff::ProfOff() { ++t_off; }
ProfOff::~ProfOff() { --t_off; }

void prof_begin(const char* name, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || capturing(st)) {
    g_open.push_back((size_t)-1);
    return;
  }
  Rec r{name, take_event(), take_event()};
  hipEventRecord(r.a, st);
  g_recs.push_back(r);
  g_open.push_back(g_recs.size() - 1);
}

void prof_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_open.empty()) return;
  size_t i = g_open.back();
  g_open.pop_back();
  if (i != (size_t)-1) hipEventRecord(g_recs[i].b, st);
}
}  // namespace mdmp

using namespace mdmp;

extern "C" int mp_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return MP_OK;
}

extern "C" int mp_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_recs) {
    hipEventSynchronize(r.b);
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return MP_OK;
}

extern "C" int mp_profile_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) return arg_error("mp_profile_read: null argument");
  std::lock_guard<std::mutex> lk(g_mu);
  double t = 0;
  int64_t n = 0;
  for (auto& r : g_recs) {
    if (r.name != name) continue;
    MP_HIP(hipEventSynchronize(r.b));
    float ms = 0.f;
    MP_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    t += ms;
    n++;
  }
  *total_ms = t;
  *launches = n;
  return MP_OK;
}
