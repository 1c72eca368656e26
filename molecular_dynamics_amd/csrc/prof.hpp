// Optional per-kernel timing with hipEvents recorded on the launching stream.
#pragma once
#include <hip/hip_runtime.h>

namespace mdmp {
bool prof_on();
void prof_begin(const char* name, hipStream_t st);
void prof_end(hipStream_t st);

// While one of these lives on a thread, that thread's launches record no events (a call
// that must not create runtime objects, such as the allocation-free evaluation).
struct ProfOff {
  ProfOff();
  ~ProfOff();
};

struct ProfScope {
  hipStream_t st;
  bool on;
  ProfScope(const char* name, hipStream_t s) : st(s), on(prof_on()) {
    if (on) prof_begin(name, st);
  }
  ~ProfScope() {
    if (on) prof_end(st);
  }
};
}  // namespace mdmp
