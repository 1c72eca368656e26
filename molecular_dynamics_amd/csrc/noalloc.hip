// mp_energy_forces_noalloc: energy + forces with the workspace in a file-scope device
// array, for callers that cannot allocate device memory.
#include <mutex>
#include <string>

#include "model.hpp"
#include "prof.hpp"

namespace mdmp {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // MP_NOALLOC_SCRATCH_BYTES in mdmp.h
static_assert(kScratchBytes == MP_NOALLOC_SCRATCH_BYTES, "scratch size shared with the header");

// The workspace of the call.  In host code this name is only a stand-in: its device
// address, one per GPU, comes from hipGetSymbolAddress and is used everywhere instead.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// the current device's address of `scratch`, looked up once per device
int scratch_ptr(void** out) {
  int dev = -1;
  MP_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return arg_error("mp_energy_forces_noalloc: device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    MP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return arg_error("mp_energy_forces_noalloc: no device address for the scratch array");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MP_OK;
}

__global__ void k_copy_flag(const int32_t* __restrict__ src, int32_t* __restrict__ dst) { *dst = *src; }

}  // namespace
}  // namespace mdmp

using namespace mdmp;

extern "C" int mp_energy_forces_noalloc(const mp_model* m, const mp_graph* g, const int32_t* perm, double* energy,
                                        float* forces, float* atom_energy, int32_t* nonfinite, hipStream_t st) {
  if (!m || !g) return arg_error("mp_energy_forces_noalloc: null model or graph");
  size_t need = 0;
  MP_TRY(mp_energy_forces_ws(m, g->n, g->n_edges, &need));
  if (need > kScratchBytes)
    return arg_error("mp_energy_forces_noalloc: this graph needs " + std::to_string(need) +
                     " bytes of workspace; the allocation-free call has " + std::to_string(kScratchBytes) +
                     " (use mp_energy_forces with a workspace)");
  void* ws = nullptr;
  MP_TRY(scratch_ptr(&ws));
  ProfOff no_events;  // per-kernel timing would create hipEvents
  MP_TRY(ef_enqueue(m, g, g->n_edges, perm, energy, forces, atom_energy, ws, kScratchBytes, nullptr, st));
  if (nonfinite) {
    // the evaluation's non-finite flag sits at the start of its workspace
    k_copy_flag<<<1, 1, 0, st>>>((const int32_t*)ws, nonfinite);
    MP_CHECK_LAUNCH();
  }
  return MP_OK;
}
